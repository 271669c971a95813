// Streaming fused phase 3 with the decayed recurrence (instantiations of the
// direct form), the cases whose registers leave room for matrix-core
// accumulators in VGPRs; the others are in la_pipe_wide.hip.  The factored form
// (la_pipe_decay_fac.hip) runs wherever it has an instantiation and gamma keeps
// its weights in range.
#include <cmath>

#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_decay_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s) {
    if (!pipe_args_ok(p, DK, DVT)) return hipErrorInvalidValue;
    const int TT = C > 64 ? C : 64;
    hipError_t e;
    if ((float)TT * std::fabs(p.log2_gamma) <= kFacMaxLog2Range && fwd_pipe_decay_fac_bf16(p, DK, C, grid, s, &e))
        return e;
    switch (DK * 1000 + C) {
        case 128032: return pipe::by_flags<128, 32, DECAY_DIRECT>(p, grid, s);
        case 128064: return pipe::by_flags<128, 64, DECAY_DIRECT>(p, grid, s);
        case 64032: return pipe::by_flags<64, 32, DECAY_DIRECT>(p, grid, s);
        case 64064: return pipe::by_flags<64, 64, DECAY_DIRECT>(p, grid, s);
        case 64128: return pipe::by_flags<64, 128, DECAY_DIRECT>(p, grid, s);
        case 128128:
        case 256032:
        case 256064: return fwd_pipe_wide_bf16(p, DK, C, true, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
