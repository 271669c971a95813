// Streaming fused phase 3 with the decayed recurrence (instantiations), the
// cases whose registers leave room for matrix-core accumulators in VGPRs; the
// others are in la_pipe_wide.hip.
#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_decay_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s) {
    if (!pipe_args_ok(p, DK, DVT)) return hipErrorInvalidValue;
    switch (DK * 1000 + C) {
        case 128032: return pipe::by_flags<128, 32, true>(p, grid, s);
        case 128064: return pipe::by_flags<128, 64, true>(p, grid, s);
        case 64032: return pipe::by_flags<64, 32, true>(p, grid, s);
        case 64064: return pipe::by_flags<64, 64, true>(p, grid, s);
        case 64128: return pipe::by_flags<64, 128, true>(p, grid, s);
        case 128128:
        case 256032:
        case 256064: return fwd_pipe_wide_bf16(p, DK, C, true, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
