// Streaming fused phase 3 for chunks of 32, 64 or 128 rows at feature width
// 64 and 128 (instantiations).  Feature width 256 is in la_pipe_wide.hip, the
// decayed recurrence in la_pipe_decay.hip.
#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s) {
    if (p.log2_gamma != 0.0f) return fwd_pipe_decay_bf16(p, DK, DVT, C, grid, s);
    if (!pipe_args_ok(p, DK, DVT)) return hipErrorInvalidValue;
    switch (DK * 1000 + C) {
        case 128032: return pipe::by_flags<128, 32, DECAY_NONE>(p, grid, s);
        case 128064: return pipe::by_flags<128, 64, DECAY_NONE>(p, grid, s);
        case 128128: return pipe::by_flags<128, 128, DECAY_NONE>(p, grid, s);
        case 64032: return pipe::by_flags<64, 32, DECAY_NONE>(p, grid, s);
        case 64064: return pipe::by_flags<64, 64, DECAY_NONE>(p, grid, s);
        case 64128: return pipe::by_flags<64, 128, DECAY_NONE>(p, grid, s);
        case 256032:
        case 256064: return fwd_pipe_wide_bf16(p, DK, C, false, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
