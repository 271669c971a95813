// Streaming fused phase 3, the cases with the most live registers: feature
// width 256, and with the decayed recurrence also 128-row tiles at feature
// width 128.  Built with the matrix-core accumulators in their own registers
// (the form with them in ordinary VGPRs fails to compile at this pressure).
#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_wide_bf16(const FwdParams& p, int DK, int C, bool decay, int64_t grid, hipStream_t s) {
    if (decay) {
        switch (DK * 1000 + C) {
            case 128128: return pipe::by_flags<128, 128, DECAY_DIRECT>(p, grid, s);
            case 256032: return pipe::by_flags<256, 32, DECAY_DIRECT>(p, grid, s);
            case 256064: return pipe::by_flags<256, 64, DECAY_DIRECT>(p, grid, s);
        }
        return hipErrorInvalidValue;
    }
    switch (DK * 1000 + C) {
        case 256032: return pipe::by_flags<256, 32, DECAY_NONE>(p, grid, s);
        case 256064: return pipe::by_flags<256, 64, DECAY_NONE>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
