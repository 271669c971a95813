// Streaming fused phase 3 with the decayed recurrence: the cases with the most
// live registers (128-row tiles at feature width 128, feature width 256),
// built with the matrix-core accumulators in their own registers.
#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_decay_wide_bf16(const FwdParams& p, int DK, int C, int64_t grid, hipStream_t s) {
    switch (DK * 1000 + C) {
        case 128128: return pipe::by_flags<128, 128, true>(p, grid, s);
        case 256032: return pipe::by_flags<256, 32, true>(p, grid, s);
        case 256064: return pipe::by_flags<256, 64, true>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
