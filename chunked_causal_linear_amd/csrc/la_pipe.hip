// Streaming fused phase 3 for chunks of 32, 64 or 128 rows (instantiations;
// feature width 256 with chunks of 32 or 64).  The decayed recurrence is
// instantiated in la_pipe_decay.hip.
#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s) {
    if (p.log2_gamma != 0.0f) return fwd_pipe_decay_bf16(p, DK, DVT, C, grid, s);
    return pipe_dispatch<false>(p, DK, DVT, C, grid, s);
}

}  // namespace la
