// Streaming fused phase 3 with the decayed recurrence (instantiations).
#include "la_pipe.hpp"

namespace la {

hipError_t fwd_pipe_decay_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s) {
    return pipe_dispatch<true>(p, DK, DVT, C, grid, s);
}

}  // namespace la
