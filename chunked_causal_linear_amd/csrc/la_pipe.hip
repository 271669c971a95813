// Streaming fused phase 3 for chunks of 64 rows (instantiations).
#include "la_fwd_pipe.hpp"

namespace la {

hipError_t fwd_pipe_bf16(const FwdParams& p, int DK, int DVT, int64_t grid, hipStream_t s) {
    switch (DK * 1000 + DVT) {
        case 128064: return launch_fwd_pipe<128, 64>(p, grid, s);
        case 64064: return launch_fwd_pipe<64, 64>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
