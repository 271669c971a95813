// Streaming fused phase 3 for chunks of 32, 64 or 128 rows (instantiations).
#include "la_fwd_pipe.hpp"

namespace la {

hipError_t fwd_pipe_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s) {
    if (DVT != 64) return hipErrorInvalidValue;
    switch (DK * 1000 + C) {
        case 128032: return launch_fwd_pipe<128, 64, 32>(p, grid, s);
        case 128064: return launch_fwd_pipe<128, 64, 64>(p, grid, s);
        case 128128: return launch_fwd_pipe<128, 64, 128>(p, grid, s);
        case 64032: return launch_fwd_pipe<64, 64, 32>(p, grid, s);
        case 64064: return launch_fwd_pipe<64, 64, 64>(p, grid, s);
        case 64128: return launch_fwd_pipe<64, 64, 128>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
