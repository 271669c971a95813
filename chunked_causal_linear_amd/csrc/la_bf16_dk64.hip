// bf16 chunked forward and per-chunk states, feature width 64 (instantiations).
#include "la_chunked_bf16.hpp"

namespace la {

hipError_t fwd_bf16_dk64(const FwdParams& p, int DVT, int T, int64_t grid, hipStream_t s) {
    switch (DVT * 1000 + T) {
        case 16032: return launch_fwd_bf16<64, 16, 32>(p, grid, s);
        case 16064: return launch_fwd_bf16<64, 16, 64>(p, grid, s);
        case 16128: return launch_fwd_bf16<64, 16, 128>(p, grid, s);
        case 32032: return launch_fwd_bf16<64, 32, 32>(p, grid, s);
        case 32064: return launch_fwd_bf16<64, 32, 64>(p, grid, s);
        case 32128: return launch_fwd_bf16<64, 32, 128>(p, grid, s);
        case 64032: return launch_fwd_bf16<64, 64, 32>(p, grid, s);
        case 64064: return launch_fwd_bf16<64, 64, 64>(p, grid, s);
        case 64128: return launch_fwd_bf16<64, 64, 128>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t states_bf16_dk64(const StatesParams& p, int DVT, int64_t grid, hipStream_t s) {
    switch (DVT) {
        case 16: return launch_states_bf16<64, 16>(p, grid, s);
        case 32: return launch_states_bf16<64, 32>(p, grid, s);
        case 64: return launch_states_bf16<64, 64>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
