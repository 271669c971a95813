// int8 chunked forward and per-chunk states (instantiations).
#include "la_chunked_i8.hpp"

namespace la {

hipError_t run_chunked_fwd_i8(const FwdParamsI8& p, int DK, int DVT, int T, int64_t grid, hipStream_t s) {
    switch (DK * 1000000 + DVT * 1000 + T) {
        case 64016064: return launch_fwd_i8<64, 16, 64>(p, grid, s);
        case 64016128: return launch_fwd_i8<64, 16, 128>(p, grid, s);
        case 64032064: return launch_fwd_i8<64, 32, 64>(p, grid, s);
        case 64032128: return launch_fwd_i8<64, 32, 128>(p, grid, s);
        case 64064064: return launch_fwd_i8<64, 64, 64>(p, grid, s);
        case 64064128: return launch_fwd_i8<64, 64, 128>(p, grid, s);
        case 128016064: return launch_fwd_i8<128, 16, 64>(p, grid, s);
        case 128032064: return launch_fwd_i8<128, 32, 64>(p, grid, s);
        case 128064064: return launch_fwd_i8<128, 64, 64>(p, grid, s);
        case 128064128: return launch_fwd_i8<128, 64, 128>(p, grid, s);
        case 256016064: return launch_fwd_i8<256, 16, 64>(p, grid, s);
        case 256032064: return launch_fwd_i8<256, 32, 64>(p, grid, s);
        case 256064064: return launch_fwd_i8<256, 64, 64>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t run_chunk_states_i8(const StatesParamsI8& p, int DK, int DVT, int64_t grid, hipStream_t s) {
    switch (DK * 1000 + DVT) {
        case 64016: return launch_states_i8<64, 16>(p, grid, s);
        case 64032: return launch_states_i8<64, 32>(p, grid, s);
        case 64064: return launch_states_i8<64, 64>(p, grid, s);
        case 128016: return launch_states_i8<128, 16>(p, grid, s);
        case 128032: return launch_states_i8<128, 32>(p, grid, s);
        case 128064: return launch_states_i8<128, 64>(p, grid, s);
        case 256016: return launch_states_i8<256, 16>(p, grid, s);
        case 256032: return launch_states_i8<256, 32>(p, grid, s);
        case 256064: return launch_states_i8<256, 64>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la
