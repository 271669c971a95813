// Streaming phase 1 (instantiations): feature width 64, 128 or 256, the three
// kinds of K, with or without z.
#include "la_states_pipe.hpp"

namespace la {

template <int DK>
static hipError_t states_pipe_dk(const StatesParams& p, int kind, int64_t grid, hipStream_t s) {
    constexpr int DVT = 64;
    const dim3 g((unsigned)grid), b(4 * WAVE);
    const bool z = p.want_z != 0;
    switch (kind * 2 + (z ? 1 : 0)) {
        case 0: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_PLAIN, false>), g, b, 0, s, p); break;
        case 1: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_PLAIN, true>), g, b, 0, s, p); break;
        case 2: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_ELU, false>), g, b, 0, s, p); break;
        case 3: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_ELU, true>), g, b, 0, s, p); break;
        case 4: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_LO, false>), g, b, 0, s, p); break;
        case 5: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_LO, true>), g, b, 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t states_pipe_bf16(const StatesParams& p, int DK, int kind, int64_t grid, hipStream_t s) {
    switch (DK) {
        case 64: return states_pipe_dk<64>(p, kind, grid, s);
        case 128: return states_pipe_dk<128>(p, kind, grid, s);
        case 256: return states_pipe_dk<256>(p, kind, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
