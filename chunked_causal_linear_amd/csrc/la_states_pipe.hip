// Streaming phase 1 (instantiations): feature width 64, 128 or 256, the three
// kinds of K, with or without z; the decayed recurrence in
// la_states_pipe_decay.hip.
#include "la_states_pipe.hpp"

namespace la {

hipError_t states_pipe_bf16(const StatesParams& p, int DK, int kind, int64_t grid, hipStream_t s) {
    if (p.log2_gamma != 0.0f) return states_pipe_decay_bf16(p, DK, kind, grid, s);
    switch (DK) {
        case 64: return states_pipe_dk<64, false>(p, kind, grid, s);
        case 128: return states_pipe_dk<128, false>(p, kind, grid, s);
        case 256: return states_pipe_dk<256, false>(p, kind, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
