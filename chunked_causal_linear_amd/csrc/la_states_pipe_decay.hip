// Streaming phase 1 with the decayed recurrence (instantiations): feature
// width 64, 128 or 256, the three kinds of K, with or without z.
#include "la_states_pipe.hpp"

namespace la {

hipError_t states_pipe_decay_bf16(const StatesParams& p, int DK, int kind, int64_t grid, hipStream_t s) {
    switch (DK) {
        case 64: return states_pipe_dk<64, true>(p, kind, grid, s);
        case 128: return states_pipe_dk<128, true>(p, kind, grid, s);
        case 256: return states_pipe_dk<256, true>(p, kind, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace la
