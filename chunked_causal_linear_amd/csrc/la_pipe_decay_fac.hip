// Streaming fused phase 3 with the decayed recurrence in its factored form
// (state held as a wave-uniform power of gamma times a rescaled state; every
// weight on the V operands, one row factor per output): instantiations for
// chunks of 32, 64 or 128 rows at feature width 64 and chunks of 32 or 64 at
// feature width 128.
#include "la_pipe.hpp"

namespace la {

bool fwd_pipe_decay_fac_bf16(const FwdParams& p, int DK, int C, int64_t grid, hipStream_t s, hipError_t* e) {
    switch (DK * 1000 + C) {
        case 128032: *e = pipe::by_flags<128, 32, DECAY_FACTORED>(p, grid, s); return true;
        case 128064: *e = pipe::by_flags<128, 64, DECAY_FACTORED>(p, grid, s); return true;
        case 64032: *e = pipe::by_flags<64, 32, DECAY_FACTORED>(p, grid, s); return true;
        case 64064: *e = pipe::by_flags<64, 64, DECAY_FACTORED>(p, grid, s); return true;
        case 64128: *e = pipe::by_flags<64, 128, DECAY_FACTORED>(p, grid, s); return true;
    }
    return false;
}

}  // namespace la
