// Dispatch of the streaming phase-3 kernel over its compile-time cases.
#pragma once

#include "la_fwd_pipe.hpp"

namespace la {

hipError_t fwd_pipe_decay_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s);
// the decayed recurrence in its factored form (la_pipe_decay_fac.hip); false
// when the case has no such instantiation
bool fwd_pipe_decay_fac_bf16(const FwdParams& p, int DK, int C, int64_t grid, hipStream_t s, hipError_t* e);
// the cases with the most live registers (la_pipe_wide.hip)
hipError_t fwd_pipe_wide_bf16(const FwdParams& p, int DK, int C, bool decay, int64_t grid, hipStream_t s);

// the cases every instantiation file accepts
inline bool pipe_args_ok(const FwdParams& p, int DK, int DVT) {
    if (DVT != (DK == 256 ? 32 : 64) || p.noncausal || p.out_f32 || p.k_lo != nullptr) return false;
    return p.fmap == FMAP_NONE || p.fmap == FMAP_ELU1;
}

namespace pipe {

// normaliser from p.normalize; elu+1 applied in the kernel from p.fmap;
// tiles of 64 value columns, 32 at feature width 256 (LDS and registers)
template <int DK, int C, int DECAY>
hipError_t by_flags(const FwdParams& p, int64_t grid, hipStream_t s) {
    constexpr int DVT = DK == 256 ? 32 : 64;
    const bool norm = p.normalize != 0;
    if (p.fmap == FMAP_ELU1)
        return norm ? launch_fwd_pipe<DK, DVT, C, true, true, DECAY>(p, grid, s)
                    : launch_fwd_pipe<DK, DVT, C, false, true, DECAY>(p, grid, s);
    return norm ? launch_fwd_pipe<DK, DVT, C, true, false, DECAY>(p, grid, s)
                : launch_fwd_pipe<DK, DVT, C, false, false, DECAY>(p, grid, s);
}

}  // namespace pipe

}  // namespace la
