// Phase 1 as a stream: the state of a long run of rows, S = phi(K)^T V (and
// z = the column sums of phi(K)), for runs whose rows are a whole number of
// 64-row tiles (page "attention と線形の間", section ②: the state of a chunk is
// the sum of its key-value outer products; page "Linear Attention /
// Performerの理論と実装", RNN view, for z).  Tiles are 64 rows (32 at feature
// width 256).
//
// The workgroup layout is that of the streaming forward: two copy waves move
// K (and the residual of a pre-mapped phi(K)) and V tiles into a ring of LDS
// stages with direct-to-LDS copies; two compute waves accumulate the state of
// half of a 64-column value tile each in fp32 accumulators, A = K columns and
// B = V columns (a block of ones for z), read with transpose reads.  There are
// no outputs to store: per tile the copy waves refill a stage and wait for the
// next tile, the compute waves multiply.
//
// Three kinds of K:
//   KIND_PLAIN  bf16 K as it is (identity map);
//   KIND_ELU    elu+1 of in_scale * K, split into bf16 hi = bf16(phi) and
//               lo = bf16(phi - hi) in LDS (all four waves map a share of the
//               landed tile; a second barrier separates that from the
//               products), both multiplied, so that the long sum carries phi
//               to about 2^-17 rather than to the bf16 rounding of phi;
//   KIND_LO     pre-mapped phi(K) with its residual in a second input
//               (FAVOR+), both copied and both multiplied.
// K rows past the end of the sequence are set to zero before the products.
//
// Decayed recurrence (DECAY; S_t = gamma S_{t-1} + k_t^T v_t): the state a run
// leaves at its end weighs row r by gamma^(e-1-r), e the run's end, and the
// scan decays the prefix by each run's row count.  With elu+1 the weight
// multiplies phi(k) in fp32 before the hi/lo split (the sum keeps its
// precision, V stays exact); with plain K the compute waves weight each V
// operand and the ones of z (fp32 multiply, rounded back to bf16, one rounding
// as with the weight on K).  Pre-mapped K with its residual has no decayed
// form here.
#pragma once

#include "la_fwd_pipe.hpp"

namespace la {

enum { KIND_PLAIN = 0, KIND_ELU = 1, KIND_LO = 2 };

namespace pipe {

template <int DK, int DVT, int TT, bool LO>
struct alignas(16) StateStage {
    u16 k[TT * DK];
    u16 klo[LO ? TT * DK : 8];
    u16 v[TT * DVT];
};

// wait until the copies of a tile have landed when those of `after` more tiles
// (NL copies each) were issued after them; after <= A (the counts are
// immediates, so each is picked by a branch)
template <int NL, int A>
__device__ __forceinline__ void wait_tiles(int after) {
    if constexpr (A > 0) {
        if (after >= A) {
            wait_vm<A * NL>();
            return;
        }
        wait_tiles<NL, A - 1>(after);
    } else {
        wait_vm<0>();
    }
}

}  // namespace pipe

// With elu+1 applied here at feature width 64, two workgroups share a CU
// (three stages each, at most 256 VGPRs), so that the mapping of one overlaps
// the other's waits (measured: 129 us against 157 with one workgroup of six
// stages per CU at 32 heads x 65536 rows in 1024 pieces); otherwise one
// workgroup per CU with as many stages as fit.
template <int DK, int KIND>
constexpr int states_pipe_per_cu() { return KIND == KIND_ELU && DK == 64 ? 2 : 1; }

template <int DK, int DVT, int KIND, bool Z, bool DECAY>
__global__ __launch_bounds__(4 * WAVE) __attribute__((amdgpu_waves_per_eu(states_pipe_per_cu<DK, KIND>(),
                                                                           states_pipe_per_cu<DK, KIND>())))
void chunk_states_pipe(StatesParams p) {
    using namespace pipe;
    constexpr int TT = DK == 256 ? 32 : 64;        // rows per tile (four stages fit at every width)
    constexpr bool LO = KIND != KIND_PLAIN;        // a residual tile
    typedef StateStage<DK, DVT, TT, LO> StageT;
    constexpr int NFIT = (int)(160 * 1024 / sizeof(StageT));
    constexpr int NMAX = states_pipe_per_cu<DK, KIND>() == 2 ? 3 : 8;
    constexpr int NSTAGE = NFIT < NMAX ? NFIT : NMAX;  // LDS stages
    constexpr int CPW = DVT / 32;                  // 16-column blocks per compute wave
    constexpr int NCB = CPW + (Z ? 1 : 0);         // + the block of z
    constexpr int NKA = DK / 32;                   // 32-row blocks of the state
    constexpr int QSEG = DK / 8, VSEG = DVT / 8;
    constexpr int NCK = TT * QSEG / WAVE / 2;      // copy instructions per tile and copy wave, K
    constexpr int NCV = TT * VSEG / WAVE / 2;      // the same for V
    constexpr int NL = NCK * (KIND == KIND_LO ? 2 : 1) + NCV;  // per tile and copy wave
    static_assert(DVT == 64, "tiles of 64 value columns");
    static_assert(DK == 64 || DK == 128 || DK == 256, "feature width 64, 128 or 256");
    static_assert(NSTAGE >= 2 && (NSTAGE - 2) * NL < 64, "stages and vmcnt range");
    static_assert(NCK % 4 == 0, "mapping shares");

    __shared__ StageT st[NSTAGE];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const bool copier = wave >= 2;                               // wave-uniform
    const int h = __builtin_amdgcn_readfirstlane(wave & 1);
    const int colw = h * CPW * 16;                               // first column of this compute wave

    const int w = work_index(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int64_t n = (w / p.n_dvt) % p.n_items;
    const int64_t bh = w / ((int64_t)p.n_dvt * p.n_items);
    const int col0 = jt * DVT;
    const int64_t L = p.L;
    const int dv = p.dv;
    const int64_t r_begin = n * p.C;
    const int64_t r_end = r_begin + p.C < L ? r_begin + p.C : L;
    const int64_t t_begin = r_begin / TT;
    const int64_t t_end = (r_end + TT - 1) / TT;

    auto valid_rows = [&](int64_t t) -> int { return (int)(L - t * TT < TT ? L - t * TT : TT); };

    // zero K rows past the end (and their residual)
    auto zero_tail = [&](StageT& s, int valid) __attribute__((always_inline)) {
        const int cnt = (TT - valid) * QSEG;
        uint4* kk = reinterpret_cast<uint4*>(s.k + valid * DK);
        for (int i = tid; i < cnt; i += 4 * WAVE) kk[i] = make_uint4(0, 0, 0, 0);
        if constexpr (LO) {
            uint4* kl = reinterpret_cast<uint4*>(s.klo + valid * DK);
            for (int i = tid; i < cnt; i += 4 * WAVE) kl[i] = make_uint4(0, 0, 0, 0);
        }
    };

    // elu+1 split of a landed K tile, in place (hi) and into the residual tile
    // (lo).  The tile is 2 NCK blocks of 64 16-byte pieces (lane l of a block
    // maps its piece l); copy wave h copies (and waits for) blocks
    // h NCK .. h NCK + NCK - 1, the list of pair h, j = 0 .. NCK - 1.  The
    // mapping is shared so that it overlaps the products: per tile t, copy wave
    // h maps FA blocks of its list of tile t + 1 as soon as its copies have
    // landed (only its own copies: the other copy wave's may still be in
    // flight) and FB more after B'(t), while the products of tile t run;
    // compute wave h maps the last FC between B(t) and B'(t).
    constexpr int FC = NCK / 4, FA = NCK / 4, FB = NCK - FC - FA;
    // FA entries before B'(t - 1) (own copies only); FB after it, when both
    // copy waves have waited for the tile; FC by the compute wave after B(t).
    // A stage is refilled only after B(t) of the tile it held, and with two
    // stages the tile mapped is the one just issued into it.
    static_assert(KIND != KIND_ELU || (piece_shares_ok<NCK, NCK, FA>() && FB >= 0 && FC >= 0),
                  "elu+1 shares: a copy wave maps only pieces it copied before the barrier; every piece once");
    // (decay: row r of the tile weighs gamma^(n - 1 - r), n its rows before the
    // run's end)
    auto phi_blocks = [&](StageT& s, int valid, int n, auto j0_, auto count) __attribute__((always_inline)) {
        constexpr int J0 = decltype(j0_)::value, N = decltype(count)::value;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int slot = PieceList<NCK>::block(h, J0 + i) * WAVE + lane;
            const uint4 x = *reinterpret_cast<const uint4*>(s.k + slot * 8);
            uint4 hi, lo;
            const float wr = DECAY ? __builtin_amdgcn_exp2f((float)(n - 1 - slot / QSEG) * p.log2_gamma) : 1.0f;
            elu1_split_bf16x8(x, p.in_scale, hi, lo, wr);
            const bool live = slot / QSEG < valid;  // rows past the end become zero
            *reinterpret_cast<uint4*>(s.k + slot * 8) = live ? hi : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(s.klo + slot * 8) = live ? lo : make_uint4(0, 0, 0, 0);
        }
    };
    // rows of tile t before the run's end
    auto rows_to_end = [&](int64_t t) -> int { return (int)(r_end - t * TT); };
    auto phi_copy_a = [&](StageT& s, int64_t t) __attribute__((always_inline)) {
        phi_blocks(s, valid_rows(t), rows_to_end(t), ic<0>{}, ic<FA>{});
    };
    auto phi_copy_b = [&](StageT& s, int64_t t) __attribute__((always_inline)) {
        phi_blocks(s, valid_rows(t), rows_to_end(t), ic<FA>{}, ic<FB>{});
    };
    auto phi_compute = [&](StageT& s, int64_t t) __attribute__((always_inline)) {
        phi_blocks(s, valid_rows(t), rows_to_end(t), ic<FA + FB>{}, ic<FC>{});
    };
    // after B(t), the landed tile t made ready for the products
    auto prepare = [&](StageT& s, int64_t t) __attribute__((always_inline)) {
        const int valid = valid_rows(t);
        if constexpr (KIND == KIND_ELU) {
            phi_compute(s, t);
            __syncthreads();  // B'(t)
        } else if (valid < TT) {
            zero_tail(s, valid);
            __syncthreads();
        }
    };

    if (copier) {
        // ================= copy wave h =================
        const u16* kh = p.k + bh * L * DK;
        const u16* klh = KIND == KIND_LO ? p.k_lo + bh * L * DK : nullptr;
        const u16* vh = p.v + bh * L * dv + col0;
        // lane l of copy instruction b lands in LDS slot 64 b + l = (row, physical
        // segment), which holds the global segment (physical ^ row) of that row;
        // rows past the end are clamped to the last row (and zeroed later)
        auto issue = [&](int64_t t, StageT& s) __attribute__((always_inline)) {
            const int64_t r0 = t * TT;
            const int last = (int)(L - 1 - r0);
            auto k_off = [&](int i) __attribute__((always_inline)) {
                const int slot = (h * NCK + i) * WAVE + lane;
                const int r = slot / QSEG, seg = (slot % QSEG) ^ (r & (QSEG - 1));
                return (uint32_t)(((r < last ? r : last) * DK + seg * 8) * 2);
            };
            const uint32_t lk = lds_addr(s.k), lv = lds_addr(s.v);
#pragma unroll
            for (int i = 0; i < NCK; ++i) dma16(kh + r0 * DK, k_off(i), lk + (h * NCK + i) * WAVE * 16);
            if constexpr (KIND == KIND_LO) {
                const uint32_t ll = lds_addr(s.klo);
#pragma unroll
                for (int i = 0; i < NCK; ++i) dma16(klh + r0 * DK, k_off(i), ll + (h * NCK + i) * WAVE * 16);
            }
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int b = h * NCV + i;
                const int slot = b * WAVE + lane;
                const int r = slot / VSEG, seg = (slot % VSEG) ^ (r & (VSEG - 1));
                dma16(vh + r0 * dv, (uint32_t)(((r < last ? r : last) * dv + seg * 8) * 2), lv + b * WAVE * 16);
            }
        };
        auto land = [&](int after) __attribute__((always_inline)) { wait_tiles<NL, NSTAGE - 2>(after); };
        auto after_of = [&](int64_t t) -> int {
            const int64_t newest = t + NSTAGE - 2 < t_end - 1 ? t + NSTAGE - 2 : t_end - 1;
            return (int)(newest - t);
        };

#pragma unroll
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (t_begin + s0 < t_end) issue(t_begin + s0, st[s0]);
        land(after_of(t_begin));
        if constexpr (KIND == KIND_ELU) {
            phi_copy_a(st[0], t_begin);
            phi_copy_b(st[0], t_begin);
        }

        int si = 0;  // stage of tile t
        for (int64_t t = t_begin; t < t_end; ++t) {
            const int sp = si == 0 ? NSTAGE - 1 : si - 1;  // stage of tile t - 1
            const int sn = si == NSTAGE - 1 ? 0 : si + 1;  // stage of tile t + 1
            __syncthreads();  // B(t): the compute waves are done with stage sp
            if (t + NSTAGE - 1 < t_end) issue(t + NSTAGE - 1, st[sp]);
            if constexpr (KIND == KIND_ELU) {
                if (t + 1 < t_end) {
                    land(after_of(t + 1));
                    phi_copy_a(st[sn], t + 1);
                }
                __syncthreads();  // B'(t): tile t is mapped
                if (t + 1 < t_end) phi_copy_b(st[sn], t + 1);
            } else {
                prepare(st[si], t);
                if (t + 1 < t_end) land(after_of(t + 1));
            }
            si = sn;
        }
        __syncthreads();  // the compute waves are done with the last stage
        return;
    }

    // ================= compute wave h =================
    // P[c][ks][hf] lane (l16, g) element i = state row a = 32 ks + 8 g + 4 hf + i,
    // column colw + 16 c + l16 (block c = CPW: z[a] in every column)
    f32x4 P[NCB][NKA][2];
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) P[c][ks][0] = P[c][ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    const int c4 = 4 * (lane & 3), c8 = 8 * (lane & 3);

    // P[a][j] += sum over the tile's keys of K[key][a] V[key][j], keys in the
    // permuted order of the column operands (the same for A and B)
    auto update = [&](const u16* ktile, const bf16x8 (&vb)[NCB][TT / 32]) __attribute__((always_inline)) {
        constexpr int NK = TT / 32;
        bf16x8 kc[2][NK];
        auto load_kc = [&](int ks, int hf, bf16x8 (&k_)[NK]) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) k_[kk] = col_op<QSEG>(ktile, kk * 32, ks * 32 + c8 + 4 * hf, lane);
        };
        load_kc(0, 0, kc[0]);
#pragma unroll
        for (int t = 0; t < 2 * NKA; ++t) {
            const int ks = t >> 1, hf = t & 1;
            if (t + 1 < 2 * NKA) load_kc((t + 1) >> 1, (t + 1) & 1, kc[(t + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                for (int c = 0; c < NCB; ++c) P[c][ks][hf] = mfma_bf16(kc[t & 1][kk], vb[c][kk], P[c][ks][hf]);
        }
    };
    auto compute = [&](const StageT& s, int64_t t) __attribute__((always_inline)) {
        constexpr int NK = TT / 32;
        bf16x8 vb[NCB][NK];
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
                vb[c][kk] = c < CPW ? col_op<VSEG>(s.v, kk * 32, colw + c * 16 + c4, lane) : ones;
        if constexpr (DECAY && KIND == KIND_PLAIN) {
            // operand element j holds row t TT + 32 kk + 4g + j (j < 4), + 16
            // (j >= 4): one power per run of four rows, taken at the run's last
            // row before the end e (so that it is at most 1), the earlier rows
            // by multiplying by gamma; rows from e on weigh 0
            const float lg = p.log2_gamma, gam = __builtin_amdgcn_exp2f(lg);
            const int n = (int)(r_end - t * TT);  // rows of the tile before e
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                float w[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r3 = 32 * kk + 16 * hh + 4 * g + 3;
                    const int top = r3 < n - 1 ? r3 : n - 1;
                    float wk = __builtin_amdgcn_exp2f((float)(n - 1 - top) * lg);
#pragma unroll
                    for (int j = 3; j >= 0; --j) {
                        const bool live = r3 - 3 + j < n;
                        w[4 * hh + j] = live ? wk : 0.f;
                        wk = live ? wk * gam : wk;
                    }
                }
#pragma unroll
                for (int c = 0; c < NCB; ++c) vb[c][kk] = c < CPW ? scale_bf16x8(vb[c][kk], w) : pack_bf16x8(w);
            }
        }
        update(s.k, vb);
        if constexpr (LO) update(s.klo, vb);
    };

    auto step = [&](auto sidx, int64_t t) __attribute__((always_inline)) {
        constexpr int SI = decltype(sidx)::value;
        __syncthreads();  // B(t)
        prepare(st[SI], t);
        compute(st[SI], t);
    };
    for (int64_t t = t_begin; t < t_end; t += NSTAGE) {
        step(ic<0>{}, t);
        if (t + 1 < t_end) step(ic<1>{}, t + 1);
        if constexpr (NSTAGE >= 3)
            if (t + 2 < t_end) step(ic<2>{}, t + 2);
        if constexpr (NSTAGE >= 4)
            if (t + 3 < t_end) step(ic<3>{}, t + 3);
        if constexpr (NSTAGE >= 5)
            if (t + 4 < t_end) step(ic<4>{}, t + 4);
        if constexpr (NSTAGE >= 6)
            if (t + 5 < t_end) step(ic<5>{}, t + 5);
        if constexpr (NSTAGE >= 7)
            if (t + 6 < t_end) step(ic<6>{}, t + 6);
        if constexpr (NSTAGE >= 8)
            if (t + 7 < t_end) step(ic<7>{}, t + 7);
    }
    __syncthreads();  // matches the copy waves' final barrier

    float* S = p.S + ((bh * p.n_out + n) * DK) * (int64_t)dv + col0 + colw + l16;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[(int64_t)(32 * ks + 8 * g + 4 * hf + i) * dv + c * 16] = P[c][ks][hf][i];
    if constexpr (Z) {
        if (jt == 0 && h == 0 && l16 == 0) {
            float* z = p.z + (bh * p.n_out + n) * DK;
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[32 * ks + 8 * g + 4 * hf + i] = P[CPW][ks][hf][i];
        }
    }
}

// launch over the compile-time cases of one feature width (z from p.want_z)
template <int DK, bool DECAY>
hipError_t states_pipe_dk(const StatesParams& p, int kind, int64_t grid, hipStream_t s) {
    constexpr int DVT = 64;
    const dim3 g((unsigned)grid), b(4 * WAVE);
    const bool z = p.want_z != 0;
    switch (kind * 2 + (z ? 1 : 0)) {
        case 0: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_PLAIN, false, DECAY>), g, b, 0, s, p); break;
        case 1: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_PLAIN, true, DECAY>), g, b, 0, s, p); break;
        case 2: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_ELU, false, DECAY>), g, b, 0, s, p); break;
        case 3: hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_ELU, true, DECAY>), g, b, 0, s, p); break;
        case 4:
        case 5:
            if constexpr (DECAY) {
                return hipErrorInvalidValue;  // no decayed form with a residual
            } else {
                if (z)
                    hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_LO, true, false>), g, b, 0, s, p);
                else
                    hipLaunchKernelGGL((chunk_states_pipe<DK, DVT, KIND_LO, false, false>), g, b, 0, s, p);
            }
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// the decayed instantiations (la_states_pipe_decay.hip)
hipError_t states_pipe_decay_bf16(const StatesParams& p, int DK, int kind, int64_t grid, hipStream_t s);

}  // namespace la
