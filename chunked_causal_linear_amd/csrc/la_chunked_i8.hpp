// Exact int8 -> int32 path of the chunked forward and of the per-chunk states
// (gfx950 int8 matrix cores, 16x16x64, int32 accumulate).
//
// Same algorithm and work split as the bf16 kernels (la_chunked_bf16.hpp):
// one workgroup walks the chunks of a group with the state P (int32) held in
// its registers, per chunk
//     O_c = Q_c P + tril(Q_c K_c^T) V_c ,   P += K_c^T V_c
// (page "attention と線形の間", section ②).  Products of int8 operands are
// exact in int32.  The two products whose left or right operand is an int32
// quantity - the masked scores S times V, and Q times the state P - split that
// operand into signed bytes (x = d0 + 256 d1 + 65536 d2 + 2^24 d3, each
// d in [-128, 127]) and run one int8 product per byte; the partial results are
// recombined with shifts in wrapping int32 arithmetic, which is exact modulo
// 2^32 and therefore exact whenever the true result fits in int32.
#pragma once

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

namespace detail_i8 {

template <int DK, int DVT, int T>
struct GeoI8 {
    static constexpr int TK = T < 64 ? 64 : T;  // key extent (k-steps of 64)
    static constexpr int QS = DK + 16;          // row stride (bytes) of Q, K tiles
    static constexpr int KS = TK + 16;          // row stride of K^T, V^T, score limbs
};

struct TileI8 {
    int64_t row0;
    int valid;
};

// A unit is 4 rows x 16 int8 columns.
template <int R, int W, int NT>
struct UnitsI8 {
    static constexpr int N = (R / 4) * (W / 16);
    static constexpr int PER_THREAD = (N + NT - 1) / NT;
};

template <int R, int W, int NT>
struct URegsI8 {
    uint4 r[UnitsI8<R, W, NT>::PER_THREAD][4];
};

template <int R, int W, int NT>
__device__ __forceinline__ void load_units_i8(URegsI8<R, W, NT>& reg, const signed char* __restrict__ base,
                                              int64_t row_stride, int col0, int cols_valid, const TileI8& t,
                                              int tid) {
    constexpr int CG = W / 16;
#pragma unroll
    for (int it = 0; it < UnitsI8<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        const int cg = u % CG, rg = u / CG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rg * 4 + i;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (u < UnitsI8<R, W, NT>::N && r < t.valid && cg * 16 < cols_valid) {
                const signed char* p = base + (t.row0 + r) * row_stride + col0 + cg * 16;
                val = *reinterpret_cast<const uint4*>(p);
            }
            reg.r[it][i] = val;
        }
    }
}

template <int R, int W, int NT>
__device__ __forceinline__ void store_rows_i8(const URegsI8<R, W, NT>& reg, signed char* dst, int stride, int tid) {
    constexpr int CG = W / 16;
#pragma unroll
    for (int it = 0; it < UnitsI8<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        if (u < UnitsI8<R, W, NT>::N) {
            const int cg = u % CG, rg = u / CG;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(dst + (rg * 4 + i) * stride + cg * 16) = reg.r[it][i];
        }
    }
}

// 4 rows of 4 bytes -> 4 columns of 4 bytes
__device__ __forceinline__ void transpose4x4_bytes(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                                   uint32_t out[4]) {
    const uint32_t x = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
    const uint32_t y = __builtin_amdgcn_perm(r3, r2, 0x05010400u);  // r2.b0 r3.b0 r2.b1 r3.b1
    const uint32_t x2 = __builtin_amdgcn_perm(r1, r0, 0x07030602u); // r0.b2 r1.b2 r0.b3 r1.b3
    const uint32_t y2 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(y, x, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(y, x, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(y2, x2, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(y2, x2, 0x07060302u);
}

// transposed store: column c (0..15) of the unit -> dst[(16*cg + c) * stride + 4*rg .. +3]
template <int R, int W, int NT>
__device__ __forceinline__ void store_transposed_i8(const URegsI8<R, W, NT>& reg, signed char* dst, int stride,
                                                    int tid) {
    constexpr int CG = W / 16;
#pragma unroll
    for (int it = 0; it < UnitsI8<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        if (u < UnitsI8<R, W, NT>::N) {
            const int cg = u % CG, rg = u / CG;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t cols[4];
                transpose4x4_bytes(word(reg.r[it][0], j), word(reg.r[it][1], j), word(reg.r[it][2], j),
                                   word(reg.r[it][3], j), cols);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<uint32_t*>(dst + (cg * 16 + j * 4 + c) * stride + rg * 4) = cols[c];
            }
        }
    }
}

__device__ __forceinline__ int work_index_i8(int remap) {
    const int b = blockIdx.x;
    if (!remap) return b;
    const int per = gridDim.x >> 3;
    return (b & 7) * per + (b >> 3);
}

// signed byte j of x (x = sum_j byte_j * 256^j, each byte in [-128, 127])
__device__ __forceinline__ void split_bytes(int x, int out[4]) {
    // exact signed-digit split computed in wrapping arithmetic
    unsigned u = (unsigned)x;
    int r0 = (int)(signed char)(u & 0xFFu);
    u = (u - (unsigned)r0) >> 8;
    int r1 = (int)(signed char)(u & 0xFFu);
    u = (u - (unsigned)r1) >> 8;
    int r2 = (int)(signed char)(u & 0xFFu);
    u = (u - (unsigned)r2) >> 8;
    int r3 = (int)(signed char)(u & 0xFFu);
    out[0] = r0;
    out[1] = r1;
    out[2] = r2;
    out[3] = r3;
}

__device__ __forceinline__ uint32_t pack4_bytes(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

}  // namespace detail_i8

using namespace detail_i8;

// ===========================================================================
// Phase 3, int8
// ===========================================================================
// With 64-row tiles at feature width up to 128, at most 256 VGPRs so that two
// workgroups share a CU (their loads and barriers overlap; measured 0.68 ->
// 0.63 ms at 128 heads x 8192 rows, d 128); wider cases keep their registers.
template <int DK, int T>
constexpr int i8_waves_per_eu() { return DK <= 128 && T == 64 ? 2 : 1; }

template <int DK, int DVT, int T, int NW>
__global__ __launch_bounds__(NW * WAVE)
__attribute__((amdgpu_waves_per_eu(i8_waves_per_eu<DK, T>(), i8_waves_per_eu<DK, T>())))
void chunked_fwd_i8(FwdParamsI8 p) {
    using G = GeoI8<DK, DVT, T>;
    constexpr int NT = NW * WAVE;
    constexpr int NB = T / 16;
    constexpr int NAB = DK / 16;
    constexpr int NKS_A = DK / 64;
    constexpr int NKS_K = G::TK / 64;
    constexpr int CB = DVT / 16;
    constexpr int CPW = CB / NW;
    constexpr int NL_S = 3;  // byte limbs of a score (|s| < 2^23)
    constexpr int NL_P = 4;  // byte limbs of a state entry (any int32)
    static_assert(CPW * NW == CB, "column blocks must split evenly over waves");

    __shared__ __attribute__((aligned(16))) signed char Qs[T * G::QS];
    __shared__ __attribute__((aligned(16))) signed char Ks[T * G::QS];
    __shared__ __attribute__((aligned(16))) signed char KTs[DK * G::KS];
    __shared__ __attribute__((aligned(16))) signed char VTs[DVT * G::KS];
    __shared__ __attribute__((aligned(16))) signed char Ss[NL_S][T * G::KS];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;

    const int w = work_index_i8(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int grp = (w / p.n_dvt) % p.n_groups;
    const int64_t bh = w / (p.n_dvt * p.n_groups);
    const int col0 = jt * DVT;

    const int64_t L = p.L;
    const int C = p.C;
    const int64_t n_chunks = (L + C - 1) / C;
    const int64_t c_begin = (int64_t)grp * p.G;
    const int64_t c_end = c_begin + p.G < n_chunks ? c_begin + p.G : n_chunks;

    const signed char* __restrict__ qh = p.q + bh * L * p.dk_g;
    const signed char* __restrict__ kh = p.k + bh * L * p.dk_g;
    const signed char* __restrict__ vh = p.v + bh * L * p.dv;

    for (int i = tid; i < T * G::QS / 4; i += NT) {
        reinterpret_cast<int*>(Qs)[i] = 0;
        reinterpret_cast<int*>(Ks)[i] = 0;
    }
    for (int i = tid; i < DK * G::KS / 4; i += NT) reinterpret_cast<int*>(KTs)[i] = 0;
    for (int i = tid; i < DVT * G::KS / 4; i += NT) reinterpret_cast<int*>(VTs)[i] = 0;
    for (int i = tid; i < NL_S * T * G::KS / 4; i += NT) reinterpret_cast<int*>(&Ss[0][0])[i] = 0;

    i32x4 P[CPW][NAB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) P[c][ab] = i32x4{0, 0, 0, 0};
    const int p0_sub = p.p0_sub > 1 ? p.p0_sub : 1;
    const int p0_groups = p.noncausal ? 1 : p.n_groups * p0_sub;
    const int p0_index = p.noncausal ? 0 : grp * p0_sub;
    if (p.P0 != nullptr && (grp > 0 || p.noncausal)) {
        const int* P0 = p.P0 + ((bh * p0_groups + p0_index) * p.dk_g) * (int64_t)p.dv;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int j = col0 + (wave + c * NW) * 16 + l16;
#pragma unroll
            for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int a = ab * 16 + g * 4 + i;
                    P[c][ab][i] = (a < p.dk_g && j < p.dv) ? P0[(int64_t)a * p.dv + j] : 0;
                }
        }
    }

    URegsI8<T, DK, NT> rq, rk;
    URegsI8<T, DVT, NT> rv;

    auto tile_of = [&](int64_t chunk, int sub) -> TileI8 {
        const int64_t cs = chunk * C;
        const int64_t ce = cs + C < L ? cs + C : L;
        const int64_t r0 = cs + (int64_t)sub * T;
        const int64_t re = r0 + T < ce ? r0 + T : ce;
        return TileI8{r0, (int)(re - r0)};
    };

    // scores -> byte limbs in Ss
    auto scores = [&](bool diagonal) {
        constexpr int NBLK = NB * NB;
        for (int blk = wave; blk < NBLK; blk += NW) {
            const int qb = blk / NB, kb = blk % NB;
            if (diagonal) {
                const int kb_lim = 4 * ((qb + 4) / 4);  // blocks covered by 64-key k-steps
                if (kb >= kb_lim) continue;
                if (kb > qb) {
#pragma unroll
                    for (int l = 0; l < NL_S; ++l)
                        *reinterpret_cast<uint32_t*>(Ss[l] + (qb * 16 + l16) * G::KS + kb * 16 + g * 4) = 0u;
                    continue;
                }
            }
            i32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < NKS_A; ++ks) {
                const i32x4 a = *reinterpret_cast<const i32x4*>(Ks + (kb * 16 + l16) * G::QS + ks * 64 + g * 16);
                const i32x4 b = *reinterpret_cast<const i32x4*>(Qs + (qb * 16 + l16) * G::QS + ks * 64 + g * 16);
                acc = mfma_i8(a, b, acc);
            }
            if (diagonal && kb == qb) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (g * 4 + i > l16) acc[i] = 0;
            }
            int d[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split_bytes(acc[i], d[i]);
#pragma unroll
            for (int l = 0; l < NL_S; ++l)
                *reinterpret_cast<uint32_t*>(Ss[l] + (qb * 16 + l16) * G::KS + kb * 16 + g * 4) =
                    pack4_bytes(d[0][l], d[1][l], d[2][l], d[3][l]);
        }
    };

    i32x4 O[NL_P][CPW][NB];

    for (int64_t chunk = c_begin; chunk < c_end; ++chunk) {
        const int64_t cs = chunk * C;
        const int64_t ce = cs + C < L ? cs + C : L;
        const int nsub = (int)((ce - cs + T - 1) / T);

        // byte limbs of the state at the chunk start (B operand of Q P)
        i32x4 Pl[NL_P][CPW][NKS_A];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKS_A; ++ks) {
                int d[4][4][4];  // [block b][i][limb]
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) split_bytes(P[c][4 * ks + b][i], d[b][i]);
#pragma unroll
                for (int l = 0; l < NL_P; ++l)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        Pl[l][c][ks][b] = (int)pack4_bytes(d[b][0][l], d[b][1][l], d[b][2][l], d[b][3][l]);
            }

        for (int sub = 0; sub < nsub; ++sub) {
            const TileI8 t = tile_of(chunk, sub);
            load_units_i8<T, DK, NT>(rq, qh, p.dk_g, 0, p.dk_g, t, tid);
            load_units_i8<T, DK, NT>(rk, kh, p.dk_g, 0, p.dk_g, t, tid);
            load_units_i8<T, DVT, NT>(rv, vh, p.dv, col0, p.dv - col0, t, tid);
            __syncthreads();
            store_rows_i8<T, DK, NT>(rq, Qs, G::QS, tid);
            store_rows_i8<T, DK, NT>(rk, Ks, G::QS, tid);
            store_transposed_i8<T, DK, NT>(rk, KTs, G::KS, tid);
            store_transposed_i8<T, DVT, NT>(rv, VTs, G::KS, tid);
            __syncthreads();
            if (!p.noncausal) scores(true);
            __syncthreads();

            i32x4 vb[CPW][NKS_K];
#pragma unroll
            for (int c = 0; c < CPW; ++c)
#pragma unroll
                for (int ks = 0; ks < NKS_K; ++ks)
                    vb[c][ks] = *reinterpret_cast<const i32x4*>(VTs + ((wave + c * NW) * 16 + l16) * G::KS + ks * 64 + g * 16);

#pragma unroll
            for (int qb = 0; qb < NB; ++qb) {
#pragma unroll
                for (int l = 0; l < NL_P; ++l)
#pragma unroll
                    for (int c = 0; c < CPW; ++c) O[l][c][qb] = i32x4{0, 0, 0, 0};
                // inter: A = Q with the a's of the state accumulators (blocks 4ks+b, rows 4g..4g+3)
#pragma unroll
                for (int ks = 0; ks < NKS_A; ++ks) {
                    const signed char* qrow = Qs + (qb * 16 + l16) * G::QS + ks * 64 + g * 4;
                    i32x4 a;
#pragma unroll
                    for (int b = 0; b < 4; ++b) a[b] = *reinterpret_cast<const int*>(qrow + 16 * b);
#pragma unroll
                    for (int l = 0; l < NL_P; ++l)
#pragma unroll
                        for (int c = 0; c < CPW; ++c) O[l][c][qb] = mfma_i8(a, Pl[l][c][ks], O[l][c][qb]);
                }
                // intra: score limbs times V
                const int nks = p.noncausal ? 0 : (qb + 4) / 4;
                for (int ks = 0; ks < nks; ++ks) {
#pragma unroll
                    for (int l = 0; l < NL_S; ++l) {
                        const i32x4 a = *reinterpret_cast<const i32x4*>(Ss[l] + (qb * 16 + l16) * G::KS + ks * 64 + g * 16);
#pragma unroll
                        for (int c = 0; c < CPW; ++c) O[l][c][qb] = mfma_i8(a, vb[c][ks], O[l][c][qb]);
                    }
                }
            }

            // state update
            if (!p.noncausal)
#pragma unroll
            for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
                for (int ks = 0; ks < NKS_K; ++ks) {
                    const i32x4 a = *reinterpret_cast<const i32x4*>(KTs + (ab * 16 + l16) * G::KS + ks * 64 + g * 16);
#pragma unroll
                    for (int c = 0; c < CPW; ++c) P[c][ab] = mfma_i8(a, vb[c][ks], P[c][ab]);
                }

            // earlier sub-tiles of the same chunk (C > T)
            for (int prev = 0; prev < sub; ++prev) {
                const TileI8 tp = tile_of(chunk, prev);
                __syncthreads();
                load_units_i8<T, DK, NT>(rk, kh, p.dk_g, 0, p.dk_g, tp, tid);
                load_units_i8<T, DVT, NT>(rv, vh, p.dv, col0, p.dv - col0, tp, tid);
                store_rows_i8<T, DK, NT>(rk, Ks, G::QS, tid);
                store_transposed_i8<T, DVT, NT>(rv, VTs, G::KS, tid);
                __syncthreads();
                scores(false);
                __syncthreads();
#pragma unroll
                for (int c = 0; c < CPW; ++c)
#pragma unroll
                    for (int ks = 0; ks < NKS_K; ++ks)
                        vb[c][ks] = *reinterpret_cast<const i32x4*>(VTs + ((wave + c * NW) * 16 + l16) * G::KS + ks * 64 + g * 16);
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                    for (int ks = 0; ks < NKS_K; ++ks)
#pragma unroll
                        for (int l = 0; l < NL_S; ++l) {
                            const i32x4 a = *reinterpret_cast<const i32x4*>(Ss[l] + (qb * 16 + l16) * G::KS + ks * 64 + g * 16);
#pragma unroll
                            for (int c = 0; c < CPW; ++c) O[l][c][qb] = mfma_i8(a, vb[c][ks], O[l][c][qb]);
                        }
            }

            // recombine the limbs and store
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const int j = col0 + (wave + c * NW) * 16 + l16;
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = qb * 16 + g * 4 + i;
                        const unsigned val = (unsigned)O[0][c][qb][i] + ((unsigned)O[1][c][qb][i] << 8) +
                                             ((unsigned)O[2][c][qb][i] << 16) + ((unsigned)O[3][c][qb][i] << 24);
                        if (r < t.valid && j < p.dv) p.o[(bh * L + t.row0 + r) * p.dv + j] = (int)val;
                    }
            }
        }
    }

    const bool writes_final = p.noncausal ? (grp == 0) : (c_end == n_chunks);
    if (writes_final && p.S_final != nullptr) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int j = col0 + (wave + c * NW) * 16 + l16;
            if (j < p.dv) {
#pragma unroll
                for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int a = ab * 16 + g * 4 + i;
                        if (a < p.dk_g) p.S_final[(bh * p.dk_g + a) * p.dv + j] = P[c][ab][i];
                    }
            }
        }
    }
}

// ===========================================================================
// Phase 1, int8
// ===========================================================================
template <int DK, int DVT, int NW>
__global__ __launch_bounds__(NW * WAVE) void chunk_states_i8(StatesParamsI8 p) {
    constexpr int T = 64;
    using G = GeoI8<DK, DVT, T>;
    constexpr int NT = NW * WAVE;
    constexpr int NAB = DK / 16;
    constexpr int NKS_K = G::TK / 64;
    constexpr int CB = DVT / 16;
    constexpr int CPW = CB / NW;

    __shared__ __attribute__((aligned(16))) signed char KTs[DK * G::KS];
    __shared__ __attribute__((aligned(16))) signed char VTs[DVT * G::KS];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int w = work_index_i8(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int64_t n = (w / p.n_dvt) % p.n_items;
    const int64_t bh = w / (p.n_dvt * p.n_items);
    const int col0 = jt * DVT;
    const int64_t L = p.L;
    const int64_t cs = n * p.C;
    const int64_t ce = cs + p.C < L ? cs + p.C : L;

    const signed char* __restrict__ kh = p.k + bh * L * p.dk_g;
    const signed char* __restrict__ vh = p.v + bh * L * p.dv;

    i32x4 P[CPW][NAB];
    int zacc[NAB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) P[c][ab] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) zacc[ab] = 0;

    URegsI8<T, DK, NT> rk;
    URegsI8<T, DVT, NT> rv;
    for (int64_t r0 = cs; r0 < ce; r0 += T) {
        const TileI8 t{r0, (int)((ce - r0) < T ? (ce - r0) : T)};
        load_units_i8<T, DK, NT>(rk, kh, p.dk_g, 0, p.dk_g, t, tid);
        load_units_i8<T, DVT, NT>(rv, vh, p.dv, col0, p.dv - col0, t, tid);
        __syncthreads();
        store_transposed_i8<T, DK, NT>(rk, KTs, G::KS, tid);
        store_transposed_i8<T, DVT, NT>(rv, VTs, G::KS, tid);
        __syncthreads();
        i32x4 vb[CPW][NKS_K];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks)
                vb[c][ks] = *reinterpret_cast<const i32x4*>(VTs + ((wave + c * NW) * 16 + l16) * G::KS + ks * 64 + g * 16);
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) {
            const bool own_z = p.z != nullptr && (ab % NW == wave);
            int part = 0;
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks) {
                const i32x4 a = *reinterpret_cast<const i32x4*>(KTs + (ab * 16 + l16) * G::KS + ks * 64 + g * 16);
#pragma unroll
                for (int c = 0; c < CPW; ++c) P[c][ab] = mfma_i8(a, vb[c][ks], P[c][ab]);
                if (own_z) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int wd = a[e];
                        part += (int)(signed char)(wd & 0xFF) + (int)(signed char)((wd >> 8) & 0xFF) +
                                (int)(signed char)((wd >> 16) & 0xFF) + (int)(signed char)((wd >> 24) & 0xFF);
                    }
                }
            }
            if (own_z) {
                part += __shfl_xor(part, 16);
                part += __shfl_xor(part, 32);
                zacc[ab] += part;
            }
        }
    }

    int* S = p.S + ((bh * p.n_out + n) * p.dk_g) * (int64_t)p.dv;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int j = col0 + (wave + c * NW) * 16 + l16;
        if (j < p.dv) {
#pragma unroll
            for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int a = ab * 16 + g * 4 + i;
                    if (a < p.dk_g) S[(int64_t)a * p.dv + j] = P[c][ab][i];
                }
        }
    }
    if (p.z != nullptr && jt == 0) {
        int* z = p.z + (bh * p.n_out + n) * p.dk_g;
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) {
            const int a = ab * 16 + l16;
            if (ab % NW == wave && g == 0 && a < p.dk_g) z[a] = zacc[ab];
        }
    }
}

template <int DK, int DVT, int T>
hipError_t launch_fwd_i8(const FwdParamsI8& p, int64_t grid, hipStream_t s) {
    constexpr int NW = DVT / 16 < 4 ? DVT / 16 : 4;
    hipLaunchKernelGGL((chunked_fwd_i8<DK, DVT, T, NW>), dim3((unsigned)grid), dim3(NW * WAVE), 0, s, p);
    return hipGetLastError();
}

template <int DK, int DVT>
hipError_t launch_states_i8(const StatesParamsI8& p, int64_t grid, hipStream_t s) {
    constexpr int NW = DVT / 16 < 4 ? DVT / 16 : 4;
    hipLaunchKernelGGL((chunk_states_i8<DK, DVT, NW>), dim3((unsigned)grid), dim3(NW * WAVE), 0, s, p);
    return hipGetLastError();
}

}  // namespace la
