// Chunkwise causal linear attention on bf16 matrix cores (gfx950).
//
// Two kernels share the tile loaders and the state-update code:
//
//  * chunk_states_bf16 - phase 1: S_n = phi(K_c)^T V_c (+ z_n = column sums of
//    phi(K_c)) for every chunk of C rows (page "attention と線形の間",
//    section ②: the state a chunk adds for the chunks after it).
//
//  * chunked_fwd_bf16 - phase 3 fused with the carry: one workgroup walks G
//    consecutive chunks of one (batch*head) slice and one tile of DVT output
//    columns.  It starts from the prefix state of its group (phase 2's
//    exclusive scan, or zero for the first group) and, per chunk,
//        O_c  = Q_c P + tril(Q_c K_c^T) V_c      (diagonal kept)
//        den  = Q_c z + row sums of tril(Q_c K_c^T)   (normalised variant)
//        P   += K_c^T V_c ;  z += column sums of K_c
//    which is the chunked algorithm of the same section, with the normaliser of
//    the page "Linear Attention / Performerの理論と実装" (RNN view: numerator
//    and denominator each sum their parts before the division).
//
// Tiles.  A chunk of C <= T rows is one tile of T rows (rows past the chunk are
// zero) and the next chunk's loads are in flight while it computes.  A chunk of
// C > T rows is walked in sub-tiles of T rows; the intra-chunk part of sub-tile
// t then also visits sub-tiles 0..t-1 of the same chunk (full blocks, no mask)
// and the state grows only at the chunk's end.
//
// Matrix-core mapping (16x16x32 bf16, fp32 accumulate; see la_common.hpp).
// Q, K and V sit in LDS row-major, exactly as loaded:
//   scores   S^T[key][q] = sum_a K[key][a] Q[q][a]     A = K rows, B = Q rows
//   intra    O[q][j]    += sum_key S[q][key] V[key][j]  A = S rows, B = V columns
//   inter    O[q][j]    += sum_a Q[q][a] P[a][j]        A = Q rows, B = P from registers
//   update   P[a][j]    += sum_key K[key][a] V[key][j]  A = K columns, B = V columns
// The column operands (fixed a or j, eight keys) come from gfx950's LDS
// transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4r + c supplies the address of four consecutive elements of row r, and lane
// n receives element n of each of the four rows.
//
// Inside each 32-wide k-step the reduction index is permuted the same way on
// both operands: lane group g holds the indices 4g..4g+3 and 16+4g..16+4g+3.
// That is where the P accumulators of a wave already hold their a's
// (lane: j = l%16, a = 16*ab + 4*(l/16) + i), so P feeds the inter product
// without leaving registers; the key operands follow the same order.  Wave w
// owns output column block(s) j of O and of P.
#pragma once

#include "la_common.hpp"
#include "la_kernels.hpp"

#ifndef LA_PREFETCH
#define LA_PREFETCH 1
#endif
#ifndef LA_WAVES_PER_EU
#define LA_WAVES_PER_EU 2
#endif

namespace la {

namespace detail {

// LDS geometry for one instantiation (strides in elements).
template <int DK, int DVT, int T>
struct Geo {
    static constexpr int TK = T < 32 ? 32 : T;  // key extent of the products (k-steps of 32)
    static constexpr int QS = DK + 16;          // row stride of the Q and K tiles
    static constexpr int VS = DVT + 16;         // row stride of the V tile
    static constexpr int KS = TK + 8;           // row stride of the score tile
    static constexpr int Q_ELEMS = TK * QS;
    static constexpr int V_ELEMS = TK * VS;
    static constexpr int S_ELEMS = T * KS;
};

struct Tile {
    int64_t row0;  // first global row of the tile
    int valid;     // rows [row0, row0 + valid) are real; the rest are zero
};

// ---------------------------------------------------------------------------
// Global -> register loads of 4x8 units, register -> LDS row stores.
// A unit is 4 rows x 8 columns; unit u covers column group u % (W/8) and row
// group u / (W/8), so consecutive lanes read consecutive 16-byte pieces of a row.
// ---------------------------------------------------------------------------
template <int R, int W, int NT>
struct Units {
    static constexpr int N = (R / 4) * (W / 8);
    static constexpr int PER_THREAD = (N + NT - 1) / NT;
};

// registers holding the units a thread loads for one tile
template <int R, int W, int NT>
struct URegs {
    uint4 r[Units<R, W, NT>::PER_THREAD][4];
};

template <int R, int W, int NT>
__device__ __forceinline__ void load_units(URegs<R, W, NT>& reg, const u16* __restrict__ base, int64_t row_stride,
                                           int col0, int cols_valid, const Tile& t, int tid) {
    constexpr int CG = W / 8;
    constexpr bool EVEN = Units<R, W, NT>::N % NT == 0;
    const u16* tb = base + t.row0 * row_stride + col0;
    if (EVEN && t.valid == R && cols_valid >= W) {
        // full tile: no per-row checks
#pragma unroll
        for (int it = 0; it < Units<R, W, NT>::PER_THREAD; ++it) {
            const int u = tid + it * NT;
            const int cg = u % CG, rg = u / CG;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                reg.r[it][i] = *reinterpret_cast<const uint4*>(tb + (int64_t)(rg * 4 + i) * row_stride + cg * 8);
        }
        return;
    }
#pragma unroll
    for (int it = 0; it < Units<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        const int cg = u % CG, rg = u / CG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rg * 4 + i;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (u < Units<R, W, NT>::N && r < t.valid && cg * 8 < cols_valid)
                val = *reinterpret_cast<const uint4*>(tb + (int64_t)r * row_stride + cg * 8);
            reg.r[it][i] = val;
        }
    }
}

// Apply elu+1 to the valid rows of loaded units (zero rows stay zero).
template <int R, int W, int NT>
__device__ __forceinline__ void phi_units(URegs<R, W, NT>& reg, int cols_valid, const Tile& t, int tid,
                                          float in_scale) {
    constexpr int CG = W / 8;
#pragma unroll
    for (int it = 0; it < Units<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        const int cg = u % CG, rg = u / CG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rg * 4 + i;
            if (u < Units<R, W, NT>::N && r < t.valid && cg * 8 < cols_valid)
                reg.r[it][i] = elu1_bf16x8(reg.r[it][i], in_scale);
        }
    }
}

// elu+1 split into bf16 hi/lo parts: reg becomes hi, lo receives the residual.
template <int R, int W, int NT>
__device__ __forceinline__ void phi_split_units(URegs<R, W, NT>& reg, URegs<R, W, NT>& lo, int cols_valid,
                                                const Tile& t, int tid, float in_scale) {
    constexpr int CG = W / 8;
#pragma unroll
    for (int it = 0; it < Units<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        const int cg = u % CG, rg = u / CG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rg * 4 + i;
            uint4 h = reg.r[it][i], l = make_uint4(0, 0, 0, 0);
            if (u < Units<R, W, NT>::N && r < t.valid && cg * 8 < cols_valid)
                elu1_split_bf16x8(reg.r[it][i], in_scale, h, l);
            reg.r[it][i] = h;
            lo.r[it][i] = l;
        }
    }
}

// Decayed recurrence: row r of a chunk ending at row e enters the chunk's
// state weighted gamma^(e-1-r).  The weight goes onto K (so the normaliser's
// column sums carry it too), computed in fp32 and rounded back to bf16; with
// the hi/lo split, w (hi + lo) is split again into a new hi/lo pair.
template <int R, int W, int NT, bool SPLIT>
__device__ __forceinline__ void decay_units(URegs<R, W, NT>& reg, URegs<R, W, NT>& lo, const Tile& t, int tid,
                                            int64_t e, float lg) {
    constexpr int CG = W / 8;
#pragma unroll
    for (int it = 0; it < Units<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        const int rg = u / CG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rg * 4 + i;
            const float w = (u < Units<R, W, NT>::N && r < t.valid)
                                ? __builtin_amdgcn_exp2f((float)(e - 1 - (t.row0 + r)) * lg)
                                : 0.f;
            const uint4 h = reg.r[it][i];
            const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
            uint32_t nh[4], nl[4];
            if constexpr (SPLIT) {
                const uint4 l = lo.r[it][i];
                const uint32_t lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = w * (__uint_as_float(hw[j] << 16) + __uint_as_float(lw[j] << 16));
                    const float b = w * (__uint_as_float(hw[j] & 0xFFFF0000u) + __uint_as_float(lw[j] & 0xFFFF0000u));
                    nh[j] = pack2_bf16(a, b);
                    nl[j] = pack2_bf16(a - __uint_as_float(nh[j] << 16), b - __uint_as_float(nh[j] & 0xFFFF0000u));
                }
                lo.r[it][i] = make_uint4(nl[0], nl[1], nl[2], nl[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    nh[j] = pack2_bf16(w * __uint_as_float(hw[j] << 16), w * __uint_as_float(hw[j] & 0xFFFF0000u));
            }
            reg.r[it][i] = make_uint4(nh[0], nh[1], nh[2], nh[3]);
        }
    }
}

__device__ __forceinline__ float sum_bf16x8(const uint4& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += bf2f((u16)(w[j] & 0xFFFF)) + bf2f((u16)(w[j] >> 16));
    return s;
}

// row-major store: dst[r * stride + 8*cg ..]
template <int R, int W, int NT>
__device__ __forceinline__ void store_rows(const URegs<R, W, NT>& reg, u16* dst, int stride, int tid) {
    constexpr int CG = W / 8;
#pragma unroll
    for (int it = 0; it < Units<R, W, NT>::PER_THREAD; ++it) {
        const int u = tid + it * NT;
        if (u < Units<R, W, NT>::N) {
            const int cg = u % CG, rg = u / CG;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(dst + (rg * 4 + i) * stride + cg * 8) = reg.r[it][i];
        }
    }
}

template <typename E>
__device__ __forceinline__ void zero_lds(E* p, int n, int tid, int nt) {
    for (int i = tid; i < n; i += nt) p[i] = E(0);
}

__device__ __forceinline__ float xor_sum_groups(float x) {
    // sum over the four 16-lane groups (lanes l, l^16, l^32, l^48)
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Column operand of a 32-key k-step: eight keys of one column of a row-major
// tile (rows = keys), in the permuted key order of the file header.  Lane
// (g = l/16, r = (l%16)/4, c = l%4) supplies rows key0 + 4g + r and
// key0 + 16 + 4g + r, columns col0 + 4c .. +3.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ uint2 lds_tr16(const u16* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p));
}

__device__ __forceinline__ uint4 column_operand(const u16* tile, int stride, int key0, int col0, int lane) {
    const int g = lane >> 4, r = (lane & 15) >> 2, c = lane & 3;
    const u16* ptr = tile + (key0 + 4 * g + r) * stride + col0 + 4 * c;
    const uint2 lo = lds_tr16(ptr);
    const uint2 hi = lds_tr16(ptr + 16 * stride);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Row operand in the permuted order: row[k0 + 4g .. +3] and row[k0 + 16 + 4g .. +3]
__device__ __forceinline__ uint4 row_operand_perm(const u16* row, int k0, int g) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + k0 + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + k0 + 16 + 4 * g);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// XCD-aware work index: workgroups are dispatched round-robin over the 8 XCDs;
// give each XCD a contiguous range of work items so that the column tiles of
// one head (consecutive items) share that XCD's L2.
__device__ __forceinline__ int work_index(int remap) {
    const int b = blockIdx.x;
    if (!remap) return b;
    const int per = gridDim.x >> 3;
    return (b & 7) * per + (b >> 3);
}

}  // namespace detail

using namespace detail;

// ===========================================================================
// Phase 3 (fused with the carry across the G chunks of a group)
// ===========================================================================
template <int DK, int DVT, int T, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * WAVE) __attribute__((amdgpu_waves_per_eu(SPLIT ? 1 : LA_WAVES_PER_EU, SPLIT ? 1 : LA_WAVES_PER_EU))) void chunked_fwd_bf16(FwdParams p) {
    using G = Geo<DK, DVT, T>;
    constexpr int NT = NW * WAVE;
    constexpr int NB = T / 16;             // 16-row blocks per tile
    constexpr int NAB = DK / 16;           // 16-row blocks of the state (a index)
    constexpr int NKS_A = DK / 32;         // k-steps over a
    constexpr int NKS_K = G::TK / 32;      // k-steps over keys
    constexpr int CB = DVT / 16;           // column blocks per workgroup
    constexpr int CPW = CB / NW;           // column blocks per wave
    static_assert(CPW * NW == CB, "column blocks must split evenly over waves");

    __shared__ __attribute__((aligned(16))) u16 Qs[G::Q_ELEMS];
    __shared__ __attribute__((aligned(16))) u16 Ks[G::Q_ELEMS];
    __shared__ __attribute__((aligned(16))) u16 KLs[SPLIT ? G::Q_ELEMS : 8];  // lo part of phi(K)
    __shared__ __attribute__((aligned(16))) u16 Vs[G::V_ELEMS];
    __shared__ __attribute__((aligned(16))) u16 Ss[G::S_ELEMS];
    __shared__ float zs[DK];
    __shared__ float dens[T];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;

    const int w = work_index(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int grp = (w / p.n_dvt) % p.n_groups;
    const int64_t bh = w / (p.n_dvt * p.n_groups);
    const int col0 = jt * DVT;

    const int64_t L = p.L;
    const int C = p.C;
    const int64_t n_chunks = (L + C - 1) / C;
    const int64_t c_begin = (int64_t)grp * p.G;
    const int64_t c_end = c_begin + p.G < n_chunks ? c_begin + p.G : n_chunks;

    const u16* __restrict__ qh = p.q + bh * L * p.dk_g;
    const u16* __restrict__ kh = p.k + bh * L * p.dk_g;
    const u16* __restrict__ vh = p.v + bh * L * p.dv;
    const u16* __restrict__ klh = p.k_lo != nullptr ? p.k_lo + bh * L * p.dk_g : nullptr;

    // rows past the tile (T < 32) and score blocks never written stay zero
    zero_lds(Qs, G::Q_ELEMS, tid, NT);
    zero_lds(Ks, G::Q_ELEMS, tid, NT);
    if (SPLIT) zero_lds(KLs, G::Q_ELEMS, tid, NT);
    zero_lds(Vs, G::V_ELEMS, tid, NT);
    zero_lds(Ss, G::S_ELEMS, tid, NT);

    // ---- state: P accumulators for this wave's column blocks, z for its a-blocks
    f32x4 P[CPW][NAB];
    float zacc[NAB];  // lane holds z[16*ab + l16] for ab = wave, wave + NW, ...
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) P[c][ab] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) zacc[ab] = 0.f;

    // prefix state of this group: phase 2's exclusive scan at group granularity
    // (causal, groups after the first) or the total state (non-causal)
    const int p0_sub = p.p0_sub > 1 ? p.p0_sub : 1;
    const int p0_groups = p.noncausal ? 1 : p.n_groups * p0_sub;
    const int p0_index = p.noncausal ? 0 : grp * p0_sub;
    if (p.P0 != nullptr && (grp > 0 || p.noncausal)) {
        const float* P0 = p.P0 + ((bh * p0_groups + p0_index) * p.dk_g) * (int64_t)p.dv;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int j = col0 + (wave + c * NW) * 16 + l16;
#pragma unroll
            for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int a = ab * 16 + g * 4 + i;
                    P[c][ab][i] = (a < p.dk_g) ? P0[(int64_t)a * p.dv + j] : 0.f;
                }
        }
        if (p.normalize) {
            const float* z0 = p.z0 + (bh * p0_groups + p0_index) * p.dk_g;
#pragma unroll
            for (int ab = 0; ab < NAB; ++ab) {
                const int a = ab * 16 + l16;
                if (ab % NW == wave) zacc[ab] = (a < p.dk_g) ? z0[a] : 0.f;
            }
        }
    }
    if (p.normalize) {
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab)
            if (ab % NW == wave && g == 0) zs[ab * 16 + l16] = zacc[ab];
    }

    URegs<T, DK, NT> rq, rk, rkl;
    URegs<T, DVT, NT> rv;

    auto tile_of = [&](int64_t chunk, int sub) -> Tile {
        const int64_t cs = chunk * C;
        const int64_t ce = cs + C < L ? cs + C : L;
        const int64_t r0 = cs + (int64_t)sub * T;
        const int64_t re = r0 + T < ce ? r0 + T : ce;
        return Tile{r0, (int)(re - r0)};
    };
    auto load_qkv = [&](const Tile& t) {
        load_units<T, DK, NT>(rq, qh, p.dk_g, 0, p.dk_g, t, tid);
        load_units<T, DK, NT>(rk, kh, p.dk_g, 0, p.dk_g, t, tid);
        if (SPLIT && klh != nullptr) load_units<T, DK, NT>(rkl, klh, p.dk_g, 0, p.dk_g, t, tid);
        load_units<T, DVT, NT>(rv, vh, p.dv, col0, p.dv - col0, t, tid);
    };
    auto write_qkv = [&](const Tile& t) {
        if (p.fmap == FMAP_ELU1) {
            phi_units<T, DK, NT>(rq, p.dk_g, t, tid, p.in_scale);
            if (SPLIT)
                phi_split_units<T, DK, NT>(rk, rkl, p.dk_g, t, tid, p.in_scale);
            else
                phi_units<T, DK, NT>(rk, p.dk_g, t, tid, p.in_scale);
        }
        store_rows<T, DK, NT>(rq, Qs, G::QS, tid);
        store_rows<T, DK, NT>(rk, Ks, G::QS, tid);
        if (SPLIT) store_rows<T, DK, NT>(rkl, KLs, G::QS, tid);
        store_rows<T, DVT, NT>(rv, Vs, G::VS, tid);
    };

    // scores for blocks (qb, kb): diagonal pass masks kb == qb and writes zeros
    // for kb > qb inside the k-steps the intra product reads.
    auto scores = [&](bool diagonal) {
        constexpr int NBLK = NB * NB;
        for (int blk = wave; blk < NBLK; blk += NW) {
            const int qb = blk / NB, kb = blk % NB;
            if (diagonal) {
                const int kb_lim = 2 * ((qb + 2) / 2);  // blocks covered by the k-steps
                if (kb >= kb_lim) continue;
                if (kb > qb) {
                    *reinterpret_cast<uint2*>(Ss + (qb * 16 + l16) * G::KS + kb * 16 + g * 4) = make_uint2(0, 0);
                    continue;
                }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS_A; ++ks) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + (kb * 16 + l16) * G::QS + ks * 32 + g * 8));
                const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(Qs + (qb * 16 + l16) * G::QS + ks * 32 + g * 8));
                acc = mfma_bf16(a, b, acc);
            }
            // acc[i] = S[q = 16qb + l16][key = 16kb + 4g + i]
            if (diagonal && kb == qb) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (g * 4 + i > l16) acc[i] = 0.f;
            }
            *reinterpret_cast<uint2*>(Ss + (qb * 16 + l16) * G::KS + kb * 16 + g * 4) =
                make_uint2(pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]));
        }
    };

    f32x4 O[CPW][NB];
    float den[NB];  // den partial for q = 16qb + l16 (blocks this wave owns)
    bf16x8 Pb[CPW][NKS_A];
    bf16x8 vb[CPW][NKS_K];

    // bf16 state snapshot for the inter product (the state at the chunk start)
    auto snapshot = [&]() {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKS_A; ++ks) Pb[c][ks] = pack_acc_bf16(P[c][2 * ks], P[c][2 * ks + 1]);
    };

    auto load_vb = [&]() {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks)
                vb[c][ks] = as_bf16x8(column_operand(Vs, G::VS, ks * 32, (wave + c * NW) * 16, lane));
    };

    // inter + diagonal intra products and the state update, for the tile in LDS.
    // With one tile per chunk (fresh == true) the inter product reads P before
    // this chunk's update, so it packs P on the fly instead of the snapshot.
    auto diag_products = [&](bool fresh) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            den[qb] = 0.f;
#pragma unroll
            for (int c = 0; c < CPW; ++c) O[c][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // inter: O = Q P  (k-steps over a outermost: one packed P operand per step)
#pragma unroll
        for (int ks = 0; ks < NKS_A; ++ks) {
            bf16x8 pb[CPW];
#pragma unroll
            for (int c = 0; c < CPW; ++c) pb[c] = fresh ? pack_acc_bf16(P[c][2 * ks], P[c][2 * ks + 1]) : Pb[c][ks];
#pragma unroll
            for (int qb = 0; qb < NB; ++qb) {
                const uint4 qa = row_operand_perm(Qs + (qb * 16 + l16) * G::QS, ks * 32, g);
#pragma unroll
                for (int c = 0; c < CPW; ++c) O[c][qb] = mfma_bf16(as_bf16x8(qa), pb[c], O[c][qb]);
                if (p.normalize && (qb % NW == wave)) {
                    // q . z over the eight a's this lane holds (a0 .. a0+3, a0+16 .. a0+19)
                    const int a0 = ks * 32 + g * 4;
                    const uint32_t qw[4] = {qa.x, qa.y, qa.z, qa.w};
                    float s = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int a = a0 + (j >> 1) * 16 + (j & 1) * 2;
                        s += bf2f((u16)(qw[j] & 0xFFFF)) * zs[a] + bf2f((u16)(qw[j] >> 16)) * zs[a + 1];
                    }
                    den[qb] += s;
                }
            }
        }
        load_vb();
        // intra: O += tril(S) V
        if (!p.noncausal) {
#pragma unroll
            for (int qb = 0; qb < NB; ++qb) {
                const bool own_den = p.normalize && (qb % NW == wave);
                const u16* srow = Ss + (qb * 16 + l16) * G::KS;
#pragma unroll
                for (int ks = 0; ks < (qb + 2) / 2; ++ks) {
                    const uint4 su = row_operand_perm(srow, ks * 32, g);
#pragma unroll
                    for (int c = 0; c < CPW; ++c) O[c][qb] = mfma_bf16(as_bf16x8(su), vb[c][ks], O[c][qb]);
                    if (own_den) den[qb] += sum_bf16x8(su);
                }
            }
        }
        // state update (the inter product of every sub-tile of a chunk reads the snapshot)
        if (!p.noncausal) {
#pragma unroll
            for (int ab = 0; ab < NAB; ++ab) {
                const bool own_z = p.normalize && (ab % NW == wave);
                float zs_part = 0.f;
#pragma unroll
                for (int ks = 0; ks < NKS_K; ++ks) {
                    const uint4 ku = column_operand(Ks, G::QS, ks * 32, ab * 16, lane);
#pragma unroll
                    for (int c = 0; c < CPW; ++c) P[c][ab] = mfma_bf16(as_bf16x8(ku), vb[c][ks], P[c][ab]);
                    if (own_z) zs_part += sum_bf16x8(ku);
                    if (SPLIT) {
                        const uint4 kl = column_operand(KLs, G::QS, ks * 32, ab * 16, lane);
#pragma unroll
                        for (int c = 0; c < CPW; ++c) P[c][ab] = mfma_bf16(as_bf16x8(kl), vb[c][ks], P[c][ab]);
                        if (own_z) zs_part += sum_bf16x8(kl);
                    }
                }
                if (own_z) zacc[ab] += xor_sum_groups(zs_part);
            }
        }
    };

    // intra products against an earlier sub-tile of the same chunk (C > T)
    auto prev_products = [&](const Tile& tp) {
        __syncthreads();  // Ks / Vs / Ss readers done
        load_units<T, DK, NT>(rk, kh, p.dk_g, 0, p.dk_g, tp, tid);
        load_units<T, DVT, NT>(rv, vh, p.dv, col0, p.dv - col0, tp, tid);
        if (p.fmap == FMAP_ELU1) phi_units<T, DK, NT>(rk, p.dk_g, tp, tid, p.in_scale);
        store_rows<T, DK, NT>(rk, Ks, G::QS, tid);
        store_rows<T, DVT, NT>(rv, Vs, G::VS, tid);
        __syncthreads();
        scores(false);
        __syncthreads();
        load_vb();
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            const bool own_den = p.normalize && (qb % NW == wave);
            const u16* srow = Ss + (qb * 16 + l16) * G::KS;
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks) {
                const uint4 su = row_operand_perm(srow, ks * 32, g);
#pragma unroll
                for (int c = 0; c < CPW; ++c) O[c][qb] = mfma_bf16(as_bf16x8(su), vb[c][ks], O[c][qb]);
                if (own_den) den[qb] += sum_bf16x8(su);
            }
        }
    };

    // denominators, then the output rows of the tile.  bf16 outputs are staged
    // through LDS (in the Q tile, free by now) so that every global store is a
    // full 16-byte row segment.
    constexpr int OS = DVT + 8;
    constexpr bool STAGE = DVT <= DK;
    auto finish_tile = [&](const Tile& t) {
        if (p.normalize) {
#pragma unroll
            for (int qb = 0; qb < NB; ++qb)
                if (qb % NW == wave) {
                    const float d = xor_sum_groups(den[qb]);
                    if (g == 0) dens[qb * 16 + l16] = 1.0f / d;
                }
        }
        __syncthreads();  // dens visible; every wave is done with Qs
        if (STAGE && !p.out_f32) {
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const int jl = (wave + c * NW) * 16 + l16;
                if (p.normalize) {
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = qb * 16 + g * 4 + i;
                            Qs[r * OS + jl] = f2bf(O[c][qb][i] * dens[r] * p.out_scale);
                        }
                } else {
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            Qs[(qb * 16 + g * 4 + i) * OS + jl] = f2bf(O[c][qb][i] * p.out_scale);
                }
            }
            __syncthreads();
            constexpr int SEGS = T * DVT / 8;
            u16* ob = reinterpret_cast<u16*>(p.o) + (bh * L + t.row0) * p.dv + col0;
#pragma unroll
            for (int it = 0; it < (SEGS + NT - 1) / NT; ++it) {
                const int sg = tid + it * NT;
                const int r = sg / (DVT / 8), c8 = sg % (DVT / 8);
                if ((SEGS % NT == 0 || sg < SEGS) && r < t.valid)
                    *reinterpret_cast<uint4*>(ob + (r * p.dv + c8 * 8)) =
                        *reinterpret_cast<const uint4*>(Qs + r * OS + c8 * 8);
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const int j = col0 + (wave + c * NW) * 16 + l16;
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = qb * 16 + g * 4 + i;
                        const float val = O[c][qb][i] * (p.normalize ? dens[r] : 1.0f) * p.out_scale;
                        if (r < t.valid && j < p.dv) {
                            const int64_t off = (bh * L + t.row0 + r) * p.dv + j;
                            if (p.out_f32)
                                reinterpret_cast<float*>(p.o)[off] = val;
                            else
                                reinterpret_cast<u16*>(p.o)[off] = f2bf(val);
                        }
                    }
            }
        }
    };

    auto publish_z = [&]() {
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab)
            if (ab % NW == wave && g == 0) zs[ab * 16 + l16] = zacc[ab];
    };

    if (C <= T) {
        // one tile per chunk: the next chunk's loads are in flight while this
        // chunk computes
        if (LA_PREFETCH && c_begin < c_end) load_qkv(tile_of(c_begin, 0));
        for (int64_t chunk = c_begin; chunk < c_end; ++chunk) {
            const Tile t = tile_of(chunk, 0);
            if (!LA_PREFETCH) load_qkv(t);
            __syncthreads();  // previous chunk's readers of the LDS tiles are done
            write_qkv(t);
            if (LA_PREFETCH && chunk + 1 < c_end) load_qkv(tile_of(chunk + 1, 0));
            __syncthreads();
            if (!p.noncausal) scores(true);
            __syncthreads();
            diag_products(true);
            finish_tile(t);  // its first barrier also ends every read of zs
            if (p.normalize) publish_z();
        }
    } else {
        for (int64_t chunk = c_begin; chunk < c_end; ++chunk) {
            const int64_t cs = chunk * C;
            const int64_t ce = cs + C < L ? cs + C : L;
            const int nsub = (int)((ce - cs + T - 1) / T);
            snapshot();
            for (int sub = 0; sub < nsub; ++sub) {
                const Tile t = tile_of(chunk, sub);
                load_qkv(t);
                __syncthreads();  // previous readers of the LDS tiles are done
                write_qkv(t);
                __syncthreads();
                scores(true);
                __syncthreads();
                diag_products(false);
                for (int prev = 0; prev < sub; ++prev) prev_products(tile_of(chunk, prev));
                finish_tile(t);
                if (sub + 1 < nsub) __syncthreads();  // staging reads done before the next tile's writes
            }
            if (p.normalize) publish_z();
        }
    }

    // final state: the group holding the last chunk (causal) or the first
    // group, which loaded the total state (non-causal)
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
                        if (a < p.dk_g) p.S_final[(bh * p.dk_g + a) * p.dv + j] = P[c][ab][i] * p.state_scale;
                    }
            }
        }
    }
    if (writes_final && p.z_final != nullptr && p.normalize && jt == 0) {
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) {
            const int a = ab * 16 + l16;
            if (ab % NW == wave && g == 0 && a < p.dk_g) p.z_final[bh * p.dk_g + a] = zacc[ab] * p.state_scale;
        }
    }
}

// ===========================================================================
// Phase 1: per-chunk states
// ===========================================================================
template <int DK, int DVT, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * WAVE) void chunk_states_bf16(StatesParams p) {
    constexpr int T = 64;
    using G = Geo<DK, DVT, T>;
    constexpr int NT = NW * WAVE;
    constexpr int NAB = DK / 16;
    constexpr int NKS_K = G::TK / 32;
    constexpr int CB = DVT / 16;
    constexpr int CPW = CB / NW;
    static_assert(CPW * NW == CB, "column blocks must split evenly over waves");

    __shared__ __attribute__((aligned(16))) u16 Ks[G::Q_ELEMS];
    __shared__ __attribute__((aligned(16))) u16 KLs[SPLIT ? G::Q_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) u16 Vs[G::V_ELEMS];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;

    const int w = work_index(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int64_t n = (w / p.n_dvt) % p.n_items;
    const int64_t bh = w / (p.n_dvt * p.n_items);
    const int col0 = jt * DVT;

    const int64_t L = p.L;
    const int64_t C = p.C;
    const int64_t cs = n * C;
    const int64_t ce = cs + C < L ? cs + C : L;

    const u16* __restrict__ kh = p.k + bh * L * p.dk_g;
    const u16* __restrict__ vh = p.v + bh * L * p.dv;
    const u16* __restrict__ klh = p.k_lo != nullptr ? p.k_lo + bh * L * p.dk_g : nullptr;

    f32x4 P[CPW][NAB];
    float zacc[NAB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) P[c][ab] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) zacc[ab] = 0.f;

    URegs<T, DK, NT> rk, rkl;
    URegs<T, DVT, NT> rv;

    for (int64_t r0 = cs; r0 < ce; r0 += T) {
        const Tile t{r0, (int)((ce - r0) < T ? (ce - r0) : T)};
        load_units<T, DK, NT>(rk, kh, p.dk_g, 0, p.dk_g, t, tid);
        if (SPLIT && klh != nullptr) load_units<T, DK, NT>(rkl, klh, p.dk_g, 0, p.dk_g, t, tid);
        load_units<T, DVT, NT>(rv, vh, p.dv, col0, p.dv - col0, t, tid);
        if (p.fmap == FMAP_ELU1) {
            if (SPLIT)
                phi_split_units<T, DK, NT>(rk, rkl, p.dk_g, t, tid, p.in_scale);
            else
                phi_units<T, DK, NT>(rk, p.dk_g, t, tid, p.in_scale);
        }
        if (p.log2_gamma != 0.0f) decay_units<T, DK, NT, SPLIT>(rk, rkl, t, tid, ce, p.log2_gamma);
        __syncthreads();
        store_rows<T, DK, NT>(rk, Ks, G::QS, tid);
        if (SPLIT) store_rows<T, DK, NT>(rkl, KLs, G::QS, tid);
        store_rows<T, DVT, NT>(rv, Vs, G::VS, tid);
        __syncthreads();
        bf16x8 vb[CPW][NKS_K];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks)
                vb[c][ks] = as_bf16x8(column_operand(Vs, G::VS, ks * 32, (wave + c * NW) * 16, lane));
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) {
            const bool own_z = p.want_z && (ab % NW == wave);
            float part = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS_K; ++ks) {
                const uint4 ku = column_operand(Ks, G::QS, ks * 32, ab * 16, lane);
#pragma unroll
                for (int c = 0; c < CPW; ++c) P[c][ab] = mfma_bf16(as_bf16x8(ku), vb[c][ks], P[c][ab]);
                if (own_z) part += sum_bf16x8(ku);
                if (SPLIT) {
                    const uint4 kl = column_operand(KLs, G::QS, ks * 32, ab * 16, lane);
#pragma unroll
                    for (int c = 0; c < CPW; ++c) P[c][ab] = mfma_bf16(as_bf16x8(kl), vb[c][ks], P[c][ab]);
                    if (own_z) part += sum_bf16x8(kl);
                }
            }
            if (own_z) zacc[ab] += xor_sum_groups(part);
        }
    }

    float* S = p.S + ((bh * p.n_out + n) * p.dk_g) * (int64_t)p.dv;
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
    if (p.want_z && jt == 0) {
        float* z = p.z + (bh * p.n_out + n) * p.dk_g;
#pragma unroll
        for (int ab = 0; ab < NAB; ++ab) {
            const int a = ab * 16 + l16;
            if (ab % NW == wave && g == 0 && a < p.dk_g) z[a] = zacc[ab];
        }
    }
}

// LDS bytes of one chunked_fwd_bf16 instantiation.
template <int DK, int DVT, int T, bool SPLIT>
constexpr int fwd_lds_bytes() {
    using G = Geo<DK, DVT, T>;
    return 2 * ((SPLIT ? 3 : 2) * G::Q_ELEMS + G::V_ELEMS + G::S_ELEMS) + 4 * (DK + T);
}

constexpr int LDS_LIMIT = 160 * 1024;

// The hi/lo split of phi(K) is compiled in when phi is applied in the kernel
// or arrives pre-mapped with its residual (instantiations whose LDS would not
// fit are rejected; the planner avoids them).
template <int DK, int DVT, int T>
hipError_t launch_fwd_bf16(const FwdParams& p, int64_t grid, hipStream_t s) {
    constexpr int NW = DVT / 16 < 4 ? DVT / 16 : 4;
    if ((p.fmap == FMAP_ELU1 || p.k_lo != nullptr) && !p.noncausal) {
        if constexpr (fwd_lds_bytes<DK, DVT, T, true>() <= LDS_LIMIT)
            hipLaunchKernelGGL((chunked_fwd_bf16<DK, DVT, T, NW, true>), dim3((unsigned)grid), dim3(NW * WAVE), 0, s, p);
        else
            return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((chunked_fwd_bf16<DK, DVT, T, NW, false>), dim3((unsigned)grid), dim3(NW * WAVE), 0, s, p);
    }
    return hipGetLastError();
}

template <int DK, int DVT>
hipError_t launch_states_bf16(const StatesParams& p, int64_t grid, hipStream_t s) {
    constexpr int NW = DVT / 16 < 4 ? DVT / 16 : 4;
    if (p.fmap == FMAP_ELU1 || p.k_lo != nullptr)
        hipLaunchKernelGGL((chunk_states_bf16<DK, DVT, NW, true>), dim3((unsigned)grid), dim3(NW * WAVE), 0, s, p);
    else
        hipLaunchKernelGGL((chunk_states_bf16<DK, DVT, NW, false>), dim3((unsigned)grid), dim3(NW * WAVE), 0, s, p);
    return hipGetLastError();
}

// Per-DK dispatchers, one translation unit each (la_bf16_dk*.hip).
hipError_t fwd_bf16_dk32(const FwdParams& p, int DVT, int T, int64_t grid, hipStream_t s);
hipError_t fwd_bf16_dk64(const FwdParams& p, int DVT, int T, int64_t grid, hipStream_t s);
hipError_t fwd_bf16_dk128(const FwdParams& p, int DVT, int T, int64_t grid, hipStream_t s);
hipError_t fwd_bf16_dk256(const FwdParams& p, int DVT, int T, int64_t grid, hipStream_t s);
hipError_t states_bf16_dk32(const StatesParams& p, int DVT, int64_t grid, hipStream_t s);
hipError_t states_bf16_dk64(const StatesParams& p, int DVT, int64_t grid, hipStream_t s);
hipError_t states_bf16_dk128(const StatesParams& p, int DVT, int64_t grid, hipStream_t s);
hipError_t states_bf16_dk256(const StatesParams& p, int DVT, int64_t grid, hipStream_t s);

}  // namespace la
