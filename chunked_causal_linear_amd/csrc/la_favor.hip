// FAVOR+ mapped inside the kernels (page "Linear Attention / Performerの理論と
// 実装", the positive random features: phi(x)_a = exp(w_a . x - |x|^2 / 2) /
// sqrt(m) for the m rows w_a of W, applied to queries and keys; the normalised
// causal output and the RNN view's state and normaliser).  Raw 64-wide q and k
// tiles are mapped on the matrix cores as they arrive, with W resident in LDS,
// so the m-wide phi(q) and phi(k) never go through memory.
//
// Mapping (both kernels): for a tile of 64 rows, wave w takes one block of 16
// rows and a range of feature blocks; W rows are the A operand and x rows the
// B operand of 16x16x32 bf16 products over the 64 input features, so a lane
// ends with four consecutive features a = 16 fb + 4 g + e of its row
// r = 16 rb + l16, and phi = exp2(log2(e) s proj - log2(e) s^2 |x_r|^2 / 2 -
// log2(m) / 2) (s = in_scale) is one fused multiply-add and one exp2 per
// feature, packed to bf16 and written as 8 bytes.  Key rows past the end of the
// sequence are mapped to zero.
//
//  * favor_states_kernel: phase 1, the state of a run of rows,
//    S = phi(K)^T V and z = sum of phi(K) rows, with phi(k) carried as a bf16
//    pair hi = bf16(phi), lo = bf16(phi - hi) (about 2^-17 relative), both
//    multiplied: the long sums do not collect the bf16 rounding of phi.
//  * favor_fwd_kernel: phase 3, the chunks (of 64 rows) of a group from its
//    prefix state: O = phi(Q) P + tril(phi(Q) phi(K)^T) V, normalised by
//    phi(Q) z + the row sums of tril(phi(Q) phi(K)^T), then P += phi(K)^T V,
//    z += the column sums of phi(K).
//
// Eight waves, two per SIMD: state waves 0-3 own 16 value columns of the
// m x 64 state each (fp32 accumulators, the layout of the other streaming
// kernels: a packed pair is an operand in feature order); prep waves 4-7 issue
// the direct-to-LDS copies of the raw tiles and the output stores and keep the
// normaliser.  All eight waves map.
#include "la_fwd_pipe.hpp"

namespace la {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// one 64-row raw tile: q (phase 3 only), k, v (64 value columns), 16-byte
// segments XOR-swizzled by row
struct alignas(16) RawStage {
    u16 q[64 * 64];
    u16 k[64 * 64];
    u16 v[64 * 64];
};
struct alignas(16) RawStageKV {
    u16 k[64 * 64];
    u16 v[64 * 64];
};

// phi of one 16-row block of a raw 64-wide tile for feature blocks FB0 .. FB0 + NFB - 1
// into a [64 x M] bf16 tile (hi, and the residual lo when lo != nullptr);
// rows at or past `valid` map to zero when zero_tail
template <int M, int NFB>
__device__ __forceinline__ void map_rows(const u16* W, const u16* x, int rb, int fb0, float s, bool zero_tail,
                                         int valid, u16* hi, u16* lo, int lane) {
    using namespace pipe;
    constexpr int FSEG = M / 8;
    const int l16 = lane % 16, g = lane / 16;
    const int r = 16 * rb + l16;
    // |x_r|^2 (the four lane groups compute the same row)
    float xx = 0.f;
#pragma unroll
    for (int seg = 0; seg < 8; ++seg) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + tile_off<8>(r, seg * 8));
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = __uint_as_float(w4[j] << 16), b = __uint_as_float(w4[j] & 0xFFFF0000u);
            xx = fmaf(a, a, fmaf(b, b, xx));
        }
    }
    const float c1 = kLog2e * s;
    const float c0 = -0.5f * kLog2e * s * s * xx - 0.5f * __builtin_amdgcn_logf((float)M);
    const bool dead = zero_tail && r >= valid;
    const bf16x8 xb0 = row_op<8>(x, r, 0, g), xb1 = row_op<8>(x, r, 32, g);
#pragma unroll 4
    for (int f = 0; f < NFB; ++f) {
        const int fb = fb0 + f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_bf16(row_op<8>(W, 16 * fb + l16, 0, g), xb0, acc);
        acc = mfma_bf16(row_op<8>(W, 16 * fb + l16, 32, g), xb1, acc);
        float ph[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ph[e] = dead ? 0.f : __builtin_amdgcn_exp2f(fmaf(c1, acc[e], c0));
        const uint32_t h0 = pack2_bf16(ph[0], ph[1]), h1 = pack2_bf16(ph[2], ph[3]);
        const int off = tile_off<FSEG>(r, 16 * fb + 4 * g);
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(hi) + off) = make_uint2(h0, h1);
        if (lo != nullptr) {
            const uint32_t l0 = pack2_bf16(ph[0] - __uint_as_float(h0 << 16), ph[1] - __uint_as_float(h0 & 0xFFFF0000u));
            const uint32_t l1 = pack2_bf16(ph[2] - __uint_as_float(h1 << 16), ph[3] - __uint_as_float(h1 & 0xFFFF0000u));
            *reinterpret_cast<uint2*>(reinterpret_cast<char*>(lo) + off) = make_uint2(l0, l1);
        }
    }
}

// W [M x 64] bf16 into LDS (row-major, swizzled), by all threads of the workgroup
template <int M>
__device__ __forceinline__ void load_W(const u16* Wg, u16* Wl, int tid, int nthreads) {
    using namespace pipe;
    for (int i = tid; i < M * 8; i += nthreads) {
        const int r = i / 8, seg = i % 8;
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Wl) + tile_off<8>(r, seg * 8)) =
            *reinterpret_cast<const uint4*>(Wg + r * 64 + seg * 8);
    }
}

// direct-to-LDS copy of this prep wave's share (two instructions) of one
// 64 x 64 bf16 tile of rows r0 .. r0 + 63 (clamped to `last`) with row stride
// `stride` (elements)
__device__ __forceinline__ void copy_tile(const u16* base, int stride, int last, u16* dst, int pw, int lane) {
    using namespace pipe;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int b = pw * 2 + i, slot = b * WAVE + lane;
        const int r = slot / 8, seg = (slot % 8) ^ (r & 7);
        dma16(base, (uint32_t)(((r < last ? r : last) * stride + seg * 8) * 2), lds_addr(dst) + b * WAVE * 16);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// phase 1: one workgroup per (head, run of rows, 64 value columns)
// ---------------------------------------------------------------------------
template <int M, bool Z>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void favor_states_kernel(FavorParams p) {
    using namespace pipe;
    constexpr int FSEG = M / 8, NKS = M / 32;
    constexpr int FIXED = M * 64 * 2 + 2 * 64 * M * 2;  // W, hi, lo
    constexpr int NFIT = (int)((160 * 1024 - FIXED) / sizeof(RawStageKV));
    constexpr int NSTAGE = NFIT < 4 ? NFIT : 4;
    constexpr int NL = 4;  // copy instructions per tile and prep wave
    static_assert(NSTAGE >= 2, "stages");

    __shared__ __attribute__((aligned(16))) u16 Wl[M * 64];
    __shared__ RawStageKV st[NSTAGE];
    __shared__ __attribute__((aligned(16))) u16 hi[64 * M];
    __shared__ __attribute__((aligned(16))) u16 lo[64 * M];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const bool prep = wave >= 4;
    const int pw = wave & 3;
    const int lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int wi = work_index(p.xcd_remap);
    const int jt = wi % p.n_dvt;
    const int64_t n = (wi / p.n_dvt) % p.n_groups;
    const int64_t bh = wi / ((int64_t)p.n_dvt * p.n_groups);
    const int col0 = jt * 64, cw = 16 * pw;
    const int64_t L = p.L;
    const int dv = p.dv;
    const int64_t r_begin = n * p.rows;
    const int64_t r_end = r_begin + p.rows < L ? r_begin + p.rows : L;
    const int64_t t_begin = r_begin / 64, t_end = (r_end + 63) / 64;
    auto valid_of = [&](int64_t t) -> int { return (int)(L - t * 64 < 64 ? L - t * 64 : 64); };
    const u16* kh = p.k + bh * L * 64;
    const u16* vh = p.v + bh * L * dv + col0;
    auto issue = [&](int64_t t, RawStageKV& s) __attribute__((always_inline)) {
        const int last = (int)(L - 1 - t * 64);
        copy_tile(kh + t * 64 * 64, 64, last, s.k, pw, lane);
        copy_tile(vh + t * 64 * dv, dv, last, s.v, pw, lane);
    };
    auto land = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t newest = t + NSTAGE - 2 < t_end - 1 ? t + NSTAGE - 2 : t_end - 1;
        const int after = (int)(newest - t);
        if constexpr (NSTAGE >= 4)
            if (after >= 2) {
                wait_vm<2 * NL>();
                return;
            }
        if constexpr (NSTAGE >= 3)
            if (after >= 1) {
                wait_vm<NL>();
                return;
            }
        wait_vm<0>();
    };

    if (prep)
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (t_begin + s0 < t_end) issue(t_begin + s0, st[s0]);
    load_W<M>(p.W, Wl, tid, 8 * WAVE);
    if (prep) land(t_begin);

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 P[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) P[ks][0] = P[ks][1] = zero4;
    float zacc = 0.f;  // prep waves: z of feature 64 pw + lane
    const int c4 = 4 * (lane & 3), c8 = 8 * (lane & 3);

    int si = 0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        RawStageKV& s = st[si];
        const int sp = si == 0 ? NSTAGE - 1 : si - 1;
        __syncthreads();  // B1(t): tile t is in; the products of tile t - 1 are done
        if (prep && t + NSTAGE - 1 < t_end) issue(t + NSTAGE - 1, st[sp]);
        // every wave maps one 16-row block, half of the feature blocks
        map_rows<M, M / 32>(Wl, s.k, wave & 3, (wave >> 2) * (M / 32), p.in_scale, true, valid_of(t), hi, lo, lane);
        __syncthreads();  // B2(t): hi and lo of tile t are complete
        if (!prep) {
            bf16x8 vb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) vb[kk] = col_op<8>(s.v, 32 * kk, cw + c4, lane);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        P[ks][hf] = mfma_bf16(col_op<FSEG>(hi, 32 * kk, 32 * ks + c8 + 4 * hf, lane), vb[kk], P[ks][hf]);
                        P[ks][hf] = mfma_bf16(col_op<FSEG>(lo, 32 * kk, 32 * ks + c8 + 4 * hf, lane), vb[kk], P[ks][hf]);
                    }
        } else {
            if (Z && 64 * pw < M) {
                const int a = 64 * pw + lane;
                float acc = 0.f;
#pragma unroll 8
                for (int r = 0; r < 64; ++r) {
                    const int off = tile_off<FSEG>(r, a);
                    acc += bf2f(*reinterpret_cast<const u16*>(reinterpret_cast<const char*>(hi) + off)) +
                           bf2f(*reinterpret_cast<const u16*>(reinterpret_cast<const char*>(lo) + off));
                }
                zacc += acc;
            }
            if (t + 1 < t_end) land(t + 1);
        }
        si = si == NSTAGE - 1 ? 0 : si + 1;
    }
    if (!prep) {
        float* S = p.S + ((bh * p.n_out + n) * M) * (int64_t)dv + col0 + cw + l16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[(int64_t)(32 * ks + 8 * g + 4 * hf + e) * dv] = P[ks][hf][e];
    } else if (Z && jt == 0 && 64 * pw < M) {
        p.z[(bh * p.n_out + n) * M + 64 * pw + lane] = zacc;
    }
}

// ---------------------------------------------------------------------------
// phase 3: one workgroup per (head, group of chunks of 64, 64 value columns)
// ---------------------------------------------------------------------------
// Three barriers per chunk t:
//   B1(t): tile t is in; the state waves are done with chunk t - 1 (its output
//          rows are in its stage's V columns; phi(q), phi(k) and the score tile
//          are free); the prep waves have added chunk t - 1 to z;
//   B2(t): phi(q) and phi(k) of tile t are complete (all eight waves map);
//   B3(t): the score tile (tril(phi(Q) phi(K)^T), columns in operand key
//          order) is complete and, with the normaliser, both parts of each
//          row's denominator: phi(q_i) . z and sum_{j <= i} S_ij.
// Right after B1(t) the prep waves store chunk t - 1's outputs and issue tile
// t + 1 into the stage they leave.  After B3 the state waves form the outputs
// and update their state while the prep waves add the chunk's keys to z and
// wait for tile t + 1.
template <int M, bool NORM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void favor_fwd_kernel(FavorParams p) {
    using namespace pipe;
    constexpr int FSEG = M / 8, NKS = M / 32;

    __shared__ __attribute__((aligned(16))) u16 Wl[M * 64];
    __shared__ RawStage st[2];
    __shared__ __attribute__((aligned(16))) u16 fq[64 * M];
    __shared__ __attribute__((aligned(16))) u16 fk[64 * M];
    __shared__ __attribute__((aligned(16))) u16 stile[64 * 64];
    __shared__ __attribute__((aligned(16))) float zl[NORM ? M : 4];
    __shared__ __attribute__((aligned(16))) float rowsum[64];
    __shared__ __attribute__((aligned(16))) float qz[64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const bool prep = wave >= 4;
    const int pw = wave & 3;
    const int lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int wi = work_index(p.xcd_remap);
    const int jt = wi % p.n_dvt;
    const int grp = (wi / p.n_dvt) % p.n_groups;
    const int64_t bh = wi / ((int64_t)p.n_dvt * p.n_groups);
    const int col0 = jt * 64, cw = 16 * pw;
    const int64_t L = p.L;
    const int dv = p.dv;
    const int64_t n_tiles = (L + 63) / 64;
    const int64_t t_begin = (int64_t)grp * p.G;
    const int64_t t_end = t_begin + p.G < n_tiles ? t_begin + p.G : n_tiles;
    auto valid_of = [&](int64_t t) -> int { return (int)(L - t * 64 < 64 ? L - t * 64 : 64); };
    const u16* qh = p.q + bh * L * 64;
    const u16* kh = p.k + bh * L * 64;
    const u16* vh = p.v + bh * L * dv + col0;
    const int64_t slot = (bh * p.n_groups + grp) * (int64_t)(p.p0_sub > 1 ? p.p0_sub : 1);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    auto issue = [&](int64_t t, RawStage& s) __attribute__((always_inline)) {
        const int last = (int)(L - 1 - t * 64);
        copy_tile(qh + t * 64 * 64, 64, last, s.q, pw, lane);
        copy_tile(kh + t * 64 * 64, 64, last, s.k, pw, lane);
        copy_tile(vh + t * 64 * dv, dv, last, s.v, pw, lane);
    };
    // output rows from the V tile of a stage: piece (pw * 2 + i) * 64 + lane
    auto read_out = [&](const RawStage& s, u32x4 (&ob)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = (pw * 2 + i) * WAVE + lane, r = piece / 8, seg = piece % 8;
            ob[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(s.v) + tile_off<8>(r, seg * 8));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage may be refilled
    };
    auto store_out = [&](int64_t t, const u32x4 (&ob)[2]) __attribute__((always_inline)) {
        const int valid = valid_of(t);
        u16* o = p.o + (bh * L + t * 64) * dv + col0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = (pw * 2 + i) * WAVE + lane, r = piece / 8, seg = piece % 8;
            if (r < valid) __builtin_nontemporal_store(ob[i], reinterpret_cast<u32x4*>(o + (int64_t)r * dv + seg * 8));
        }
    };

    // prologue: the first tile, W, the group's prefix state and normaliser
    if (prep) issue(t_begin, st[0]);
    load_W<M>(p.W, Wl, tid, 8 * WAVE);
    f32x4 P[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) P[ks][0] = P[ks][1] = zero4;
    if (!prep) {
        if (p.P0 != nullptr && grp > 0) {
            const float* P0 = p.P0 + (slot * M) * (int64_t)dv + col0 + cw + l16;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e) P[ks][hf][e] = P0[(int64_t)(32 * ks + 8 * g + 4 * hf + e) * dv];
        }
    } else if (NORM && 64 * pw < M) {
        zl[64 * pw + lane] = (p.z0 != nullptr && grp > 0) ? p.z0[slot * M + 64 * pw + lane] : 0.f;
    }
    if (prep) wait_vm<0>();

    int si = 0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        RawStage& s = st[si];
        RawStage& sn = st[si ^ 1];
        const int valid = valid_of(t);
        // the lane's values formed again each chunk (opaque to the compiler), so
        // that the LDS addresses derived from them are not all held in registers
        // across the chunk loop
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int l16 = lane_o % 16, g = lane_o / 16, c4 = 4 * (lane_o & 3), c8 = 8 * (lane_o & 3);
        __syncthreads();  // B1(t)
        if (prep) {
            // chunk t - 1's outputs leave the other stage (stored first, so that
            // the stores drain during the chunk), which then takes tile t + 1
            if (t > t_begin) {
                u32x4 ob[2];
                read_out(sn, ob);
                store_out(t - 1, ob);
            }
            if (t + 1 < t_end) issue(t + 1, sn);
            if (NORM && pw == 0) rowsum[lane] = 0.f;
        }
        // phi(q) (waves 0-3) and phi(k) (waves 4-7), one 16-row block each
        map_rows<M, M / 16>(Wl, prep ? s.k : s.q, pw, 0, p.in_scale, prep, valid, prep ? fk : fq, nullptr, lane_o);
        __syncthreads();  // B2(t)
        // score blocks (ib, jb), jb <= ib (b = 0..9), and the two blocks above the
        // diagonal the 32-key operand reads also cover, (0, 1) and (2, 3)
        // (b = 10, 11), as zeros: wave w takes b = w and, for w < 4, b = w + 8
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int b = wave + 8 * pass;
            if (b < 12) {
                if (b >= 10) {
                    const int ib = b == 10 ? 0 : 2;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<u16*>(reinterpret_cast<char*>(stile) +
                                                tile_off<8>(16 * ib + 4 * g + e, perm_pos(16 * (ib + 1) + l16))) = 0;
                } else {
                    const int ib = b < 1 ? 0 : (b < 3 ? 1 : (b < 6 ? 2 : 3));
                    const int jb = b - ib * (ib + 1) / 2;
                    f32x4 acc = zero4;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        acc = mfma_bf16(row_op<FSEG>(fq, 16 * ib + l16, 32 * ks, g),
                                        row_op<FSEG>(fk, 16 * jb + l16, 32 * ks, g), acc);
                    const int j = 16 * jb + l16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * ib + 4 * g + e;
                        const float sv = j <= i ? acc[e] : 0.f;
                        *reinterpret_cast<u16*>(reinterpret_cast<char*>(stile) + tile_off<8>(i, perm_pos(j))) = f2bf(sv);
                        if constexpr (NORM) {
                            // the row's partial sum over this block's 16 keys
                            float rs = sv;
                            rs += __shfl_xor(rs, 1);
                            rs += __shfl_xor(rs, 2);
                            rs += __shfl_xor(rs, 4);
                            rs += __shfl_xor(rs, 8);
                            if (l16 == 0) atomicAdd(&rowsum[i], rs);
                        }
                    }
                }
            }
        }
        if (NORM && prep) {
            // phi(q_i) . z for row i = 16 pw + l16, the four lane groups a quarter of the features each
            const int i = 16 * pw + l16;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < M / 32; ++c) {
                const int a0 = g * (M / 4) + 8 * c;
                const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(fq) + tile_off<FSEG>(i, a0));
                const float4 z0 = *reinterpret_cast<const float4*>(zl + a0);
                const float4 z1 = *reinterpret_cast<const float4*>(zl + a0 + 4);
                acc = fmaf(__uint_as_float(u.x << 16), z0.x, acc);
                acc = fmaf(__uint_as_float(u.x & 0xFFFF0000u), z0.y, acc);
                acc = fmaf(__uint_as_float(u.y << 16), z0.z, acc);
                acc = fmaf(__uint_as_float(u.y & 0xFFFF0000u), z0.w, acc);
                acc = fmaf(__uint_as_float(u.z << 16), z1.x, acc);
                acc = fmaf(__uint_as_float(u.z & 0xFFFF0000u), z1.y, acc);
                acc = fmaf(__uint_as_float(u.w << 16), z1.z, acc);
                acc = fmaf(__uint_as_float(u.w & 0xFFFF0000u), z1.w, acc);
            }
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            if (g == 0) qz[i] = acc;
        }
        __syncthreads();  // B3(t)
        if (!prep) {
            // inter phi(Q) P and intra tril(S) V: lane holds row 16 ib + 4g + e, column cw + l16
            f32x4 O[4];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) O[ib] = zero4;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 pk = pack_acc_bf16(P[ks][0], P[ks][1]);
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) O[ib] = mfma_bf16(row_op<FSEG>(fq, 16 * ib + l16, 32 * ks, g), pk, O[ib]);
                __builtin_amdgcn_sched_barrier(0);
            }
            bf16x8 vb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) vb[kk] = col_op<8>(s.v, 32 * kk, cw + c4, lane_o);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                for (int kk = 0; kk <= ib / 2; ++kk) O[ib] = mfma_bf16(row_op<8>(stile, 16 * ib + l16, 32 * kk, g), vb[kk], O[ib]);
            // the output rows (normalised) into this wave's own V columns
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                float rden[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (NORM) {
                    const float4 q4 = *reinterpret_cast<const float4*>(qz + 16 * ib + 4 * g);
                    const float4 r4 = *reinterpret_cast<const float4*>(rowsum + 16 * ib + 4 * g);
                    rden[0] = __builtin_amdgcn_rcpf(q4.x + r4.x);
                    rden[1] = __builtin_amdgcn_rcpf(q4.y + r4.y);
                    rden[2] = __builtin_amdgcn_rcpf(q4.z + r4.z);
                    rden[3] = __builtin_amdgcn_rcpf(q4.w + r4.w);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<u16*>(reinterpret_cast<char*>(s.v) + tile_off<8>(16 * ib + 4 * g + e, cw + l16)) =
                        f2bf(O[ib][e] * rden[e]);
            }
            // P += phi(K)^T V
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        P[ks][hf] = mfma_bf16(col_op<FSEG>(fk, 32 * kk, 32 * ks + c8 + 4 * hf, lane_o), vb[kk], P[ks][hf]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            if (NORM && 64 * pw < M) {
                // z += the column sums of phi(K) (rows past the end are zero)
                const int a = 64 * pw + lane;
                float acc = 0.f;
#pragma unroll 8
                for (int r = 0; r < 64; ++r)
                    acc += bf2f(*reinterpret_cast<const u16*>(reinterpret_cast<const char*>(fk) + tile_off<FSEG>(r, a)));
                zl[a] += acc;
            }
            if (t + 1 < t_end) wait_vm<0>();  // tile t + 1 (and chunk t - 1's stores) are done
        }
        si ^= 1;
    }
    __syncthreads();  // B1(t_end): the last chunk's outputs are in its stage
    if (prep) {
        u32x4 ob[2];
        read_out(st[si ^ 1], ob);
        store_out(t_end - 1, ob);
    }
}

// ---------------------------------------------------------------------------
template <int M>
static void launch_states(const FavorParams& p, int norm, int64_t grid, hipStream_t s) {
    if (norm)
        hipLaunchKernelGGL((favor_states_kernel<M, true>), dim3((unsigned)grid), dim3(512), 0, s, p);
    else
        hipLaunchKernelGGL((favor_states_kernel<M, false>), dim3((unsigned)grid), dim3(512), 0, s, p);
}

template <int M>
static void launch_fwd(const FavorParams& p, int norm, int64_t grid, hipStream_t s) {
    if (norm)
        hipLaunchKernelGGL((favor_fwd_kernel<M, true>), dim3((unsigned)grid), dim3(512), 0, s, p);
    else
        hipLaunchKernelGGL((favor_fwd_kernel<M, false>), dim3((unsigned)grid), dim3(512), 0, s, p);
}

hipError_t run_favor_states(const FavorParams& p, int m, int norm, int64_t grid, hipStream_t s) {
    switch (m) {
        case 64: launch_states<64>(p, norm, grid, s); break;
        case 128: launch_states<128>(p, norm, grid, s); break;
        case 256: launch_states<256>(p, norm, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t run_favor_fwd(const FavorParams& p, int m, int norm, int64_t grid, hipStream_t s) {
    switch (m) {
        case 64: launch_fwd<64>(p, norm, grid, s); break;
        case 128: launch_fwd<128>(p, norm, grid, s); break;
        case 256: launch_fwd<256>(p, norm, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace la
