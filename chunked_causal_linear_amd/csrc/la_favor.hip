// FAVOR+ mapped inside the kernels (page "Linear Attention / Performerの理論と
// 実装", the positive random features: phi(x)_a = exp(w_a . x - |x|^2 / 2) /
// sqrt(m) for the m rows w_a of W, applied to queries and keys; the normalised
// causal output and the RNN view's state and normaliser).  Raw 64-wide q and k
// tiles are mapped on the matrix cores as they arrive; the m-wide phi(q) and
// phi(k) never go through memory.
//
// Mapping: W stays in registers.  A wave maps a fixed range of feature blocks
// (16 features each) for the rows it takes; for a 16-row block the product of
// its x rows with W rows over the 64 input features is two 16x16x32 bf16
// matrix-core steps, and each result element becomes
// phi = exp2(log2(e) s proj - log2(e) s^2 |x|^2 / 2 - log2(m) / 2) (s =
// in_scale): one fused multiply-add and one exp2.  The row norms come from the
// x fragments the products use (two lane exchanges).  Key rows past the end of
// the sequence map to zero.
//
//  * favor_states_kernel: phase 1, the state of a run of rows,
//    S = phi(K)^T V and z = the sum of the rows of phi(K).  Each wave owns
//    a range of features of S for all value columns of its tile: it maps
//    phi(k) with the features along the product's columns, so the results pack
//    straight into the update's operand (features by keys) in registers, and
//    sums z from the fp32 values.  phi(k) enters the update as a bf16 pair
//    hi = bf16(phi), lo = bf16(phi - hi) (about 2^-17 relative): the long sums
//    do not collect the bf16 rounding of phi.
//  * favor_fwd_kernel: phase 3, the chunks (of 64 rows) of a group from its
//    prefix state: O = phi(Q) P + tril(phi(Q) phi(K)^T) V, normalised by
//    phi(Q) z + the row sums of tril(phi(Q) phi(K)^T), then P += phi(K)^T V,
//    z += the column sums of phi(K).  Eight waves, two per SIMD: mapper
//    waves map phi(k) and phi(q) of the next chunk (a quarter of the features
//    each), while product waves run the current chunk, each with the state of
//    16 value columns over all features and z over a quarter of the features
//    in fp32 accumulators.
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

// W fragment of feature block fb: lane (g, l16) holds W[16 fb + l16][32 h + 8 g .. + 7]
// in wf[h] (the A operand with features as rows, the B operand with features as columns)
__device__ __forceinline__ void load_w_frag(const u16* W, int fb, int lane, bf16x8 (&wf)[2]) {
    const int l16 = lane % 16, g = lane / 16;
    const u16* row = W + (16 * fb + l16) * 64 + 8 * g;
    wf[0] = as_bf16x8(*reinterpret_cast<const uint4*>(row));
    wf[1] = as_bf16x8(*reinterpret_cast<const uint4*>(row + 32));
}

// sum of squares of the 16 bf16 values of two fragments
__device__ __forceinline__ float sumsq(const bf16x8& a, const bf16x8& b) {
    const uint4 u = __builtin_bit_cast(uint4, a), v = __builtin_bit_cast(uint4, b);
    const uint32_t w[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float lo = __uint_as_float(w[j] << 16), hi = __uint_as_float(w[j] & 0xFFFF0000u);
        s = fmaf(lo, lo, fmaf(hi, hi, s));
    }
    return s;
}

// |x_r|^2 for the row r = 16 rb + l16 whose fragments (x[r][8g .. 8g+7] and
// x[r][32 + 8g ..]) this lane holds: the four lane groups' partial sums added
__device__ __forceinline__ float row_norm(const bf16x8& a, const bf16x8& b) {
    float s = sumsq(a, b);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    return s;
}

__device__ __forceinline__ uint4 pack8(const float (&a)[4], const float (&b)[4]) {
    return make_uint4(pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]), pack2_bf16(b[0], b[1]), pack2_bf16(b[2], b[3]));
}
// the residuals x - bf16(x) of eight values packed by pack8
__device__ __forceinline__ uint4 pack8_lo(const float (&a)[4], const float (&b)[4], const uint4& h) {
    auto r2 = [](float x0, float x1, uint32_t hw) {
        return pack2_bf16(x0 - __uint_as_float(hw << 16), x1 - __uint_as_float(hw & 0xFFFF0000u));
    };
    return make_uint4(r2(a[0], a[1], h.x), r2(a[2], a[3], h.y), r2(b[0], b[1], h.z), r2(b[2], b[3], h.w));
}

// wait until at most `after` copy groups of N instructions each are in flight
template <int N, int MAXAFTER>
__device__ __forceinline__ void wait_groups(int after) {
    using pipe::wait_vm;
    if constexpr (MAXAFTER >= 4)
        if (after >= 4) {
            wait_vm<4 * N>();
            return;
        }
    if constexpr (MAXAFTER >= 3)
        if (after >= 3) {
            wait_vm<3 * N>();
            return;
        }
    if constexpr (MAXAFTER >= 2)
        if (after >= 2) {
            wait_vm<2 * N>();
            return;
        }
    if constexpr (MAXAFTER >= 1)
        if (after >= 1) {
            wait_vm<N>();
            return;
        }
    wait_vm<0>();
}

// The phi tiles' swizzle: the 16-byte segment index XOR a row key, the row
// itself (pipe::tile_off), or with SWAP the row with its two low bit pairs
// exchanged.  Measured on the LDS conflict counters at 16 and 32 segments per
// row: with the plain key the 16-byte row reads run conflict-free (4 LDS
// cycles each) and the transposed 8-byte column reads take 8; with the
// exchanged key the column reads take 4 and the row reads 8.  phi(k), read
// mostly by columns (the state update), takes the exchanged key there; phi(q)
// and every tile of 8 segments the plain one (both reads conflict-free).
template <bool SWAP>
__device__ __forceinline__ int row_key(int r) {
    return SWAP ? (((r & 3) << 2) | ((r >> 2) & 3) | (r & ~15)) : r;
}
template <int NSEG, bool SWAP>
__device__ __forceinline__ int phi_off(int r, int e) {
    return r * NSEG * 16 + ((((e >> 3) ^ row_key<SWAP>(r)) & (NSEG - 1)) << 4) + ((e & 7) << 1);
}

// Lane base addresses for the swizzled tiles.  For a 16-byte row read of row
// R0 + l16 at elements K0 + 8g .. (R0 a multiple of 16, K0 of 32) the segment
// index is ((4 ks + g) ^ key(R0 + l16)) mod NSEG with ks = K0 / 32: its low
// four bits depend on the lane and on ks mod 4 only, its higher bits on R0
// and ks only.  So four lane registers (one per ks mod 4) and a compile-time
// immediate give every such address, with no per-access arithmetic.
template <int NSEG, bool SWAP = false>
struct RowAddr {
    int b[4];
    __device__ __forceinline__ explicit RowAddr(int lane) {
        const int l16 = lane & 15, g = lane >> 4, B = g ^ row_key<SWAP>(l16);
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = l16 * NSEG * 16 + (((4 * c) ^ B) & (NSEG - 1)) * 16;
    }
    // byte offset of phi_off<NSEG, SWAP>(R0 + l16, K0 + 8g)
    __device__ __forceinline__ int off(int R0, int K0) const {
        const int ks = K0 / 32;
        return b[ks & 3] + R0 * NSEG * 16 + ((((4 * ks) ^ R0) & ~15) & (NSEG - 1)) * 16;
    }
};

// The same for the transposed 8-byte reads of a column operand: rows K0 + H +
// 4g + rr (K0 a multiple of 32, H 0 or 16, rr = (l % 16) / 4) at columns CB +
// 8c + 4hf (CB a multiple of 32, c = l % 4).
template <int NSEG, bool SWAP = false>
struct ColAddr {
    int b[4];
    __device__ __forceinline__ explicit ColAddr(int lane) {
        const int g = lane >> 4, rr = (lane & 15) >> 2, c = lane & 3, rl = 4 * g + rr, B = c ^ row_key<SWAP>(rl);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) b[cc] = rl * NSEG * 16 + (((4 * cc) ^ B) & (NSEG - 1)) * 16;
    }
    // byte offset of phi_off<NSEG, SWAP>(K0 + H + 4g + rr, CB + 8c + 4hf)
    __device__ __forceinline__ int off(int K0, int H, int CB, int hf) const {
        const int ks = CB / 32;
        return b[ks & 3] + (K0 + H) * NSEG * 16 + ((((4 * ks) ^ (K0 + H)) & ~15) & (NSEG - 1)) * 16 + 8 * hf;
    }
};

__device__ __forceinline__ bf16x8 row_at(const u16* tile, int off) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + off));
}
// the column operand (keys K0 .. K0 + 31 in operand order) from its two transposed reads
template <int NSEG, bool SWAP>
__device__ __forceinline__ bf16x8 col_at(const u16* tile, const ColAddr<NSEG, SWAP>& ca, int K0, int CB, int hf) {
    const char* t = reinterpret_cast<const char*>(tile);
    const uint2 lo = pipe::tr_read(t + ca.off(K0, 0, CB, hf));
    const uint2 hi = pipe::tr_read(t + ca.off(K0, 16, CB, hf));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Hands a value loaded before a loop to an empty asm statement: the compiler
// then waits for the load there, not at the first use inside the loop, where
// its memory-counter wait would also hold back the copies in flight.
template <typename T>
__device__ __forceinline__ void settle(T& v) {
    asm volatile("" : "+v"(v));
}

// the sum over the 16 lanes of a row of lanes: swaps within quads of lanes,
// then rotations of the row by 4 and by 8 (DPP)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x124>(v);  // row_ror 4
    v += dpp_f<0x128>(v);  // row_ror 8
    return v;
}

// Blocks (I0, J0), (I1, J1) and, when I2 >= 0, (I2, J2) of the score tile
// tril(phi(Q) phi(K)^T), computed transposed (lane (g, l16): keys 16 J + 4g + e
// of query row 16 I + l16) over all feature steps and stored, masked, in bf16
// into the score tile (columns in operand key order).  Blocks that share a
// query or key block read its fragments once.
template <int FSEG, int NKS, bool SWK, int I0, int J0, int I1, int J1, int I2, int J2>
__device__ __forceinline__ void score_blocks(const u16* q_, const u16* k_, u16* stile, const RowAddr<FSEG>& raq,
                                             const RowAddr<FSEG, SWK>& rak, int l16, int g) {
    using namespace pipe;
    constexpr int NB = I2 >= 0 ? 3 : 2;
    constexpr int I[3] = {I0, I1, I2 >= 0 ? I2 : 0}, J[3] = {J0, J1, I2 >= 0 ? J2 : 0};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[NB][2];  // two chains per block (even and odd feature steps)
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n][0] = acc[n][1] = zero4;
#pragma unroll
    for (int ks = 0; ks < NKS; ks += 2)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[n][h] = mfma_bf16(row_at(k_, rak.off(16 * J[n], 32 * (ks + h))),
                                      row_at(q_, raq.off(16 * I[n], 32 * (ks + h))), acc[n][h]);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const f32x4 s = acc[n][0] + acc[n][1];
        const int i = 16 * I[n] + l16, j0 = 16 * J[n] + 4 * g;
        const uint2 w2 = make_uint2(pack2_bf16(j0 <= i ? s[0] : 0.f, j0 + 1 <= i ? s[1] : 0.f),
                                    pack2_bf16(j0 + 2 <= i ? s[2] : 0.f, j0 + 3 <= i ? s[3] : 0.f));
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(stile) + tile_off<8>(i, perm_pos(j0))) = w2;
    }
}
// zeros into block (I, J) of the score tile (a block above the diagonal that
// the 32-key operands of the intra product also read)
template <int I, int J>
__device__ __forceinline__ void zero_block(u16* stile, int l16, int g) {
    using namespace pipe;
    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(stile) + tile_off<8>(16 * I + l16, perm_pos(16 * J + 4 * g))) =
        make_uint2(0u, 0u);
}

// one direct-to-LDS copy of 1 KiB (rows 8b .. 8b + 7 of a 64 x 64 bf16 tile,
// rows clamped to `last`, row stride `stride` elements) into piece b of dst
__device__ __forceinline__ void copy_piece(const u16* base, int stride, int last, u16* dst, int b, int lane) {
    using namespace pipe;
    const int slot = b * WAVE + lane;
    const int r = slot / 8, seg = (slot % 8) ^ (r & 7);
    // the copy takes its base and LDS address from scalar registers: both are
    // wave-uniform, made explicit for the compiler
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t alo = __builtin_amdgcn_readfirstlane((uint32_t)a), ahi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const u16* ub = reinterpret_cast<const u16*>(((uint64_t)ahi << 32) | alo);
    dma16(ub, (uint32_t)(((r < last ? r : last) * stride + seg * 8) * 2),
          __builtin_amdgcn_readfirstlane(lds_addr(dst) + b * WAVE * 16));
}

}  // namespace

// ---------------------------------------------------------------------------
// phase 1: one workgroup per (head, run of rows, 64 value columns)
// ---------------------------------------------------------------------------
// Wave w owns FPW feature blocks from fb0 for the 32-key halves kh0 .. kh0 +
// NKH - 1 of every tile (all four row blocks when there are at least eight
// feature blocks; at m = 64 two waves share a feature block, one per half, and
// add their sums at the end).  Per tile: the x fragments of its row blocks,
// the mapping (row blocks as rows, features as columns: lane (g, l16) gets
// rows 16 rb + 4g + i of feature 16 fb + l16), the operand pair of each
// 32-key half from the results of its two row blocks (key order 4g + i, then
// 16 + 4g + i: the order of the value tile's column operand), then the
// update S[f][16 cb + ..] += phi(K)^T V.  Every wave copies one eighth of each
// tile and waits for its own copies; one barrier per tile.
template <int M, bool Z>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void favor_states_kernel(FavorParams p) {
    using namespace pipe;
    constexpr int NFB = M / 16;
    constexpr int KSPLIT = NFB >= 8 ? 1 : 8 / NFB;
    constexpr int FPW = NFB >= 8 ? NFB / 8 : 1;
    constexpr int NRB = 4 / KSPLIT;
    constexpr int NKH = NRB / 2;
    constexpr int NSTAGE = 6;
    static_assert(FPW * 8 / KSPLIT == NFB && NKH >= 1, "feature split");

    __shared__ RawStageKV st[NSTAGE];
    __shared__ __attribute__((aligned(16))) float crl[NSTAGE][64];  // row constants of each stage's keys

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int fb0 = (wave % (8 / KSPLIT)) * FPW;
    const int kh0 = (wave / (8 / KSPLIT)) * NKH;
    const int wi = work_index(p.xcd_remap);
    const int jt = wi % p.n_dvt;
    const int64_t n = (wi / p.n_dvt) % p.n_groups;
    const int64_t bh = wi / ((int64_t)p.n_dvt * p.n_groups);
    const int col0 = jt * 64;
    const int64_t L = p.L;
    const int dv = p.dv;
    const int64_t r_begin = n * p.rows;
    const int64_t r_end = r_begin + p.rows < L ? r_begin + p.rows : L;
    const int64_t t_begin = r_begin / 64, t_end = (r_end + 63) / 64;
    const u16* kh = p.k + bh * L * 64;
    const u16* vh = p.v + bh * L * dv + col0;
    const float c1 = kLog2e * p.in_scale;
    const float cA = -0.5f * kLog2e * p.in_scale * p.in_scale;
    const float cB = -0.5f * __builtin_amdgcn_logf((float)M);
    auto issue = [&](int64_t t, RawStageKV& s) __attribute__((always_inline)) {
        const int last = (int)(L - 1 - t * 64);
        copy_piece(kh + t * 64 * 64, 64, last, s.k, wave, lane);
        copy_piece(vh + t * 64 * dv, dv, last, s.v, wave, lane);
    };
    auto land = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t newest = t + NSTAGE - 2 < t_end - 1 ? t + NSTAGE - 2 : t_end - 1;
        wait_groups<2, NSTAGE - 2>((int)(newest - t));
    };
    // Row constants log2(e) (-s^2 |k_r|^2 / 2) - log2(m) / 2 of the eight key
    // rows this wave copied (8w .. 8w + 7) of tile t, once its copy is in;
    // -inf past the end of the sequence, so that those rows map to exp2(-inf) = 0.
    auto row_consts = [&](int64_t t, const RawStageKV& s, float* out) __attribute__((always_inline)) {
        const int r = 8 * wave + lane / 8, seg = lane % 8;
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(s.k) + tile_off<8>(r, seg * 8));
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = __uint_as_float(w4[j] << 16), b = __uint_as_float(w4[j] & 0xFFFF0000u);
            q = fmaf(a, a, fmaf(b, b, q));
        }
        // the sum over the row's eight lanes: swaps within quads, then the
        // mirror within halves of a row of lanes (DPP)
        q += dpp_f<0xB1>(q);   // quad_perm [1, 0, 3, 2]
        q += dpp_f<0x4E>(q);   // quad_perm [2, 3, 0, 1]
        q += dpp_f<0x141>(q);  // row_half_mirror
        if (seg == 0) out[r] = t * 64 + r < L ? fmaf(cA, q, cB) : -__builtin_inff();
    };

    // W first: its loads are then waited for before the copies go out
    bf16x8 wf[FPW][2];
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        load_w_frag(p.W, fb0 + f, lane, wf[f]);
        settle(wf[f][0]);
        settle(wf[f][1]);
    }
    for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
        if (t_begin + s0 < t_end) issue(t_begin + s0, st[s0]);
    land(t_begin);
    if (t_begin < t_end) row_consts(t_begin, st[0], crl[0]);

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // bf16 ones: the operand that turns an update step into a column sum (z)
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    f32x4 P[FPW][4], Zs[FPW];
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        Zs[f] = zero4;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) P[f][cb] = zero4;
    }

    int si = 0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        RawStageKV& s = st[si];
        const int sp = si == 0 ? NSTAGE - 1 : si - 1;
        const int sn = si == NSTAGE - 1 ? 0 : si + 1;
        // the lane's values formed again each tile (opaque to the compiler), so
        // that the LDS addresses derived from them are not all held in registers
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int l16o = lane_o % 16, go = lane_o / 16, c4 = 4 * (lane_o & 3);
        __syncthreads();  // B(t): tile t and its row constants are in; every wave is done with tile t - 1
        if (t + NSTAGE - 1 < t_end) issue(t + NSTAGE - 1, st[sp]);
        // operands of this wave's 32-key halves: the x fragments of their row
        // blocks, the row constants of rows 16 rb + 4g + i, the value columns
        bf16x8 xa[NKH][2][2], vb[NKH][4];
        float4 cr[NKH][2];
#pragma unroll
        for (int kq = 0; kq < NKH; ++kq) {
            const int khh = kh0 + kq;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int rb = 2 * khh + hb;
#pragma unroll
                for (int h = 0; h < 2; ++h) xa[kq][hb][h] = row_op<8>(s.k, 16 * rb + l16o, 32 * h, go);
                cr[kq][hb] = *reinterpret_cast<const float4*>(&crl[si][16 * rb + 4 * go]);
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) vb[kq][cb] = col_op<8>(s.v, 32 * khh, 16 * cb + c4, lane_o);
        }
        // every mapping product first (independent chains), then per feature
        // block and key half the exponentials, the hi/lo pair and the updates
        f32x4 acc[NKH][FPW][2];
#pragma unroll
        for (int kq = 0; kq < NKH; ++kq)
#pragma unroll
            for (int f = 0; f < FPW; ++f)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) acc[kq][f][hb] = mfma_bf16(xa[kq][hb][0], wf[f][0], zero4);
#pragma unroll
        for (int kq = 0; kq < NKH; ++kq)
#pragma unroll
            for (int f = 0; f < FPW; ++f)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) acc[kq][f][hb] = mfma_bf16(xa[kq][hb][1], wf[f][1], acc[kq][f][hb]);
#pragma unroll
        for (int kq = 0; kq < NKH; ++kq)
#pragma unroll
            for (int f = 0; f < FPW; ++f) {
                float ph[2][4];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const f32x4 a = acc[kq][f][hb];
                    ph[hb][0] = __builtin_amdgcn_exp2f(fmaf(c1, a[0], cr[kq][hb].x));
                    ph[hb][1] = __builtin_amdgcn_exp2f(fmaf(c1, a[1], cr[kq][hb].y));
                    ph[hb][2] = __builtin_amdgcn_exp2f(fmaf(c1, a[2], cr[kq][hb].z));
                    ph[hb][3] = __builtin_amdgcn_exp2f(fmaf(c1, a[3], cr[kq][hb].w));
                }
                const uint4 hi = pack8(ph[0], ph[1]);
                const uint4 lo = pack8_lo(ph[0], ph[1], hi);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    P[f][cb] = mfma_bf16(as_bf16x8(hi), vb[kq][cb], P[f][cb]);
                    P[f][cb] = mfma_bf16(as_bf16x8(lo), vb[kq][cb], P[f][cb]);
                }
                if constexpr (Z) {
                    Zs[f] = mfma_bf16(as_bf16x8(hi), ones, Zs[f]);
                    Zs[f] = mfma_bf16(as_bf16x8(lo), ones, Zs[f]);
                }
            }
        if (t + 1 < t_end) {
            land(t + 1);
            row_consts(t + 1, st[sn], crl[sn]);
        }
        si = sn;
    }
    float* S = p.S + ((bh * p.n_out + n) * M) * (int64_t)dv + col0 + l16;
    float* zo = (Z && jt == 0) ? p.z + (bh * p.n_out + n) * M : nullptr;
    if constexpr (KSPLIT > 1) {
        // the second key half's sums to the first through the (idle) stages
        __syncthreads();
        float* red = reinterpret_cast<float*>(&st[0]);
        const int pw = wave % (8 / KSPLIT);
        if (wave >= 8 / KSPLIT) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[((pw * 4 + cb) * 4 + e) * WAVE + lane] = P[0][cb][e];
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((8 / KSPLIT) * 16 + pw * 4 + e) * WAVE + lane] = Zs[0][e];
        }
        __syncthreads();
        if (wave < 8 / KSPLIT) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) P[0][cb][e] += red[((pw * 4 + cb) * 4 + e) * WAVE + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) Zs[0][e] += red[((8 / KSPLIT) * 16 + pw * 4 + e) * WAVE + lane];
        } else {
            return;
        }
    }
    // S[f][feature 16 fb + 4g + e][column 16 cb + l16]; z of feature 16 fb + 4g + e
    // is in every column of Zs
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        const int a0 = 16 * (fb0 + f);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[(int64_t)(a0 + 4 * g + e) * dv + 16 * cb] = P[f][cb][e];
        if (Z && zo != nullptr && l16 == 0)
#pragma unroll
            for (int e = 0; e < 4; ++e) zo[a0 + 4 * g + e] = Zs[f][e];
    }
}

// ---------------------------------------------------------------------------
// phase 3: one workgroup per (head, group of chunks of 64, 64 value columns)
// ---------------------------------------------------------------------------
// Two groups of four waves, one of each on every SIMD, a chunk apart:
//  * product waves 0-3 run chunk t: the score tile, phi(q_i) . z, the inter
//    and intra products, the outputs and the state update, with the state of
//    value columns 16 w .. 16 w + 15 over all features in fp32 accumulators (a
//    packed pair is an operand in feature order); they also move the value
//    tiles (direct-to-LDS copies) and store the output rows;
//  * mapper waves 4-7 map chunk t + 1 meanwhile: each keeps W for a quarter of
//    the features in registers and reads the raw q and k rows it needs straight
//    into registers (one chunk ahead), so the raw q and k never occupy LDS;
//    phi(k) of chunk t + 1 before BS(t), phi(q) after it.
// With the normaliser each product wave also keeps z for a quarter of the
// feature steps in fp32 accumulators: z += the column sums of phi(K) comes
// from the matrix cores with a ones operand on the state update's phi(K)
// operands, and the rows' partial products phi(q_r) . z over those steps from
// z as a bf16 hi/lo operand against the inter product's phi(q) operands; the
// four partials meet in LDS.  phi(k) is double-buffered by chunk parity;
// phi(q) is read before BS only, so it has one buffer.  Two barriers per chunk t:
//   B(t):  phi of chunk t is complete (mapped during chunk t - 1), its value
//          tile has landed, and chunk t - 1's products are done (the other
//          phi(k) buffer, the score tile and chunk t - 1's stage are free);
//   BS(t): the score tile (tril(phi(Q) phi(K)^T), columns in operand key
//          order) is complete, and so are the inter products phi(Q) P (the
//          phi(q) buffer is free).
// Scores and outputs are computed transposed (keys, resp. value columns, as
// rows), so a lane holds four consecutive keys or columns of one row (one
// 8-byte store); the row sums of the score tile come from the matrix cores with
// a ones operand, in the outputs' layout.  Row norms come from the matrix
// cores too: the diagonal of x x^T for each 16-row block.  The ten score blocks
// on and below the diagonal go to the product waves in groups that share query
// or key blocks: (0,0) (1,0) (1,1) | (2,0) (2,1) (3,0) | (2,2) (3,2) | (3,1) (3,3).
template <int M, bool NORM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void favor_fwd_kernel(FavorParams p) {
    using namespace pipe;
    constexpr int FSEG = M / 8, NKS = M / 32, FPW = M / 64;
    constexpr bool SWK = FSEG >= 16;  // phi(k)'s swizzle key (phi_off)
    constexpr int PHI_E = 64 * M;  // elements of one phi tile
    // as many value stages as the LDS holds beside the rest, at most four
    // z is kept by the product waves, KPW feature steps each (waves w < NKS / KPW)
    constexpr int KPW = NKS >= 4 ? NKS / 4 : 1;
    constexpr int FIXED = 3 * PHI_E * 2 + 64 * 64 * 2 + 64 * 4 * 4;
    constexpr int NVFIT = (160 * 1024 - FIXED) / (64 * 64 * 2);
    constexpr int NV = NVFIT < 4 ? NVFIT : 4;
    static_assert(NV >= 2, "value stages");

    __shared__ __attribute__((aligned(16))) u16 fq[PHI_E];
    __shared__ __attribute__((aligned(16))) u16 fk[2][PHI_E];
    __shared__ __attribute__((aligned(16))) u16 vst[NV][64 * 64];
    __shared__ __attribute__((aligned(16))) u16 stile[64 * 64];
    // phi(q_r) . z partials: [row r][product wave]
    __shared__ __attribute__((aligned(16))) float qzp[NORM ? 64 * 4 : 4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const bool mapper = wave >= 4;
    const int pw = wave & 3;
    const int lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int wi = work_index(p.xcd_remap);
    const int jt = wi % p.n_dvt;
    const int grp = (wi / p.n_dvt) % p.n_groups;
    const int64_t bh = wi / ((int64_t)p.n_dvt * p.n_groups);
    const int col0 = jt * 64, cw = 16 * pw;
    const int fb0 = pw * FPW;  // mapper: first feature block (FPW blocks of 16 features)
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
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    const float c1 = kLog2e * p.in_scale;
    const float cA = -0.5f * kLog2e * p.in_scale * p.in_scale;
    const float cB = -0.5f * __builtin_amdgcn_logf((float)M);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

    if (mapper) {
        // ================= mapper waves =================
        bf16x8 wf[FPW][2];
#pragma unroll
        for (int f = 0; f < FPW; ++f) load_w_frag(p.W, fb0 + f, lane, wf[f]);
        // x fragments of tile t: rows 16 rb + l16 (clamped to the last row),
        // inputs 32 h + 8g .. + 7
        auto load_x = [&](const u16* base, int64_t t, bf16x8 (&x)[4][2]) __attribute__((always_inline)) {
            const int last = (int)(L - 1 - t * 64);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int r = 16 * rb + l16;
                const u16* row = base + (t * 64 + (r < last ? r : last)) * 64 + 8 * g;
#pragma unroll
                for (int h = 0; h < 2; ++h) x[rb][h] = as_bf16x8(*reinterpret_cast<const uint4*>(row + 32 * h));
            }
        };
        // phi of a tile into a phi tile: row norms from the diagonal of x x^T
        // (lane (g, l16) holds rows 16 rb + 4g + i against row 16 rb + l16; the
        // diagonal of row r sits in lane (r / 4, r), element r mod 4), then the
        // features fb0 .. fb0 + FPW - 1 of every row (lane (g, l16): features
        // 16 fb + 4g + i of row 16 rb + l16); key rows at or past `valid` map to 0
        auto map = [&](const bf16x8 (&x)[4][2], u16* phi, int valid, auto swap) __attribute__((always_inline)) {
            constexpr bool SW = decltype(swap)::value;
            // the row norms of all four row blocks first (their lane exchanges overlap)
            float nrm[4];
            const int e = l16 & 3;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                f32x4 d = mfma_bf16(x[rb][0], x[rb][0], zero4);
                d = mfma_bf16(x[rb][1], x[rb][1], d);
                const float d01 = (e & 1) ? d[1] : d[0], d23 = (e & 1) ? d[3] : d[2];
                nrm[rb] = __shfl((e & 2) ? d23 : d01, (l16 >> 2) * 16 + l16);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int r = 16 * rb + l16;
                const float cr = r < valid ? fmaf(cA, nrm[rb], cB) : -__builtin_inff();
                // the feature blocks' products as independent chains, then their exponentials
                f32x4 acc[FPW];
#pragma unroll
                for (int f = 0; f < FPW; ++f) acc[f] = mfma_bf16(wf[f][0], x[rb][0], zero4);
#pragma unroll
                for (int f = 0; f < FPW; ++f) acc[f] = mfma_bf16(wf[f][1], x[rb][1], acc[f]);
#pragma unroll
                for (int f = 0; f < FPW; ++f) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(c1, acc[f][0], cr));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(c1, acc[f][1], cr));
                    const float p2 = __builtin_amdgcn_exp2f(fmaf(c1, acc[f][2], cr));
                    const float p3 = __builtin_amdgcn_exp2f(fmaf(c1, acc[f][3], cr));
                    const uint2 w2 = make_uint2(pack2_bf16(p0, p1), pack2_bf16(p2, p3));
                    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(phi) + phi_off<FSEG, SW>(r, 16 * (fb0 + f) + 4 * g)) = w2;
                }
            }
        };
        bf16x8 xq[4][2], xk[4][2];
        // prologue: chunk t_begin mapped into buffer 0 (queries need no zeroing:
        // their rows past the end give outputs that are not stored)
        load_x(qh, t_begin, xq);
        load_x(kh, t_begin, xk);
        map(xq, fq, 64, std::false_type{});
        map(xk, fk[0], valid_of(t_begin), std::integral_constant<bool, SWK>{});
        if (t_begin + 1 < t_end) {
            load_x(qh, t_begin + 1, xq);
            load_x(kh, t_begin + 1, xk);
        }
        for (int64_t t = t_begin; t < t_end; ++t) {
            const int b = (int)((t - t_begin) & 1);
            __syncthreads();  // B(t)
            if (t + 1 < t_end) {
                map(xk, fk[b ^ 1], valid_of(t + 1), std::integral_constant<bool, SWK>{});
                if (t + 2 < t_end) load_x(kh, t + 2, xk);
            }
            __syncthreads();  // BS(t)
            if (t + 1 < t_end) {
                map(xq, fq, 64, std::false_type{});
                if (t + 2 < t_end) load_x(qh, t + 2, xq);
            }
        }
        __syncthreads();  // B(t_end)
        return;
    }

    // ================= product waves =================
    // value tile t: this wave's two 1 KiB pieces (rows 16 pw .. 16 pw + 15)
    auto issue = [&](int64_t t, u16* dst) __attribute__((always_inline)) {
        const int last = (int)(L - 1 - t * 64);
#pragma unroll
        for (int i = 0; i < 2; ++i) copy_piece(vh + t * 64 * dv, dv, last, dst, pw * 2 + i, lane);
    };
    // this wave's copies of value tile t are in (two copy instructions per tile)
    auto land = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t newest = t + NV - 2 < t_end - 1 ? t + NV - 2 : t_end - 1;
        wait_groups<2, NV - 2>((int)(newest - t));
    };
    // output rows of a stage (the same rows as this wave's copies): piece
    // (pw * 2 + i) * 64 + lane
    auto read_out = [&](const u16* from, u32x4 (&ob)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = (pw * 2 + i) * WAVE + lane, r = piece / 8, seg = piece % 8;
            ob[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(from) + tile_off<8>(r, seg * 8));
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
    // state: P[ks][hf] lane (g, l16) element i = P[32 ks + 8g + 4hf + i][cw + l16]
    f32x4 P[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) P[ks][0] = P[ks][1] = zero4;
    // z at feature steps KPW pw + k2: Zs[k2][hf] lane (g, l16) element i =
    // z[32 (KPW pw + k2) + 8g + 4hf + i] (every column the same)
    const bool has_z = NORM && pw < NKS / KPW;
    f32x4 Zs[KPW][2];
#pragma unroll
    for (int k2 = 0; k2 < KPW; ++k2) Zs[k2][0] = Zs[k2][1] = zero4;
    const bool has_prefix = grp > 0;
    if (p.P0 != nullptr && has_prefix) {
        const float* P0 = p.P0 + (slot * M) * (int64_t)dv + col0 + cw + l16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) P[ks][hf][e] = P0[(int64_t)(32 * ks + 8 * g + 4 * hf + e) * dv];
    }
    if (has_z && p.z0 != nullptr && has_prefix)
#pragma unroll
        for (int k2 = 0; k2 < KPW; ++k2)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) Zs[k2][hf][e] = p.z0[slot * M + 32 * (KPW * pw + k2) + 8 * g + 4 * hf + e];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        settle(P[ks][0]);
        settle(P[ks][1]);
    }
#pragma unroll
    for (int k2 = 0; k2 < KPW; ++k2) {
        settle(Zs[k2][0]);
        settle(Zs[k2][1]);
    }
    // the copies go out after the loads above have been waited for
    for (int s0 = 0; s0 < NV - 1; ++s0)
        if (t_begin + s0 < t_end) issue(t_begin + s0, vst[s0]);
    land(t_begin);
    const RowAddr<FSEG> raf(lane);
    const RowAddr<FSEG, SWK> rak(lane);
    const RowAddr<8> ra8(lane);
    const ColAddr<FSEG, SWK> caf(lane);

    u32x4 ob[2];  // chunk t - 1's output rows, stored once tile t + 1 has landed
    int si = 0;   // value stage of chunk t
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int b = (int)((t - t_begin) & 1);
        const int sp = si == 0 ? NV - 1 : si - 1;  // stage of chunk t - 1
        const int sn = si == NV - 1 ? 0 : si + 1;  // stage of tile t + 1
        const u16* q_ = fq;
        const u16* k_ = fk[b];
        u16* v_ = vst[si];
        // the lane's values formed again each chunk (opaque to the compiler), so
        // that the LDS addresses derived from them are not all held in registers
        // across the chunk loop
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int l16 = lane_o % 16, g = lane_o / 16, c4 = 4 * (lane_o & 3);
        __syncthreads();  // B(t)
        // chunk t - 1's output rows leave its stage, which takes value tile t + NV - 1
        if (t > t_begin) read_out(vst[sp], ob);
        if (t + NV - 1 < t_end) issue(t + NV - 1, vst[sp]);
        // the score tile: this wave's group of blocks (the product waves'
        // groups share query or key blocks), and zeros in blocks (0, 1) and
        // (2, 3), which the 32-key operands of the intra product also read
        if (pw == 0) {
            score_blocks<FSEG, NKS, SWK, 0, 0, 1, 0, 1, 1>(q_, k_, stile, raf, rak, l16, g);
            zero_block<0, 1>(stile, l16, g);
        } else if (pw == 1) {
            score_blocks<FSEG, NKS, SWK, 2, 0, 2, 1, 3, 0>(q_, k_, stile, raf, rak, l16, g);
        } else if (pw == 2) {
            score_blocks<FSEG, NKS, SWK, 2, 2, 3, 2, -1, -1>(q_, k_, stile, raf, rak, l16, g);
        } else {
            score_blocks<FSEG, NKS, SWK, 3, 1, 3, 3, -1, -1>(q_, k_, stile, raf, rak, l16, g);
            zero_block<2, 3>(stile, l16, g);
        }
        // the inter product O^T = P^T phi(Q)^T: lane (g, l16) holds output row
        // 16 ib + l16, columns cw + 4g + e; with the normaliser, at this wave's
        // feature steps, phi(q_r) . z from the same phi(q) operands (z as a
        // bf16 hi/lo pair broadcast over the rows of the A operand)
        f32x4 O[4], R[4], QZ[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) O[ib] = R[ib] = QZ[ib] = zero4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 pk = pack_acc_bf16(P[ks][0], P[ks][1]);
            if (has_z && ks / KPW == pw) {
                const f32x4& za = Zs[ks % KPW][0];
                const f32x4& zb = Zs[ks % KPW][1];
                const float a4[4] = {za[0], za[1], za[2], za[3]}, b4[4] = {zb[0], zb[1], zb[2], zb[3]};
                const uint4 zh = pack8(a4, b4), zl = pack8_lo(a4, b4, zh);
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const bf16x8 qf = row_at(q_, raf.off(16 * ib, 32 * ks));
                    O[ib] = mfma_bf16(pk, qf, O[ib]);
                    QZ[ib] = mfma_bf16(as_bf16x8(zh), qf, QZ[ib]);
                    QZ[ib] = mfma_bf16(as_bf16x8(zl), qf, QZ[ib]);
                }
            } else {
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) O[ib] = mfma_bf16(pk, row_at(q_, raf.off(16 * ib, 32 * ks)), O[ib]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NORM)
            if (g == 0)
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) qzp[(16 * ib + l16) * 4 + pw] = QZ[ib][0];
        __syncthreads();  // BS(t)
        {
            bf16x8 vb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) vb[kk] = col_op<8>(v_, 32 * kk, cw + c4, lane_o);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                for (int kk = 0; kk <= ib / 2; ++kk) {
                    const bf16x8 sb = row_at(stile, ra8.off(16 * ib, 32 * kk));
                    O[ib] = mfma_bf16(vb[kk], sb, O[ib]);
                    if constexpr (NORM) R[ib] = mfma_bf16(ones, sb, R[ib]);
                }
            // the output rows (normalised by phi(q_r) . z, the product waves'
            // four partials, + the row's score sum) into this wave's own V columns
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const int r = 16 * ib + l16;
                float rd = 1.f;
                if constexpr (NORM) {
                    const float4 qq = *reinterpret_cast<const float4*>(qzp + r * 4);
                    rd = __builtin_amdgcn_rcpf((qq.x + qq.y) + (qq.z + qq.w) + R[ib][0]);
                }
                *reinterpret_cast<uint2*>(reinterpret_cast<char*>(v_) + tile_off<8>(r, cw + 4 * g)) =
                    make_uint2(pack2_bf16(O[ib][0] * rd, O[ib][1] * rd), pack2_bf16(O[ib][2] * rd, O[ib][3] * rd));
            }
            // P += phi(K)^T V, and at this wave's feature steps z += the column
            // sums of phi(K) from the same operands
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if (has_z && ks / KPW == pw) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const bf16x8 a = col_at(k_, caf, 32 * kk, 32 * ks, hf);
                            P[ks][hf] = mfma_bf16(a, vb[kk], P[ks][hf]);
                            Zs[ks % KPW][hf] = mfma_bf16(a, ones, Zs[ks % KPW][hf]);
                        }
                } else {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf)
                            P[ks][hf] = mfma_bf16(col_at(k_, caf, 32 * kk, 32 * ks, hf), vb[kk], P[ks][hf]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // tile t + 1 must be in before B(t + 1); then chunk t - 1's rows go out
        if (t + 1 < t_end) land(t + 1);
        if (t > t_begin) store_out(t - 1, ob);
        si = sn;
    }
    __syncthreads();  // B(t_end): the last chunk's outputs are in its stage
    read_out(vst[si == 0 ? NV - 1 : si - 1], ob);
    store_out(t_end - 1, ob);
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
