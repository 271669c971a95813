// Chunked causal linear attention, fused phase 3, streaming variant for chunks
// of 64 rows (gfx950).
//
// Same mathematics as chunked_fwd_bf16 (page "attention と線形の間",
// section ②: O_c = Q_c P + tril(Q_c K_c^T) V_c with the diagonal kept, then
// P += K_c^T V_c), organised for HBM streaming:
//
//  * Global -> LDS copies go through the direct-to-LDS load
//    (global_load_lds_dwordx4): no register staging, no LDS store pass.  Three
//    LDS stages per workgroup; the copy of chunk i+2 is issued right after the
//    barrier that opens chunk i, so two chunks are in flight while one computes.
//    One barrier per chunk.
//  * Each wave computes every score block it needs itself (S^T = K Q^T on the
//    matrix cores) and keeps the masked scores in registers: the accumulator
//    layout of S^T is exactly the operand layout of the intra product in the
//    permuted key order below, so scores never go through LDS.
//  * Output blocks are produced transposed (O^T = P^T Q^T + V^T tril(S)^T), so
//    a lane holds four consecutive output columns of one row and writes them
//    as one 8-byte store; the store of chunk i is issued after the barrier of
//    chunk i+1, before that chunk's copies, which keeps the memory counter
//    arithmetic exact (stores never sit between a copy and its wait).
//
// LDS tiles are row-major with a per-row XOR swizzle of the 16-byte segment
// index (the copy picks, per lane, which global segment lands in which LDS
// slot).  The swizzle never touches bit 1 of the segment index, so the two
// 8-byte halves of a permuted row operand stay 32 bytes apart.
//
// Matrix-core mapping (16x16x32 bf16; permuted order inside every 32-wide
// k-step: lane group g holds indices 4g..4g+3 and 16+4g..16+4g+3):
//   scores  S^T[key][q] += K[key][a]  Q[q][a]      A = K rows,    B = Q rows
//   inter   O^T[j][q]   += P[a][j]    Q[q][a]      A = P (regs),  B = Q rows
//   intra   O^T[j][q]   += V[key][j]  S^T[key][q]  A = V columns, B = S^T (regs)
//   update  P[a][j]     += K[key][a]  V[key][j]    A = K columns, B = V columns
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

namespace pipe {

constexpr int T = 64;   // rows per chunk (this kernel is for C == 64)
#ifndef LA_PIPE_NW
#define LA_PIPE_NW 2
#endif
constexpr int NW = LA_PIPE_NW;  // compute waves per workgroup
constexpr int NCP = 2;          // copy waves per workgroup

// Byte offset of element e of row r in a tile with NSEG 16-byte segments per
// row: segment index XOR (row mod NSEG).  Row reads of 16 bytes over 16
// consecutive rows and the transpose reads over 16 rows both spread over all
// banks with this swizzle.
template <int NSEG>
__device__ __forceinline__ int tile_off(int r, int e) {
    return r * NSEG * 16 + ((((e >> 3) ^ r) & (NSEG - 1)) << 4) + ((e & 7) << 1);
}

template <int DK, int DVT>
struct alignas(16) Stage {
    u16 q[T * DK];
    u16 k[T * DK];
    u16 v[T * DVT];
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

__device__ __forceinline__ uint2 tr_read(const char* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p));
}

// Row operand: row r, elements k0 + 8g .. k0 + 8g + 7 (one 16-byte read).
template <int NSEG>
__device__ __forceinline__ bf16x8 row_op(const u16* tile, int r, int k0, int g) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + tile_off<NSEG>(r, k0 + 8 * g)));
}

// Column operand over keys in the permuted order: lane (g, rr = (l%16)/4, c = l%4)
// addresses rows key0 + 4g + rr and key0 + 16 + 4g + rr at column col_c .. +3; the
// transpose read hands lane (g, n) the column of lane c = n/4, element n%4.
template <int NSEG>
__device__ __forceinline__ bf16x8 col_op(const u16* tile, int key0, int col_c, int lane) {
    const int g = lane >> 4, rr = (lane & 15) >> 2;
    const int r = key0 + 4 * g + rr;
    const char* t = reinterpret_cast<const char*>(tile);
    const uint2 lo = tr_read(t + tile_off<NSEG>(r, col_c));
    const uint2 hi = tr_read(t + tile_off<NSEG>(r + 16, col_c));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// One direct-to-LDS copy instruction: lane l fetches the 16 bytes at
// base + voff(l) and the wave's 64 pieces land contiguously at LDS byte address
// `lds` (wave-uniform) in lane order.  Written as inline assembly so that the
// compiler does not order LDS reads against copies in flight; completion is
// tracked explicitly with the memory counter and a barrier.  M0 (the LDS base
// of the copy) is saved and restored around it.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds)
        : "memory");
}

// LDS byte address of a pointer into a __shared__ object: the low 32 bits of
// its generic address (the shared aperture sits in the high half).
template <typename E>
__device__ __forceinline__ uint32_t lds_addr(const E* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// s_waitcnt vmcnt(N) with every other counter left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int work_index(int remap) {
    const int b = blockIdx.x;
    if (!remap) return b;
    const int per = gridDim.x >> 3;
    return (b & 7) * per + (b >> 3);
}

}  // namespace pipe

// One workgroup: (head, group of chunks, tile of DVT value columns); NW
// compute waves (two by default: each then owns 32 value columns, which halves
// the LDS reads of Q and K per output column against four waves of 16) and
// two copy waves.  Compute wave w owns value columns [w*DVT/NW, (w+1)*DVT/NW)
// of O and of the state; it touches only LDS and the
// matrix cores.  The copy waves issue every global access of the chunk loop,
// half each: the direct-to-LDS copies of Q, K, V and the output stores.  A
// wave stalls when it has 63 memory instructions in flight (the counter's
// limit) or the memory queue is full; keeping those stalls on waves of their
// own lets the copies stream continuously while the compute waves work, and
// two copy waves keep two chunks of copies in flight under that limit.
//
// Per chunk j, after the barrier B(j) that makes chunk j's tiles visible:
//   compute waves: products of chunk j from stage j % NSTAGE; the output rows
//     go back into that stage's V tile, into the columns the same wave read V
//     from (no other wave reads them);
//   copy waves: read the output of chunk j - 1 from stage (j - 1) % NSTAGE,
//     refill that stage with chunk j + NSTAGE - 1, stores the output rows
//     (full 16-byte segments of a row), then wait until chunk j + 1 has
//     landed and meet the compute waves at B(j + 1).
//
// Index orders inside 32-wide k-steps.  Keys: permuted (lane group g holds keys
// 4g..4g+3 and 16+4g..16+4g+3), the order in which the score accumulators
// S^T[key][q] come out of the matrix core (C rows 4g + i of 16-key blocks), so
// the masked scores feed the intra product straight from registers.  Features
// a: natural (lane group g holds 8g..8g+7) for the 16-byte row reads of Q and
// K; the state update reads K's columns with lane c of each row quad pointing
// at column 8c (+4 for the second half), so the update's accumulator rows come
// out as a = 32ks + 8g + 4h + i (h = half) and a packed pair (h = 0, 1) is the
// inter product's operand in natural order, again without leaving registers.
template <int DK, int DVT, int NSTAGE, bool SCALED>
__global__ __launch_bounds__((pipe::NW + pipe::NCP) * WAVE)
__attribute__((amdgpu_waves_per_eu((pipe::NW + pipe::NCP + 3) / 4, (pipe::NW + pipe::NCP + 3) / 4)))
void chunked_fwd_pipe(FwdParams p) {
    using namespace pipe;
    constexpr int CPW = DVT / 16 / NW;     // 16-column blocks per compute wave
    constexpr int NQB = T / 16;            // 16-row blocks per chunk
    constexpr int NKA = DK / 32;           // k-steps over the feature index
    constexpr int NKK = T / 32;            // k-steps over keys
    constexpr int QSEG = DK / 8, VSEG = DVT / 8;
    constexpr int NCQ = T * QSEG / WAVE / NCP;  // copy instructions per chunk and copy wave, Q (and K)
    constexpr int NCV = T * VSEG / WAVE / NCP;  // the same for V (and for the output stores)
    constexpr int NL = 2 * NCQ + NCV;
    constexpr int NTRI = NQB * (NQB + 1) / 2;
    constexpr int RPV = WAVE / VSEG;       // output rows per store instruction
    static_assert(CPW >= 1 && CPW * 16 * NW == DVT, "DVT must be 64 or 128");
    static_assert(NSTAGE == 3, "three LDS stages");
    static_assert(NL < 64, "vmcnt range");
    static_assert(NCV >= 1, "tile too small for the copy split");

    __shared__ Stage<DK, DVT> st[NSTAGE];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const bool copier = wave >= NW;  // wave-uniform
    const int cw = __builtin_amdgcn_readfirstlane(wave - NW);  // copy wave index (wave-uniform)

    const int w = work_index(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int grp = (w / p.n_dvt) % p.n_groups;
    const int64_t bh = w / (p.n_dvt * p.n_groups);
    const int col0 = jt * DVT;

    const int64_t L = p.L;
    const int dv = p.dv;
    const int64_t n_chunks = (L + T - 1) / T;
    const int64_t c_begin = (int64_t)grp * p.G;
    const int64_t c_end = c_begin + p.G < n_chunks ? c_begin + p.G : n_chunks;

    // rows of chunk c that exist
    auto valid_rows = [&](int64_t c) -> int { return (int)(L - c * T < T ? L - c * T : T); };

    // rows past the end of the sequence: zero their K rows (scores and state
    // contributions vanish; their Q rows produce outputs that are not stored)
    auto zero_tail = [&](Stage<DK, DVT>& s, int valid) __attribute__((always_inline)) {
        const int n = (T - valid) * QSEG;
        uint4* kk = reinterpret_cast<uint4*>(s.k + valid * DK);
        for (int i = tid; i < n; i += (NW + NCP) * WAVE) kk[i] = make_uint4(0, 0, 0, 0);
    };

    if (copier) {
        // ================= copy wave =================
        const u16* qh = p.q + bh * L * DK;
        const u16* kh = p.k + bh * L * DK;
        const u16* vh = p.v + bh * L * dv + col0;
        // Lane l of copy instruction b lands in LDS slot 64b + l = (row,
        // physical segment) = (slot / NSEG, slot % NSEG), which holds the
        // global segment (physical ^ row) of that row.
        auto issue = [&](int64_t chunk, Stage<DK, DVT>& s) __attribute__((always_inline)) {
            const int64_t r0 = chunk * T;
            const int last = (int)(L - 1 - r0);  // rows past it are clamped to it
            const u16* qb_ = qh + r0 * DK;
            const u16* kb_ = kh + r0 * DK;
            const u16* vb_ = vh + r0 * dv;
            const uint32_t lq = lds_addr(s.q), lk = lds_addr(s.k), lv = lds_addr(s.v);
#pragma unroll
            for (int i = 0; i < NCQ; ++i) {
                const int b = cw * NCQ + i;  // copy instruction within the tile
                const int slot = b * WAVE + lane;
                const int r = slot / QSEG, seg = (slot % QSEG) ^ (r & (QSEG - 1));
                const uint32_t off = (uint32_t)(((r < last ? r : last) * DK + seg * 8) * 2);
                dma16(qb_, off, lq + b * WAVE * 16);
                dma16(kb_, off, lk + b * WAVE * 16);
            }
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int b = cw * NCV + i;
                const int slot = b * WAVE + lane;
                const int r = slot / VSEG, seg = (slot % VSEG) ^ (r & (VSEG - 1));
                dma16(vb_, (uint32_t)(((r < last ? r : last) * dv + seg * 8) * 2), lv + b * WAVE * 16);
            }
        };
        // Output rows of chunk c sit in the V tile of stage `from`: instruction
        // i, lane l covers row i * RPV + l / VSEG, segment l % VSEG.  Read them,
        // refill the stage with chunk `refill` (if any), store them.
        auto drain_refill = [&](const Stage<DK, DVT>& from, int64_t c, int64_t refill, Stage<DK, DVT>& to)
            __attribute__((always_inline)) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            u32x4 ob[NCV];
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int r = (cw * NCV + i) * RPV + lane / VSEG, seg = lane % VSEG;
                ob[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(from.v) +
                                                        tile_off<VSEG>(r, seg * 8));
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads done before the refill
            if (refill >= 0) issue(refill, to);
            const int valid = valid_rows(c);
            u16* o = reinterpret_cast<u16*>(p.o) + (bh * L + c * T) * dv + col0;
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int r = (cw * NCV + i) * RPV + lane / VSEG, seg = lane % VSEG;
                if (r < valid) *reinterpret_cast<u32x4*>(o + (int64_t)r * dv + seg * 8) = ob[i];
            }
        };

#pragma unroll
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (c_begin + s0 < c_end) issue(c_begin + s0, st[s0]);
        // wait for the first chunk: the copies issued after it are those of the second
        if (c_begin + 1 < c_end)
            wait_vm<NL>();
        else
            wait_vm<0>();

        auto step = [&](auto sidx, int64_t chunk) __attribute__((always_inline)) {
            constexpr int SI = decltype(sidx)::value;
            constexpr int SP = (SI + NSTAGE - 1) % NSTAGE;  // stage of chunk - 1
            __syncthreads();  // B(chunk)
            if (valid_rows(chunk) < T) {
                zero_tail(st[SI], valid_rows(chunk));
                __syncthreads();
            }
            const int64_t refill = chunk + NSTAGE - 1 < c_end ? chunk + NSTAGE - 1 : -1;
            if (chunk > c_begin)
                drain_refill(st[SP], chunk - 1, refill, st[SP]);
            else if (refill >= 0)
                issue(refill, st[SP]);
            // chunk + 1 must have landed before B(chunk + 1); the loads issued after
            // it are those of chunk + 2 (if any); loads complete in order
            if (chunk + 2 < c_end)
                wait_vm<NL>();
            else
                wait_vm<0>();
        };
        for (int64_t chunk = c_begin; chunk < c_end; chunk += NSTAGE) {
            step(std::integral_constant<int, 0>{}, chunk);
            if (chunk + 1 < c_end) step(std::integral_constant<int, 1>{}, chunk + 1);
            if (chunk + 2 < c_end) step(std::integral_constant<int, 2>{}, chunk + 2);
        }
        __syncthreads();  // the last chunk's output is in its stage
        const int sl = (int)((c_end - 1 - c_begin) % NSTAGE);
        if (sl == 0)
            drain_refill(st[0], c_end - 1, -1, st[0]);
        else if (sl == 1)
            drain_refill(st[1], c_end - 1, -1, st[1]);
        else
            drain_refill(st[2], c_end - 1, -1, st[2]);
        return;
    }

    // ================= compute waves =================
    // ---- state P: P[c][ks][h] lane (l16, g) element i = P[a = 32ks + 8g + 4h + i][j = colw + 16c + l16]
    const int colw = wave * CPW * 16;
    f32x4 P[CPW][NKA][2];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) P[c][ks][0] = P[c][ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.P0 != nullptr && grp > 0) {
        const float* P0 = p.P0 + ((bh * p.n_groups + grp) * DK) * (int64_t)dv + col0 + colw + l16;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        P[c][ks][h][i] = P0[(int64_t)(32 * ks + 8 * g + 4 * h + i) * dv + c * 16];
    }
    const float osc = p.out_scale;

    // Operands of one 32-wide feature step: Q rows (B of the scores and of the
    // inter product) and K rows (A of the scores).
    auto load_qk = [&](const Stage<DK, DVT>& s, int ks, bf16x8 (&qa)[NQB], bf16x8 (&ka)[NQB])
        __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NQB; ++b) {
            qa[b] = row_op<QSEG>(s.q, b * 16 + l16, ks * 32, g);
            ka[b] = row_op<QSEG>(s.k, b * 16 + l16, ks * 32, g);
        }
    };

    // K column operands of one feature step for the state update: columns
    // 32ks + 8c + 4h (lane c of each row quad), keys in the permuted order.
    const int c4 = 4 * (lane & 3), c8 = 8 * (lane & 3);
    auto load_kc = [&](const Stage<DK, DVT>& s, int ks, bf16x8 (&kc)[2][NKK]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) kc[h][kk] = col_op<QSEG>(s.k, kk * 32, ks * 32 + c8 + 4 * h, lane);
    };

    // The chunk's products, one 32-wide feature step at a time: scores, the
    // inter product (which reads the state as it was before this chunk) and
    // that step's rows of the state update, with the next step's operands
    // loaded ahead.  Then the mask, the intra product and the output, which
    // goes back into this wave's V columns.
    auto compute = [&](Stage<DK, DVT>& s) __attribute__((always_inline)) {
        bf16x8 qa0[NQB], ka0[NQB], qa1[NQB], ka1[NQB];
        bf16x8 kc0[2][NKK], kc1[2][NKK];
        bf16x8 vb[CPW][NKK];
        load_qk(s, 0, qa0, ka0);
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) vb[c][kk] = col_op<VSEG>(s.v, kk * 32, colw + c * 16 + c4, lane);
        load_kc(s, 0, kc0);
        f32x4 S[NTRI];  // S^T blocks (kb <= qb), index qb(qb+1)/2 + kb
        f32x4 O[CPW][NQB];  // O^T blocks: lane holds O[q = 16qb + l16][j = colw + 16c + 4g + i]
#pragma unroll
        for (int t = 0; t < NTRI; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) O[c][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) {
            bf16x8 (&qa)[NQB] = (ks & 1) ? qa1 : qa0;
            bf16x8 (&ka)[NQB] = (ks & 1) ? ka1 : ka0;
            bf16x8 (&kc)[2][NKK] = (ks & 1) ? kc1 : kc0;
            if (ks + 1 < NKA) {
                load_qk(s, ks + 1, (ks & 1) ? qa0 : qa1, (ks & 1) ? ka0 : ka1);
                load_kc(s, ks + 1, (ks & 1) ? kc0 : kc1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int kb = 0; kb <= qb; ++kb)
                    S[qb * (qb + 1) / 2 + kb] = mfma_bf16(ka[kb], qa[qb], S[qb * (qb + 1) / 2 + kb]);
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const bf16x8 pb = pack_acc_bf16(P[c][ks][0], P[c][ks][1]);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) O[c][qb] = mfma_bf16(pb, qa[qb], O[c][qb]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) P[c][ks][h] = mfma_bf16(kc[h][kk], vb[c][kk], P[c][ks][h]);
            }
        }
        // causal mask on the diagonal blocks: keep key 16qb + 4g + i <= q = 16qb + l16
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i > l16) S[qb * (qb + 1) / 2 + qb][i] = 0.f;
        // intra: key steps kk <= qb / 2 (blocks past the diagonal are zero)
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
            for (int kk = 0; kk <= qb / 2; ++kk) {
                const int kb0 = 2 * kk, kb1 = 2 * kk + 1;
                const f32x4 s0 = S[qb * (qb + 1) / 2 + kb0];
                const f32x4 s1 = kb1 <= qb ? S[qb * (qb + 1) / 2 + kb1] : zero4;
                const bf16x8 sb = pack_acc_bf16(s0, s1);
#pragma unroll
                for (int c = 0; c < CPW; ++c) O[c][qb] = mfma_bf16(vb[c][kk], sb, O[c][qb]);
            }
        }
        // output rows into this wave's V columns (after its last V read, in order)
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                f32x4 o = O[c][qb];
                if (SCALED) o *= osc;
                *reinterpret_cast<uint2*>(reinterpret_cast<char*>(s.v) +
                                          tile_off<VSEG>(qb * 16 + l16, colw + c * 16 + 4 * g)) =
                    make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
            }
    };

    auto step = [&](auto sidx, int64_t chunk) __attribute__((always_inline)) {
        constexpr int SI = decltype(sidx)::value;
        __syncthreads();  // B(chunk)
        if (valid_rows(chunk) < T) {
            zero_tail(st[SI], valid_rows(chunk));
            __syncthreads();
        }
        compute(st[SI]);
    };
    for (int64_t chunk = c_begin; chunk < c_end; chunk += NSTAGE) {
        step(std::integral_constant<int, 0>{}, chunk);
        if (chunk + 1 < c_end) step(std::integral_constant<int, 1>{}, chunk + 1);
        if (chunk + 2 < c_end) step(std::integral_constant<int, 2>{}, chunk + 2);
    }
    __syncthreads();  // matches the copy wave's final barrier

    if (c_end == n_chunks && p.S_final != nullptr) {
        float* Sf = p.S_final + (bh * DK) * (int64_t)dv + col0 + colw + l16;
        const float ss = p.state_scale;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Sf[(int64_t)(32 * ks + 8 * g + 4 * h + i) * dv + c * 16] = P[c][ks][h][i] * ss;
    }
}

template <int DK, int DVT>
hipError_t launch_fwd_pipe(const FwdParams& p, int64_t grid, hipStream_t s) {
    const dim3 block((pipe::NW + pipe::NCP) * WAVE);
    if (p.out_scale != 1.0f)
        hipLaunchKernelGGL((chunked_fwd_pipe<DK, DVT, 3, true>), dim3((unsigned)grid), block, 0, s, p);
    else
        hipLaunchKernelGGL((chunked_fwd_pipe<DK, DVT, 3, false>), dim3((unsigned)grid), block, 0, s, p);
    return hipGetLastError();
}

}  // namespace la
