// Chunked causal linear attention, fused phase 3, streaming kernel (gfx950)
// for chunks of 32, 64 or 128 rows, bf16 in and out, with or without the
// normaliser, with or without the bf16 residual of pre-mapped phi(k).
//
// Same mathematics as chunked_fwd_bf16 (page "attention と線形の間",
// section ②: O_c = Q_c P + tril(Q_c K_c^T) V_c with the diagonal kept, then
// P += K_c^T V_c), organised for HBM streaming.
//
// One workgroup: (head, group of chunks, tile of DVT = 64 value columns; 32 at
// feature width 256, where the state of 64 columns would not fit the
// registers), four waves, one per SIMD, in two pairs.  Pair h owns value
// columns [h DVT/2, (h+1) DVT/2):
//
//  * compute wave h touches only LDS and the matrix cores: the scores of each
//    chunk (S^T = K Q^T), the inter product Q P, the intra product tril(S) V and
//    the state update P += K^T V for its 32 columns (P in fp32 accumulators).
//    Its output rows go back into its own V columns of the LDS stage (no other
//    wave reads them).
//  * copy wave h issues half of every global access: direct-to-LDS copies
//    (global_load_lds_dwordx4) of the coming tiles of Q, K and V, and the output
//    stores (16-byte row segments read back from the stage).  A wave stalls when
//    it has 63 memory instructions in flight or the memory queue is full; those
//    stalls stay on the copy waves.
//
// The sequence is walked in tiles of TT rows (64, or 128 for chunks of 128),
// NSTAGE LDS stages of (Q, K, V) tiles (as many as fit 160 KB, at most four).
// Per tile j, after the barrier B(j) that makes tile j visible:
//   compute waves: products of tile j from stage j % NSTAGE, output into the V
//     tile of that stage;
//   copy waves: read the output of tile j - 1 from stage (j - 1) % NSTAGE,
//     refill that stage with tile j + NSTAGE - 1, wait until tile j + 1 has
//     landed, store the output rows of tile j - 1, B(j + 1).
// The wait counts only the copies of the tiles issued after tile j + 1: loads
// complete in order, so once no more than those are outstanding, tile j + 1 is
// in, whatever the order in which the stores in between complete.  The stores
// go out after the wait so that it does not hold on them.
//
// LDS tiles are row-major with the 16-byte segment index XORed with the row
// (the copy picks, per lane, which global segment lands in which LDS slot):
// 16-byte row reads and transpose reads are conflict-free.
//
// Matrix-core mapping (16x16x32 bf16, fp32 accumulate):
//   scores  S^T[key][q] += K[key][a]  Q[q][a]      A = K rows,    B = Q rows
//   inter   O^T[j][q]   += P[a][j]    Q[q][a]      A = P (regs),  B = Q rows
//   intra   O^T[j][q]   += V[key][j]  S^T[key][q]  A = V columns, B = S^T (regs)
//   update  P[a][j]     += K[key][a]  V[key][j]    A = K columns, B = V columns
// Keys are permuted inside each 32-wide k-step (lane group g holds keys
// 4g..4g+3 and 16+4g..16+4g+3): the order in which S^T comes out of the
// matrix core, so masked scores feed the intra product from registers; V and K
// column operands are transpose reads (ds_read_b64_tr_b16) with that row order.
// Features a are in natural order (lane group g holds 8g..8g+7, one 16-byte
// read per row operand); the update reads K's columns with lane c of each row
// quad pointing at column 8c (+4 for the second half), so its accumulator rows
// come out as a = 32ks + 8g + 4h + i and a packed pair (h = 0, 1) is the inter
// product's operand in natural order.  Outputs come out transposed
// (O^T = P^T Q^T + V^T tril(S)^T): a lane holds four consecutive columns of one
// row.
//
// Normaliser (page "Linear Attention / Performerの理論と実装", RNN view: the
// denominator phi(q) . sum phi(k) next to the numerator): one more 16-column
// block whose V operand is all ones.  Its state block is z in every column
// (z += K^T 1), its inter product is Q z and its intra product the row sums of
// the masked scores, so every lane ends up holding the denominator of its row
// next to the four numerators it divides.
//
// elu+1 (same page, the ELU feature map; PHI): all four waves map the Q and K
// of a landed tile in place, in LDS, so the mapped values never go through
// memory.  Each copy wave maps its share as soon as the tile has landed (before
// B(j)); each compute wave maps its share after B(j), and a second barrier
// B'(j) separates that from the products.  K rows past the end of the sequence
// are set to zero by the mapping instead of by a separate pass.  The state
// here sums
// bf16(phi(k)): the products read it rounded to bf16 anyway, so that rounding
// stays below the operand rounding of the inter product; a returned final
// state or normaliser, where it would not, is summed elsewhere with phi(k)'s
// residual (phase 1 and the scan), and the kernel then writes none.
//
// Decayed recurrence (S_t = gamma S_{t-1} + k_t^T v_t, the Retention form): row
// i of a chunk of n rows reads gamma^(i+1) P and gamma^(i-j) of key j's score,
// and the chunk enters as P <- gamma^n P + sum_j gamma^(n-1-j) k_j^T v_j.  Two
// forms compute it:
//  * direct: every score times gamma^(i-j) (per-lane powers in registers), the
//    inter product times gamma^(i+1), P times gamma^n at every update;
//  * factored: P = sigma P' with a wave-uniform sigma (a power of gamma).  With
//    c_j = gamma^(-1-j) / sigma, gamma^(i-j) = rho_i c_j for rho_i =
//    gamma^(i+1) sigma, so row i is rho_i (q_i P' + sum_{j<=i} (q_i k_j) c_j v_j)
//    and the update is P' += sum_j c_j k_j^T v_j, sigma *= gamma^n: one set of
//    weighted V operands serves the intra product and the update, the scores
//    need only the causal mask, rho_i is applied once per output (and cancels
//    in the normalised ratio), and P' is rescaled only when sigma falls below
//    2^-16.  Then c_j <= gamma^(-TT) 2^16: the host takes this form when
//    TT |log2 gamma| <= 48 (c_j and P' stay below 2^64 times their scale).
//    sigma = gamma^nr, nr the rows since the last rescale (an integer both
//    sides of the workgroup count alike), and the copy waves weight the V rows
//    of a tile in LDS as it lands (V is read only weighted), so the compute
//    waves read V as without the decay.
#pragma once

#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

enum { DECAY_NONE = 0, DECAY_DIRECT = 1, DECAY_FACTORED = 2 };
// threshold of the factored form's rescaling, and its eligibility (see above)
constexpr float kFacRescaleLog2 = -16.0f;
constexpr float kFacMaxLog2Range = 48.0f;

namespace pipe {

// Byte offset of element e of row r in a tile with NSEG 16-byte segments per
// row: segment index XOR (row mod NSEG).
template <int NSEG>
__device__ __forceinline__ int tile_off(int r, int e) {
    return r * NSEG * 16 + ((((e >> 3) ^ r) & (NSEG - 1)) << 4) + ((e & 7) << 1);
}

template <int DK, int DVT, int TT>
struct alignas(16) Stage {
    u16 q[TT * DK];
    u16 k[TT * DK];
    u16 v[TT * DVT];
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
// of the copy) is saved and restored around it.  The copy carries the
// non-temporal hint: every byte is read once per workgroup (and once more at
// most, right away, by the workgroup of the other value columns), so the
// caches need not keep it (measured 5 % faster than without).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds)
        : "memory");
}

// Eight bf16 values times per-element weights (fp32 math, rounded to nearest
// even), and eight floats packed to bf16.
__device__ __forceinline__ bf16x8 scale_bf16x8(const bf16x8& v, const float (&w)[8]) {
    const uint4 u = __builtin_bit_cast(uint4, v);
    const uint32_t x[4] = {u.x, u.y, u.z, u.w};
    uint32_t y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        y[j] = pack2_bf16(__uint_as_float(x[j] << 16) * w[2 * j], __uint_as_float(x[j] & 0xFFFF0000u) * w[2 * j + 1]);
    return as_bf16x8(make_uint4(y[0], y[1], y[2], y[3]));
}
__device__ __forceinline__ uint4 scale_bf16x8_by(const uint4& u, float w) {
    const uint32_t x[4] = {u.x, u.y, u.z, u.w};
    uint32_t y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = pack2_bf16(__uint_as_float(x[j] << 16) * w, __uint_as_float(x[j] & 0xFFFF0000u) * w);
    return make_uint4(y[0], y[1], y[2], y[3]);
}
__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&w)[8]) {
    return as_bf16x8(make_uint4(pack2_bf16(w[0], w[1]), pack2_bf16(w[2], w[3]), pack2_bf16(w[4], w[5]),
                                pack2_bf16(w[6], w[7])));
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

template <int I>
using ic = std::integral_constant<int, I>;

// Position of key j (0..63) in a row of an operand whose k index runs in the
// permuted order of packed accumulator pairs and of column operands: inside
// each 32-key step, lane group g' holds keys 4g'..4g'+3 (elements 0..3) and
// 16+4g'..16+4g'+3 (elements 4..7).
__device__ __forceinline__ int perm_pos(int j) {
    const int jj = j & 31;
    return (j & 32) + (jj < 16 ? 8 * (jj >> 2) + (jj & 3) : 8 * ((jj - 16) >> 2) + 4 + (jj & 3));
}

// The elu+1 pass over a landed tile of the streaming kernels.  A tile's Q (or
// K) is 2 NC blocks of 64 16-byte pieces; copy wave h copies blocks
// h NC .. h NC + NC - 1 of each tensor it moves.  The pieces of pair h are a
// list: entry j is block h NC + (j mod NC) of the first tensor (j < NC) or of
// the second.  A wave waits only for its own copies, so the entries a copy
// wave maps before the barrier that follows every copy wave's wait must be
// its own; the compute waves map after that barrier.  Both kernels take the
// block of an entry from here, and the checks below run at compile time for
// every instantiation.
template <int NC>
struct PieceList {
    static constexpr bool first(int j) { return j < NC; }
    static constexpr int block(int h, int j) { return h * NC + (j < NC ? j : j - NC); }
    static constexpr bool copied_by(int h, int j) { return block(h, j) >= h * NC && block(h, j) < h * NC + NC; }
};

// Shares of a list of NE entries per pair (NE = 2 NC with two tensors, NC with
// one): entries [0, EARLY) are mapped by the copy wave before the barrier,
// the rest after it (by the copy wave or the compute wave).  True when the two
// pairs' lists together name every block of every tensor exactly once and the
// early entries are the copy wave's own.
template <int NC, int NE, int EARLY>
constexpr bool piece_shares_ok() {
    if (EARLY < 0 || EARLY > NE || (NE != NC && NE != 2 * NC)) return false;
    int seen[2][2 * NC] = {};
    for (int h = 0; h < 2; ++h)
        for (int j = 0; j < NE; ++j) {
            seen[PieceList<NC>::first(j) ? 0 : 1][PieceList<NC>::block(h, j)] += 1;
            if (j < EARLY && !PieceList<NC>::copied_by(h, j)) return false;
        }
    for (int t = 0; t < NE / NC; ++t)
        for (int b = 0; b < 2 * NC; ++b)
            if (seen[t][b] != 1) return false;
    return true;
}

}  // namespace pipe

template <int DK, int DVT, int CH, bool SCALED, bool NORM, bool PHI, int DECAY>
__global__ __launch_bounds__(4 * WAVE) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunked_fwd_pipe(FwdParams p) {
    using namespace pipe;
    constexpr int TT = CH > 64 ? CH : 64;          // rows per tile
    // chunks of 128 rows without the decay: the two compute waves split the
    // tile's score blocks and exchange them (20 operand fragments of 1 KB)
    // through its Q slot, the fragments past the slot's end through XF more
    // KB of their own (two more barriers per tile, SYNC1 and SYNC2)
    // (not with elu+1 mapped in the kernel: there the two barriers hold back
    // the copy waves' mapping of the next tile, measured 7 % slower)
    constexpr bool SHARE = CH == 128 && DECAY == DECAY_NONE && !PHI;
    constexpr int QF = SHARE ? (TT * DK * 2 / 1024 < 20 ? TT * DK * 2 / 1024 : 20) : 0;  // fragments in the Q slot
    constexpr int XF = SHARE ? 20 - QF : 0;
    constexpr int NFIT = (int)((160 * 1024 - XF * 1024) / sizeof(Stage<DK, DVT, TT>));
    constexpr int NSTAGE = NFIT < 4 ? NFIT : 4;    // LDS stages
    constexpr int CPW = DVT / 32;                  // 16-column blocks per pair
    constexpr int NCB = CPW + (NORM ? 1 : 0);      // + the denominator block
    constexpr int NKA = DK / 32;                   // k-steps over the feature index
    constexpr int QSEG = DK / 8, VSEG = DVT / 8;
    constexpr int NCQ = TT * QSEG / WAVE / 2;      // copy instructions per tile and copy wave, Q (and K)
    constexpr int NCV = TT * VSEG / WAVE / 2;      // the same for V (and for the output stores)
    constexpr int NL = 2 * NCQ + NCV;              // copy instructions per tile and copy wave
    constexpr int RPV = WAVE / VSEG;               // output rows per store instruction
    constexpr bool DIR = DECAY == DECAY_DIRECT, FAC = DECAY == DECAY_FACTORED;
    static_assert(DVT == 64 || (DVT == 32 && DK == 256), "tile of 64 value columns (32 at feature width 256)");
    static_assert(CH == 32 || CH == 64 || CH == 128, "chunks of 32, 64 or 128 rows");
    static_assert(DK == 64 || DK == 128 || DK == 256, "feature width 64, 128 or 256");
    static_assert(NSTAGE >= 2, "two stages at least");
    static_assert((NSTAGE - 2) * NL + NCQ + NCV < 64, "vmcnt range");
    static_assert(NSTAGE * (int)sizeof(Stage<DK, DVT, TT>) + XF * 1024 <= 160 * 1024, "LDS");
    typedef Stage<DK, DVT, TT> StageT;

    __shared__ StageT st[NSTAGE];
    __shared__ __attribute__((aligned(16))) char xfrag[XF > 0 ? XF * 1024 : 16];

    const int tid = threadIdx.x;
    const int wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const bool copier = wave >= 2;                               // wave-uniform
    const int h = __builtin_amdgcn_readfirstlane(wave & 1);      // pair (wave-uniform)
    const int colw = h * CPW * 16;                               // first column of the pair
    // factored decay: rows after which the state is rescaled (sigma >= 2^-16)
    const int nr_max = p.log2_gamma < 0.f ? (int)fminf(-kFacRescaleLog2 / -p.log2_gamma, 1e9f) : 1 << 30;

    const int w = work_index(p.xcd_remap);
    const int jt = w % p.n_dvt;
    const int grp = (w / p.n_dvt) % p.n_groups;
    const int64_t bh = w / (p.n_dvt * p.n_groups);
    const int col0 = jt * DVT;

    const int64_t L = p.L;
    const int dv = p.dv;
    // This group's chunks and the tiles that hold them (for chunks of 32 the
    // plan keeps an even number of chunks per group, so groups start on a tile).
    const int64_t n_chunks = (L + CH - 1) / CH;
    const int64_t c_begin = (int64_t)grp * p.G;
    const int64_t c_end = c_begin + p.G < n_chunks ? c_begin + p.G : n_chunks;
    const int64_t r_end = c_end * CH < L ? c_end * CH : L;
    const int64_t t_begin = c_begin * CH / TT;
    const int64_t t_end = (r_end + TT - 1) / TT;
    const int64_t n_tiles = (L + TT - 1) / TT;

    // rows of tile t that exist
    auto valid_rows = [&](int64_t t) -> int { return (int)(L - t * TT < TT ? L - t * TT : TT); };

    // rows past the end of the sequence: zero their K rows (scores and state
    // contributions vanish; their Q rows produce outputs that are not stored)
    auto zero_tail = [&](StageT& s, int valid) __attribute__((always_inline)) {
        const int n = (TT - valid) * QSEG;
        uint4* kk = reinterpret_cast<uint4*>(s.k + valid * DK);
        for (int i = tid; i < n; i += 4 * WAVE) kk[i] = make_uint4(0, 0, 0, 0);
    };

    // elu+1 of a landed tile's Q and K in place.  Each tile is NP = 2 NCQ
    // blocks of 64 16-byte pieces, and lane l of a block maps its piece l.
    // Copy wave h copies (and waits for) Q blocks h NCQ .. h NCQ + NCQ - 1 and
    // the same K blocks: the list of pair h, Q's then K's, j = 0 .. NP - 1.
    // Copy wave h maps the first NPK of that list as soon as its copies have
    // landed (only its own copies: the other copy wave's may still be in
    // flight), compute wave h the other NPC after B(j).  The compute waves take
    // half with 64-row tiles and a quarter with 128-row tiles, whose products
    // leave them less time, and an eighth with the decay, whose products leave
    // them the least (the shares that measured fastest).
    constexpr int NP = 2 * NCQ;
    constexpr int NPC = DECAY ? NP / 8 : (TT > 64 && !SHARE ? NP / 4 : NP / 2), NPK = NP - NPC;
    constexpr bool MAP2 = PHI && NPC > 0;  // the compute waves map too
    static_assert(!PHI || piece_shares_ok<NCQ, NP, NPK>(),
                  "elu+1 shares: a copy wave maps only pieces it copied before the barrier; every piece once");
    auto phi_blocks = [&](StageT& s, int valid, auto j0_, auto count) __attribute__((always_inline)) {
        constexpr int J0 = decltype(j0_)::value, N = decltype(count)::value;
        // four pieces in flight at a time (bounded registers)
#pragma unroll
        for (int i0 = 0; i0 < N; i0 += 4) {
            uint4 x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = J0 + i0 + i;
                const int slot = PieceList<NCQ>::block(h, j) * WAVE + lane;
                if (i0 + i < N) x[i] = *reinterpret_cast<const uint4*>((j < NCQ ? s.q : s.k) + slot * 8);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = J0 + i0 + i;
                const int slot = PieceList<NCQ>::block(h, j) * WAVE + lane;
                if (i0 + i < N) {
                    const bool live = j < NCQ || slot / QSEG < valid;  // K rows past the end become zero
                    *reinterpret_cast<uint4*>((j < NCQ ? s.q : s.k) + slot * 8) =
                        live ? elu1_bf16x8(x[i], p.in_scale) : make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    // this wave's share of the mapping of a landed tile (a whole tile without
    // the per-piece row test, so that the reads are not each sunk into a branch)
    auto phi_share = [&](StageT& s, int valid) __attribute__((always_inline)) {
        if (copier) {
            if (valid == TT)
                phi_blocks(s, TT, ic<0>{}, ic<NPK>{});
            else
                phi_blocks(s, valid, ic<0>{}, ic<NPK>{});
        } else {
            if (valid == TT)
                phi_blocks(s, TT, ic<NPK>{}, ic<NPC>{});
            else
                phi_blocks(s, valid, ic<NPK>{}, ic<NPC>{});
        }
    };

    // factored decay: this copy wave's own V slots of a landed tile (V
    // instruction i, lane l: slot (h NCV + i) WAVE + l, row slot / VSEG) times
    // c_j = gamma^(-(1 + j + nr)), j the row within its chunk and gamma^nr the
    // state scale at the chunk's start (chunks of 32: the second chunk of the
    // tile starts after the first one's rows)
    auto weigh_v_tile = [&](StageT& s, int valid, int nr) __attribute__((always_inline)) {
        const int na = valid < 32 ? valid : 32;
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int slot = (h * NCV + i) * WAVE + lane;
            const int r = slot / VSEG;
            const int e = CH == 32 && r >= 32 ? r - 32 + 1 + nr + na : r + 1 + nr;
            uint4* x = reinterpret_cast<uint4*>(s.v) + slot;
            *x = scale_bf16x8_by(*x, __builtin_amdgcn_exp2f(-(float)e * p.log2_gamma));
        }
    };
    // the copy side's count of rows since the rescale, advanced past a tile
    auto next_nr = [&](int nr, int64_t t) __attribute__((always_inline)) {
        const int n = nr > nr_max ? 0 : nr;
        return n + valid_rows(t);
    };

    if (copier) {
        // ================= copy wave h =================
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u16* qh = p.q + bh * L * DK;
        const u16* kh = p.k + bh * L * DK;
        const u16* vh = p.v + bh * L * dv + col0;
        // Lane l of copy instruction b lands in LDS slot 64b + l = (row,
        // physical segment) = (slot / NSEG, slot % NSEG), which holds the
        // global segment (physical ^ row) of that row.
        auto issue = [&](int64_t t, StageT& s) __attribute__((always_inline)) {
            const int64_t r0 = t * TT;
            const int last = (int)(L - 1 - r0);  // rows past it are clamped to it
            const u16* qb_ = qh + r0 * DK;
            const u16* kb_ = kh + r0 * DK;
            const u16* vb_ = vh + r0 * dv;
            const uint32_t lq = lds_addr(s.q), lk = lds_addr(s.k), lv = lds_addr(s.v);
            auto qk_off = [&](int i) __attribute__((always_inline)) {
                const int b = h * NCQ + i;  // copy instruction within the tile
                const int slot = b * WAVE + lane;
                const int r = slot / QSEG, seg = (slot % QSEG) ^ (r & (QSEG - 1));
                return (uint32_t)(((r < last ? r : last) * DK + seg * 8) * 2);
            };
#pragma unroll
            for (int i = 0; i < NCQ; ++i) dma16(qb_, qk_off(i), lq + (h * NCQ + i) * WAVE * 16);
#pragma unroll
            for (int i = 0; i < NCQ; ++i) dma16(kb_, qk_off(i), lk + (h * NCQ + i) * WAVE * 16);
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int b = h * NCV + i;
                const int slot = b * WAVE + lane;
                const int r = slot / VSEG, seg = (slot % VSEG) ^ (r & (VSEG - 1));
                dma16(vb_, (uint32_t)(((r < last ? r : last) * dv + seg * 8) * 2), lv + b * WAVE * 16);
            }
        };
        // Output rows of a tile sit in the V tile of its stage: instruction i,
        // lane l covers row (h * NCV + i) * RPV + l / VSEG, segment l % VSEG.
        // read_out takes them into registers (and waits for the reads, so the
        // stage can be refilled); store_out writes them to rows of tile t.
        auto read_out = [&](const StageT& from, u32x4 (&ob)[NCV]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int r = (h * NCV + i) * RPV + lane / VSEG, seg = lane % VSEG;
                ob[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(from.v) +
                                                        tile_off<VSEG>(r, seg * 8));
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        };
        auto store_out = [&](int64_t t, const u32x4 (&ob)[NCV]) __attribute__((always_inline)) {
            const int valid = valid_rows(t);
            u16* o = reinterpret_cast<u16*>(p.o) + (bh * L + t * TT) * dv + col0;
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const int r = (h * NCV + i) * RPV + lane / VSEG, seg = lane % VSEG;
                if (r < valid) __builtin_nontemporal_store(ob[i], reinterpret_cast<u32x4*>(o + (int64_t)r * dv + seg * 8));
            }
        };

        // wait until this wave's copies of a tile have landed, given that the
        // copies of `after` more tiles were issued after them (the wait counts
        // are immediates, so each is picked by a branch)
        auto land = [&](int after) __attribute__((always_inline)) {
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
        // tiles issued after tile t while t is the oldest in flight
        auto after_of = [&](int64_t t) -> int {
            const int64_t newest = t + NSTAGE - 2 < t_end - 1 ? t + NSTAGE - 2 : t_end - 1;
            return (int)(newest - t);
        };

#pragma unroll
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (t_begin + s0 < t_end) issue(t_begin + s0, st[s0]);
        land(after_of(t_begin));
        if constexpr (PHI) phi_share(st[0], valid_rows(t_begin));
        int nr_c = 0;  // factored decay: rows since the rescale before tile t
        if constexpr (FAC) weigh_v_tile(st[0], valid_rows(t_begin), 0);

        // The copy side walks the stages with a run-time index (its accesses
        // take computed addresses anyway), so its code appears once.
        int si = 0;  // stage of tile t
        for (int64_t t = t_begin; t < t_end; ++t) {
            const int sp = si == 0 ? NSTAGE - 1 : si - 1;  // stage of tile t - 1
            const int sn = si == NSTAGE - 1 ? 0 : si + 1;  // stage of tile t + 1
            __syncthreads();  // B(t)
            if (!PHI && valid_rows(t) < TT) {
                zero_tail(st[si], valid_rows(t));
                __syncthreads();
            }
            // the output of tile t - 1 leaves stage sp, which takes tile
            // t + NSTAGE - 1; the stores go out after the wait for tile t + 1,
            // so that the wait does not hold on them
            u32x4 ob[NCV];
            if (t > t_begin) read_out(st[sp], ob);
            if (t + NSTAGE - 1 < t_end) issue(t + NSTAGE - 1, st[sp]);
            if constexpr (MAP2) __syncthreads();  // B'(t): the compute waves have mapped their share of tile t
            if constexpr (SHARE) {
                __syncthreads();  // SYNC1(t): the compute waves have read Q
                __syncthreads();  // SYNC2(t): the score operands are in the Q slot
            }
            // tile t + 1 must have landed (and this wave's share of it been
            // mapped) before B(t + 1); the newest tile issued is now
            // t + NSTAGE - 1 (or the last one)
            if (t + 1 < t_end) {
                land(after_of(t + 1));
                if constexpr (PHI) phi_share(st[sn], valid_rows(t + 1));
                if constexpr (FAC) {
                    nr_c = next_nr(nr_c, t);
                    weigh_v_tile(st[sn], valid_rows(t + 1), nr_c > nr_max ? 0 : nr_c);
                }
            }
            if (t > t_begin) store_out(t - 1, ob);
            si = sn;
        }
        __syncthreads();  // the last tile's output is in its stage
        {
            const int sl = si == 0 ? NSTAGE - 1 : si - 1;
            u32x4 ob[NCV];
            read_out(st[sl], ob);
            store_out(t_end - 1, ob);
        }
        return;
    }

    // ================= compute wave h =================
    // state P: P[c][ks][hf] lane (l16, g) element i = P[a = 32ks + 8g + 4hf + i][j = colw + 16c + l16];
    // with the normaliser, block c = CPW holds z[a] in every column
    f32x4 P[NCB][NKA][2];
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) P[c][ks][0] = P[c][ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.P0 != nullptr && grp > 0) {
        const int64_t slot = (bh * p.n_groups + grp) * (int64_t)(p.p0_sub > 1 ? p.p0_sub : 1);
        const float* P0 = p.P0 + (slot * DK) * (int64_t)dv + col0 + colw + l16;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        P[c][ks][hf][i] = P0[(int64_t)(32 * ks + 8 * g + 4 * hf + i) * dv + c * 16];
        if constexpr (NORM) {
            const float* z0 = p.z0 + slot * DK;
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) P[CPW][ks][hf][i] = z0[32 * ks + 8 * g + 4 * hf + i];
        }
    }
    // V operand of the denominator block: all ones (bf16 1.0)
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    const float osc = p.out_scale;
    const int c4 = 4 * (lane & 3), c8 = 8 * (lane & 3);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // Decay (the decayed recurrence S_t = gamma S_{t-1} + k_t^T v_t): powers of
    // gamma as exp2(e log2 gamma) (v_exp_f32), 0 for negative e (masked).
    //   fd[D][i] = gamma^(16 D + l16 - 4g - i): score of query 16 qb + l16 and key
    //             16 kb + 4g + i of the same tile, D = qb - kb (the cross block
    //             of 128-row chunks reaches D = 7);
    //   fin[qb] = gamma^(16 qb + l16 + 1): the inter read of that query row at
    //             the start of its chunk (fin64: 64 rows further on).
    const float lg = p.log2_gamma;
    auto gpow = [&](int e) __attribute__((always_inline)) {
        return e < 0 ? 0.f : __builtin_amdgcn_exp2f((float)e * lg);
    };
    constexpr int ND = CH == 128 ? 8 : 4;
    float fd[DIR ? ND : 1][4], fin[4], fin64[4];
    if constexpr (DIR) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) fd[d][i] = gpow(16 * d + l16 - 4 * g - i);
    }
    if constexpr (DECAY) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
            fin[qb] = gpow(16 * qb + l16 + 1);
            fin64[qb] = gpow(64 + 16 * qb + l16 + 1);
        }
    }
    // inter parts of query blocks [B0, B1) read the carried state from the start
    // of their chunk: scale them before the intra parts are added
    auto decay_inter = [&](f32x4 (&O)[NCB][4], const float (&f)[4], int b0, int b1, int shift)
        __attribute__((always_inline)) {
        if constexpr (DIR) {
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
                    if (qb >= b0 && qb < b1) O[c][qb] *= f[qb - shift];
        }
    };

    // Scores of the lower-triangle window of query blocks Q0 + qb and key blocks
    // K0 + kb, kb <= qb < 4 (10 blocks, index qb(qb+1)/2 + kb; with HALVES only
    // the blocks inside each 32-row half), masked on the diagonal, and the
    // inter product with the packed state for the query blocks in INTER (a bit
    // mask); feature steps one at a time, the next step's operands loaded ahead.
    auto tri_window = [&](const StageT& s, auto q0c, auto k0c, auto halvesc, auto interc, f32x4 (&S)[10],
                          f32x4 (&O)[NCB][4], const bf16x8 (&pst)[NCB][NKA]) __attribute__((always_inline)) {
        constexpr int Q0 = decltype(q0c)::value, K0 = decltype(k0c)::value;
        constexpr bool HALVES = decltype(halvesc)::value != 0;
        constexpr int INTER = decltype(interc)::value;
        bf16x8 qa[2][4], ka[2][4];
        auto load = [&](int ks, bf16x8 (&q_)[4], bf16x8 (&k_)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                q_[b] = row_op<QSEG>(s.q, (Q0 + b) * 16 + l16, ks * 32, g);
                k_[b] = row_op<QSEG>(s.k, (K0 + b) * 16 + l16, ks * 32, g);
            }
        };
#pragma unroll
        for (int i = 0; i < 10; ++i) S[i] = zero4;
        load(0, qa[0], ka[0]);
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) {
            if (ks + 1 < NKA) load(ks + 1, qa[(ks + 1) & 1], ka[(ks + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int kb = 0; kb <= qb; ++kb)
                    if (!HALVES || (qb >> 1) == (kb >> 1))
                        S[qb * (qb + 1) / 2 + kb] =
                            mfma_bf16(ka[ks & 1][kb], qa[ks & 1][qb], S[qb * (qb + 1) / 2 + kb]);
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
                    if ((INTER >> qb) & 1) O[c][qb] = mfma_bf16(pst[c][ks], qa[ks & 1][qb], O[c][qb]);
        }
        if constexpr (DIR) {
            // every score times gamma^(query - key); 0 above the diagonal
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int kb = 0; kb <= qb; ++kb)
                    if (!HALVES || (qb >> 1) == (kb >> 1))
#pragma unroll
                        for (int i = 0; i < 4; ++i) S[qb * (qb + 1) / 2 + kb][i] *= fd[qb - kb][i];
        } else {
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i > l16) S[qb * (qb + 1) / 2 + qb][i] = 0.f;
        }
    };

    // intra product of a window: query blocks qb < 4 of O against the key steps
    // kk <= qb / 2 of its own 64 keys (V key rows 32 * (KK0 + kk))
    auto tri_intra_v = [&](const bf16x8 (&vb)[NCB][2], const f32x4 (&S)[10], f32x4 (&O)[NCB][4])
        __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
            for (int kk = 0; kk <= qb / 2; ++kk) {
                const f32x4 s1 = 2 * kk + 1 <= qb ? S[qb * (qb + 1) / 2 + 2 * kk + 1] : zero4;
                const bf16x8 sb = pack_acc_bf16(S[qb * (qb + 1) / 2 + 2 * kk], s1);
#pragma unroll
                for (int c = 0; c < NCB; ++c) O[c][qb] = mfma_bf16(vb[c][kk], sb, O[c][qb]);
            }
    };
    // V column operands of key steps KK0 .. KK0 + NK - 1 (the ones of the
    // denominator block last)
    auto load_v = [&](const StageT& s, auto kk0c, auto nkc, bf16x8 (&vb)[NCB][decltype(nkc)::value])
        __attribute__((always_inline)) {
        constexpr int KK0 = decltype(kk0c)::value, NK = decltype(nkc)::value;
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
                vb[c][kk] = c < CPW ? col_op<VSEG>(s.v, (KK0 + kk) * 32, colw + c * 16 + c4, lane) : ones;
    };
    auto tri_intra = [&](const StageT& s, auto kk0c, const f32x4 (&S)[10], f32x4 (&O)[NCB][4])
        __attribute__((always_inline)) {
        bf16x8 vb[NCB][2];
        load_v(s, kk0c, ic<2>{}, vb);
        tri_intra_v(vb, S, O);
    };
    // the same operands with key j (local to a chunk of n_rows keys starting at
    // tile row kbase) weighted by exp2((n_rows - 1 - j) lg - shift), 0 for
    // j >= n_rows: one power per run of four keys, taken at the run's last key
    // before n_rows (so that no power exceeds the first key's), the earlier
    // keys by multiplying by gamma.  Operand element e holds key
    // 32 (KK0 + kk) + 4g + e (e < 4), + 16 (e >= 4).
    auto load_v_weighted = [&](const StageT& s, auto kk0c, auto nkc, int n_rows, int kbase, float shift,
                               bf16x8 (&vb)[NCB][decltype(nkc)::value]) __attribute__((always_inline)) {
        constexpr int KK0 = decltype(kk0c)::value, NK = decltype(nkc)::value;
        load_v(s, kk0c, nkc, vb);
        const float gam = __builtin_amdgcn_exp2f(lg);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            float w[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int key3 = 32 * (KK0 + kk) + 16 * hh + 4 * g + 3 - kbase;
                const int top = key3 < n_rows - 1 ? key3 : n_rows - 1;
                float wk = __builtin_amdgcn_exp2f((float)(n_rows - 1 - top) * lg - shift);
#pragma unroll
                for (int j = 3; j >= 0; --j) {
                    const bool live = key3 - 3 + j < n_rows;
                    w[4 * hh + j] = live ? wk : 0.f;
                    wk = live ? wk * gam : wk;
                }
            }
#pragma unroll
            for (int c = 0; c < NCB; ++c) vb[c][kk] = c < CPW ? scale_bf16x8(vb[c][kk], w) : pack_bf16x8(w);
        }
    };
    // P += K^T V over key steps KK0 .. KK0 + NK - 1 with the given V operands,
    // K column operands one (ks, hf) step ahead
    auto update_v = [&](const StageT& s, auto kk0c, const auto& vb) __attribute__((always_inline)) {
        constexpr int KK0 = decltype(kk0c)::value;
        constexpr int NK = sizeof(vb[0]) / sizeof(vb[0][0]);
        bf16x8 kc[2][NK];
        auto load_kc = [&](int ks, int hf, bf16x8 (&k_)[NK]) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) k_[kk] = col_op<QSEG>(s.k, (KK0 + kk) * 32, ks * 32 + c8 + 4 * hf, lane);
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

    // state update with the key steps KK0 .. KK0 + NK - 1 of the tile.  With
    // the direct decay the chunk (keys from row kbase, n_rows of them) enters as
    // P <- gamma^n P + sum_j gamma^(n-1-j) k_j^T v_j: the state is scaled and
    // each key's V operand (the ones of the denominator block too) weighted.
    auto update = [&](const StageT& s, auto kk0c, auto nkc, int n_rows, int kbase) __attribute__((always_inline)) {
        constexpr int NK = decltype(nkc)::value;
        bf16x8 vb[NCB][NK];
        if constexpr (DIR) {
            load_v_weighted(s, kk0c, nkc, n_rows, kbase, 0.f, vb);
            const float gn = __builtin_amdgcn_exp2f((float)n_rows * lg);
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int ks = 0; ks < NKA; ++ks) {
                    P[c][ks][0] *= gn;
                    P[c][ks][1] *= gn;
                }
        } else {
            load_v(s, kk0c, nkc, vb);
        }
        update_v(s, kk0c, vb);
    };

    auto pack_state = [&](bf16x8 (&pst)[NCB][NKA]) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks) pst[c][ks] = pack_acc_bf16(P[c][ks][0], P[c][ks][1]);
    };

    // inter product of query blocks Q0 + b, b in [B0, B0 + 2), reading Q again
    auto inter2 = [&](const StageT& s, auto q0c, auto b0c, f32x4 (&O)[NCB][4], const bf16x8 (&pst)[NCB][NKA])
        __attribute__((always_inline)) {
        constexpr int Q0 = decltype(q0c)::value, B0 = decltype(b0c)::value;
        bf16x8 qa[NKA][2];
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
            for (int b = 0; b < 2; ++b) qa[ks][b] = row_op<QSEG>(s.q, (Q0 + B0 + b) * 16 + l16, ks * 32, g);
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int b = 0; b < 2; ++b) O[c][B0 + b] = mfma_bf16(pst[c][ks], qa[ks][b], O[c][B0 + b]);
    };

    // output rows of query blocks Q0 + qb into this wave's V columns (after its
    // last V read of the tile, in program order)
    // (factored decay without the normaliser: times the row factor rf[qb], which
    // then holds the output scale too)
    auto write_out = [&](StageT& s, auto q0c, f32x4 (&O)[NCB][4], const float (&rf)[4])
        __attribute__((always_inline)) {
        constexpr int Q0 = decltype(q0c)::value;
        // the denominator block holds the row's denominator in every column:
        // one reciprocal (v_rcp_f32, about 1 ulp) per row and lane
        float rden[4];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) rden[qb] = NORM ? __builtin_amdgcn_rcpf(O[NCB - 1][qb][0]) : 1.0f;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                f32x4 o = O[c][qb];
                if constexpr (NORM) o *= rden[qb];
                if constexpr (FAC && !NORM)
                    o *= rf[qb];
                else if (SCALED)
                    o *= osc;
                *reinterpret_cast<uint2*>(reinterpret_cast<char*>(s.v) +
                                          tile_off<VSEG>((Q0 + qb) * 16 + l16, colw + c * 16 + 4 * g)) =
                    make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
            }
    };

    auto zero_o = [&](f32x4 (&O)[NCB][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) O[c][qb] = zero4;
    };

    // ---- factored decay: P = gamma^nr P' (nr rows since the last rescale,
    // wave-uniform); V arrives weighted from the copy waves
    int nr = 0;
    const float one4[4] = {1.f, 1.f, 1.f, 1.f};
    // row factors rho = gamma^(row + 1 + nrc) (times the output scale) of query
    // blocks whose chunk starts at the state gamma^nrc P'
    auto row_factors = [&](const float (&f)[4], int nrc, float (&rf)[4]) __attribute__((always_inline)) {
        const float sg = __builtin_amdgcn_exp2f((float)nrc * lg) * (SCALED ? osc : 1.f);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) rf[qb] = f[qb] * sg;
    };
    // V operands of key steps KK0 .. KK0 + NK - 1 (weighted in LDS); with the
    // normaliser, the denominator block's operand holds the weights c_j =
    // gamma^(-(1 + j + nrc)) of keys j (from tile row kbase), one power per run
    // of four keys, the earlier keys by multiplying by gamma
    auto load_v_fac = [&](const StageT& s, auto kk0c, auto nkc, int kbase, int nrc,
                          bf16x8 (&vb)[NCB][decltype(nkc)::value]) __attribute__((always_inline)) {
        constexpr int KK0 = decltype(kk0c)::value, NK = decltype(nkc)::value;
        load_v(s, kk0c, nkc, vb);
        if constexpr (NORM) {
            const float gam = __builtin_amdgcn_exp2f(lg);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                float w[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int key3 = 32 * (KK0 + kk) + 16 * hh + 4 * g + 3 - kbase;
                    float wk = __builtin_amdgcn_exp2f(-(float)(1 + key3 + nrc) * lg);
#pragma unroll
                    for (int j = 3; j >= 0; --j) {
                        w[4 * hh + j] = wk;
                        wk *= gam;
                    }
                }
                vb[CPW][kk] = pack_bf16x8(w);
            }
        }
    };
    auto compute_fac = [&](StageT& s, int valid) __attribute__((always_inline)) {
        if (nr > nr_max) {
            const float f = __builtin_amdgcn_exp2f((float)nr * lg);
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int ks = 0; ks < NKA; ++ks) {
                    P[c][ks][0] *= f;
                    P[c][ks][1] *= f;
                }
            nr = 0;
        }
        bf16x8 pst[NCB][NKA];
        pack_state(pst);
        if constexpr (CH == 64) {
            f32x4 S[10], O[NCB][4];
            zero_o(O);
            tri_window(s, ic<0>{}, ic<0>{}, ic<0>{}, ic<15>{}, S, O, pst);
            bf16x8 vb[NCB][2];
            load_v_fac(s, ic<0>{}, ic<2>{}, 0, nr, vb);
            tri_intra_v(vb, S, O);
            update_v(s, ic<0>{}, vb);
            float rf[4];
            if constexpr (!NORM) row_factors(fin, nr, rf);
            write_out(s, ic<0>{}, O, rf);
            nr += valid;
        } else if constexpr (CH == 32) {
            // chunk A (rows 0..31), then chunk B (rows 32..63) from A's state
            const int na = valid < 32 ? valid : 32, nb = valid > 32 ? valid - 32 : 0;
            f32x4 S[10], O[NCB][4];
            zero_o(O);
            tri_window(s, ic<0>{}, ic<0>{}, ic<1>{}, ic<3>{}, S, O, pst);
            bf16x8 va[NCB][1];
            load_v_fac(s, ic<0>{}, ic<1>{}, 0, nr, va);
            update_v(s, ic<0>{}, va);
            {
                const bf16x8 s0 = pack_acc_bf16(S[0], zero4);
                const bf16x8 s1 = pack_acc_bf16(S[1], S[2]);
#pragma unroll
                for (int c = 0; c < NCB; ++c) {
                    O[c][0] = mfma_bf16(va[c][0], s0, O[c][0]);
                    O[c][1] = mfma_bf16(va[c][0], s1, O[c][1]);
                }
            }
            pack_state(pst);
            inter2(s, ic<0>{}, ic<2>{}, O, pst);
            bf16x8 vb[NCB][1];
            load_v_fac(s, ic<1>{}, ic<1>{}, 32, nr + na, vb);
            update_v(s, ic<1>{}, vb);
            {
                const bf16x8 s2 = pack_acc_bf16(S[5], zero4);
                const bf16x8 s3 = pack_acc_bf16(S[8], S[9]);
#pragma unroll
                for (int c = 0; c < NCB; ++c) {
                    O[c][2] = mfma_bf16(vb[c][0], s2, O[c][2]);
                    O[c][3] = mfma_bf16(vb[c][0], s3, O[c][3]);
                }
            }
            float rf[4];
            if constexpr (!NORM) {
                float ra[4], rb[4];
                row_factors(fin, nr, ra);
                row_factors(fin, nr + na, rb);
                rf[0] = ra[0];
                rf[1] = ra[1];
                rf[2] = rb[0];
                rf[3] = rb[1];
            }
            write_out(s, ic<0>{}, O, rf);
            nr += na + nb;
        } else {
            // query rows 0..63: own keys; rows 64..127: keys 0..63 (whole block)
            // and own keys; the V operands of keys 0..63 serve the intra product
            // of rows 0..63, the cross block and their update, then keys 64..127
            f32x4 Ob[NCB][4];
            zero_o(Ob);
            {
                f32x4 S[10], Oa[NCB][4];
                zero_o(Oa);
                tri_window(s, ic<0>{}, ic<0>{}, ic<0>{}, ic<15>{}, S, Oa, pst);
                bf16x8 vb[NCB][2];
                load_v_fac(s, ic<0>{}, ic<2>{}, 0, nr, vb);
                tri_intra_v(vb, S, Oa);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    f32x4 X[4][2];
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb) X[qb][0] = X[qb][1] = zero4;
                    bf16x8 qa[2][4], ka[2][2];
                    auto load = [&](int ks, bf16x8 (&q_)[4], bf16x8 (&k_)[2]) __attribute__((always_inline)) {
#pragma unroll
                        for (int b = 0; b < 4; ++b) q_[b] = row_op<QSEG>(s.q, (4 + b) * 16 + l16, ks * 32, g);
#pragma unroll
                        for (int b = 0; b < 2; ++b) k_[b] = row_op<QSEG>(s.k, (2 * kk + b) * 16 + l16, ks * 32, g);
                    };
                    load(0, qa[0], ka[0]);
#pragma unroll
                    for (int ks = 0; ks < NKA; ++ks) {
                        if (ks + 1 < NKA) load(ks + 1, qa[(ks + 1) & 1], ka[(ks + 1) & 1]);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                            for (int b = 0; b < 2; ++b)
                                X[qb][b] = mfma_bf16(ka[ks & 1][b], qa[ks & 1][qb], X[qb][b]);
                    }
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb) {
                        const bf16x8 xb = pack_acc_bf16(X[qb][0], X[qb][1]);
#pragma unroll
                        for (int c = 0; c < NCB; ++c) Ob[c][qb] = mfma_bf16(vb[c][kk], xb, Ob[c][qb]);
                    }
                }
                update_v(s, ic<0>{}, vb);
                float rf[4];
                if constexpr (!NORM) row_factors(fin, nr, rf);
                write_out(s, ic<0>{}, Oa, rf);  // V rows 0..63 are no longer read
            }
            {
                f32x4 S[10];
                tri_window(s, ic<4>{}, ic<4>{}, ic<0>{}, ic<15>{}, S, Ob, pst);
                bf16x8 vb[NCB][2];
                load_v_fac(s, ic<2>{}, ic<2>{}, 0, nr, vb);
                tri_intra_v(vb, S, Ob);
                update_v(s, ic<2>{}, vb);
                float rf[4];
                if constexpr (!NORM) row_factors(fin64, nr, rf);
                write_out(s, ic<4>{}, Ob, rf);
            }
            nr += valid;
        }
    };

    // ---- one tile's products
    auto compute = [&](StageT& s, int valid) __attribute__((always_inline)) {
        if constexpr (FAC) {
            compute_fac(s, valid);
            return;
        }
        bf16x8 pst[NCB][NKA];
        pack_state(pst);
        if constexpr (CH == 64) {
            f32x4 S[10], O[NCB][4];
            zero_o(O);
            tri_window(s, ic<0>{}, ic<0>{}, ic<0>{}, ic<15>{}, S, O, pst);
            decay_inter(O, fin, 0, 4, 0);
            tri_intra(s, ic<0>{}, S, O);
            update(s, ic<0>{}, ic<2>{}, valid, 0);
            write_out(s, ic<0>{}, O, one4);
        } else if constexpr (CH == 32) {
            // two chunks per tile: rows 0..31 (A) and 32..63 (B).  Scores only
            // inside each chunk; A's inter product reads the state before A,
            // B's the state after A's update.
            f32x4 S[10], O[NCB][4];
            zero_o(O);
            tri_window(s, ic<0>{}, ic<0>{}, ic<1>{}, ic<3>{}, S, O, pst);
            decay_inter(O, fin, 0, 2, 0);
            update(s, ic<0>{}, ic<1>{}, valid < 32 ? valid : 32, 0);  // A's keys (key step 0)
            pack_state(pst);
            inter2(s, ic<0>{}, ic<2>{}, O, pst);
            decay_inter(O, fin, 2, 4, 2);
            update(s, ic<1>{}, ic<1>{}, valid > 32 ? valid - 32 : 0, 32);  // B's keys (key step 1)
            bf16x8 vb[NCB][2];
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    vb[c][kk] = c < CPW ? col_op<VSEG>(s.v, kk * 32, colw + c * 16 + c4, lane) : ones;
            // intra inside each chunk: query block 0 (key block 0), 1 (key blocks
            // 0, 1), 2 (key block 2), 3 (key blocks 2, 3); diagonals masked
            const bf16x8 s0 = pack_acc_bf16(S[0], zero4);
            const bf16x8 s1 = pack_acc_bf16(S[1], S[2]);
            const bf16x8 s2 = pack_acc_bf16(S[5], zero4);
            const bf16x8 s3 = pack_acc_bf16(S[8], S[9]);
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                O[c][0] = mfma_bf16(vb[c][0], s0, O[c][0]);
                O[c][1] = mfma_bf16(vb[c][0], s1, O[c][1]);
                O[c][2] = mfma_bf16(vb[c][1], s2, O[c][2]);
                O[c][3] = mfma_bf16(vb[c][1], s3, O[c][3]);
            }
            write_out(s, ic<0>{}, O, one4);
        } else if constexpr (SHARE) {
            // one chunk of 128 rows per tile (windows A = rows 0..63 and B =
            // rows 64..127, B also against the full block of A's keys), the 36
            // score blocks split between the two compute waves: wave 0 takes
            // window A and the cross block's keys 0..31, wave 1 window B and
            // the cross keys 32..63 (18 blocks each).  Each packs its blocks
            // into the intra product's operands (ten per wave, 1 KB each,
            // lane-major) and, once both waves are done with Q, puts them into
            // the Q slot (and xfrag) for the other wave: fragment f at byte
            // 1024 f + 16 lane,
            // f = 0..5 window A (query block qb, key step kk <= qb / 2 in order),
            // 6..11 window B, 12..15 cross keys 0..31 (query block 4 + qb),
            // 16..19 cross keys 32..63.
            f32x4 Oa[NCB][4], Ob[NCB][4];
            zero_o(Oa);
            zero_o(Ob);
            bf16x8 fr[10];
            auto pack_window = [&](const f32x4 (&S)[10]) __attribute__((always_inline)) {
                int f = 0;
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                    for (int kk = 0; kk <= qb / 2; ++kk) {
                        const f32x4 s1 = 2 * kk + 1 <= qb ? S[qb * (qb + 1) / 2 + 2 * kk + 1] : zero4;
                        fr[f++] = pack_acc_bf16(S[qb * (qb + 1) / 2 + 2 * kk], s1);
                    }
            };
            // the cross scores of query rows 64 .. 127 against keys 32 KK ..
            // 32 KK + 31 (fragments 6 .. 9 of this wave), and with WITH_B the
            // inter product of window B from the same query operands
            auto cross = [&](auto kkc, auto with_bc) __attribute__((always_inline)) {
                constexpr int KK = decltype(kkc)::value;
                constexpr bool WITH_B = decltype(with_bc)::value != 0;
                f32x4 X[4][2];
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) X[qb][0] = X[qb][1] = zero4;
                bf16x8 qa[2][4], ka[2][2];
                auto load = [&](int ks, bf16x8 (&q_)[4], bf16x8 (&k_)[2]) __attribute__((always_inline)) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) q_[b] = row_op<QSEG>(s.q, (4 + b) * 16 + l16, ks * 32, g);
#pragma unroll
                    for (int b = 0; b < 2; ++b) k_[b] = row_op<QSEG>(s.k, (2 * KK + b) * 16 + l16, ks * 32, g);
                };
                load(0, qa[0], ka[0]);
#pragma unroll
                for (int ks = 0; ks < NKA; ++ks) {
                    if (ks + 1 < NKA) load(ks + 1, qa[(ks + 1) & 1], ka[(ks + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                        for (int b = 0; b < 2; ++b) X[qb][b] = mfma_bf16(ka[ks & 1][b], qa[ks & 1][qb], X[qb][b]);
                    if constexpr (WITH_B)
#pragma unroll
                        for (int c = 0; c < NCB; ++c)
#pragma unroll
                            for (int qb = 0; qb < 4; ++qb) Ob[c][qb] = mfma_bf16(pst[c][ks], qa[ks & 1][qb], Ob[c][qb]);
                }
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) fr[6 + qb] = pack_acc_bf16(X[qb][0], X[qb][1]);
            };
            if (h == 0) {
                f32x4 S[10];
                tri_window(s, ic<0>{}, ic<0>{}, ic<0>{}, ic<15>{}, S, Oa, pst);
                pack_window(S);
                cross(ic<0>{}, ic<1>{});
            } else {
                f32x4 S[10];
                tri_window(s, ic<4>{}, ic<4>{}, ic<0>{}, ic<15>{}, S, Ob, pst);
                pack_window(S);
                cross(ic<1>{}, ic<0>{});
                // window A's inter product, the next feature step's query
                // operands read during this one's products
                bf16x8 qa[2][4];
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) qa[0][qb] = row_op<QSEG>(s.q, qb * 16 + l16, 0, g);
#pragma unroll
                for (int ks = 0; ks < NKA; ++ks) {
                    if (ks + 1 < NKA)
#pragma unroll
                        for (int qb = 0; qb < 4; ++qb) qa[(ks + 1) & 1][qb] = row_op<QSEG>(s.q, qb * 16 + l16, (ks + 1) * 32, g);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                        for (int c = 0; c < NCB; ++c) Oa[c][qb] = mfma_bf16(pst[c][ks], qa[ks & 1][qb], Oa[c][qb]);
                }
            }
            // intra products of ten fragments: window A's (with V keys 0..63,
            // into Oa) or window B's (keys 64..127, into Ob), and the cross
            // block's keys 32 CK .. 32 CK + 31 (into Ob).  Each wave applies its
            // own fragments before SYNC1 and the other wave's after SYNC2, so
            // that its own are dead by the time the other's are read.
            auto apply = [&](const bf16x8 (&f)[10], auto wac, auto ckc) __attribute__((always_inline)) {
                constexpr bool WA = decltype(wac)::value != 0;
                constexpr int CK = decltype(ckc)::value;
                bf16x8 vw[NCB][2], vx[NCB][1];
                load_v(s, ic<WA ? 0 : 2>{}, ic<2>{}, vw);
                if constexpr (WA && CK == 0) {
#pragma unroll
                    for (int c = 0; c < NCB; ++c) vx[c][0] = vw[c][0];
                } else {
                    load_v(s, ic<CK>{}, ic<1>{}, vx);
                }
                int i = 0;
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                    for (int kk = 0; kk <= qb / 2; ++kk, ++i)
#pragma unroll
                        for (int c = 0; c < NCB; ++c) {
                            if constexpr (WA)
                                Oa[c][qb] = mfma_bf16(vw[c][kk], f[i], Oa[c][qb]);
                            else
                                Ob[c][qb] = mfma_bf16(vw[c][kk], f[i], Ob[c][qb]);
                        }
#pragma unroll
                for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                    for (int c = 0; c < NCB; ++c) Ob[c][qb] = mfma_bf16(vx[c][0], f[6 + qb], Ob[c][qb]);
            };
            if (h == 0)
                apply(fr, ic<1>{}, ic<0>{});
            else
                apply(fr, ic<0>{}, ic<1>{});
            __syncthreads();  // SYNC1(t): both compute waves are done reading Q
            // fragment f: in the Q slot while f < QF, then in xfrag
            auto fa = [&](int f) __attribute__((always_inline)) {
                return (f < QF ? reinterpret_cast<char*>(s.q) + 1024 * f : xfrag + 1024 * (f - QF)) + 16 * lane;
            };
            const int own_w = h == 0 ? 0 : 6, own_x = h == 0 ? 12 : 16;
            const int oth_w = h == 0 ? 6 : 0, oth_x = h == 0 ? 16 : 12;
#pragma unroll
            for (int i = 0; i < 6; ++i) *reinterpret_cast<bf16x8*>(fa(own_w + i)) = fr[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<bf16x8*>(fa(own_x + i)) = fr[6 + i];
            __syncthreads();  // SYNC2(t): every score operand is in place
            bf16x8 ot[10];
#pragma unroll
            for (int i = 0; i < 6; ++i) ot[i] = *reinterpret_cast<const bf16x8*>(fa(oth_w + i));
#pragma unroll
            for (int i = 0; i < 4; ++i) ot[6 + i] = *reinterpret_cast<const bf16x8*>(fa(oth_x + i));
            if (h == 0)
                apply(ot, ic<0>{}, ic<1>{});
            else
                apply(ot, ic<1>{}, ic<0>{});
            update(s, ic<0>{}, ic<4>{}, valid, 0);
            write_out(s, ic<0>{}, Oa, one4);
            write_out(s, ic<4>{}, Ob, one4);
        } else {
            // one chunk of 128 rows per tile: query rows 0..63 against their own
            // keys; query rows 64..127 against their own keys and the full block
            // of keys 0..63; then the update with all 128 keys.
            f32x4 Oa[NCB][4], Ob[NCB][4];
            zero_o(Oa);
            zero_o(Ob);
            {
                f32x4 S[10];
                tri_window(s, ic<0>{}, ic<0>{}, ic<0>{}, ic<15>{}, S, Oa, pst);
                decay_inter(Oa, fin, 0, 4, 0);
                tri_intra(s, ic<0>{}, S, Oa);
            }
            {
                f32x4 S[10];
                tri_window(s, ic<4>{}, ic<4>{}, ic<0>{}, ic<15>{}, S, Ob, pst);
                decay_inter(Ob, fin64, 0, 4, 0);
                tri_intra(s, ic<2>{}, S, Ob);
            }
            // cross block, one key step (two 16-key blocks) at a time
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                f32x4 X[4][2];
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) X[qb][0] = X[qb][1] = zero4;
                bf16x8 qa[2][4], ka[2][2];
                auto load = [&](int ks, bf16x8 (&q_)[4], bf16x8 (&k_)[2]) __attribute__((always_inline)) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) q_[b] = row_op<QSEG>(s.q, (4 + b) * 16 + l16, ks * 32, g);
#pragma unroll
                    for (int b = 0; b < 2; ++b) k_[b] = row_op<QSEG>(s.k, (2 * kk + b) * 16 + l16, ks * 32, g);
                };
                load(0, qa[0], ka[0]);
#pragma unroll
                for (int ks = 0; ks < NKA; ++ks) {
                    if (ks + 1 < NKA) load(ks + 1, qa[(ks + 1) & 1], ka[(ks + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                        for (int b = 0; b < 2; ++b) X[qb][b] = mfma_bf16(ka[ks & 1][b], qa[ks & 1][qb], X[qb][b]);
                }
                bf16x8 vb[NCB];
#pragma unroll
                for (int c = 0; c < NCB; ++c) vb[c] = c < CPW ? col_op<VSEG>(s.v, kk * 32, colw + c * 16 + c4, lane) : ones;
                if constexpr (DECAY) {
                    // query 64 + 16 qb + l16, key 32 kk + 16 b + 4g + i: D = 4 + qb - 2 kk - b
#pragma unroll
                    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
                        for (int b = 0; b < 2; ++b)
#pragma unroll
                            for (int i = 0; i < 4; ++i) X[qb][b][i] *= fd[4 + qb - 2 * kk - b][i];
                }
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) {
                    const bf16x8 xb = pack_acc_bf16(X[qb][0], X[qb][1]);
#pragma unroll
                    for (int c = 0; c < NCB; ++c) Ob[c][qb] = mfma_bf16(vb[c], xb, Ob[c][qb]);
                }
            }
            update(s, ic<0>{}, ic<4>{}, valid, 0);
            write_out(s, ic<0>{}, Oa, one4);
            write_out(s, ic<4>{}, Ob, one4);
        }
    };

    auto step = [&](auto sidx, int64_t t) __attribute__((always_inline)) {
        constexpr int SI = decltype(sidx)::value;
        __syncthreads();  // B(t)
        if constexpr (MAP2) {
            phi_share(st[SI], valid_rows(t));
            __syncthreads();  // B'(t)
        } else if (!PHI && valid_rows(t) < TT) {
            zero_tail(st[SI], valid_rows(t));
            __syncthreads();
        }
        compute(st[SI], valid_rows(t));
    };
    for (int64_t t = t_begin; t < t_end; t += NSTAGE) {
        step(ic<0>{}, t);
        if (t + 1 < t_end) step(ic<1>{}, t + 1);
        if constexpr (NSTAGE >= 3)
            if (t + 2 < t_end) step(ic<2>{}, t + 2);
        if constexpr (NSTAGE >= 4)
            if (t + 3 < t_end) step(ic<3>{}, t + 3);
    }
    __syncthreads();  // matches the copy waves' final barrier

    const float ss_fin = p.state_scale * (FAC ? __builtin_amdgcn_exp2f((float)nr * lg) : 1.f);
    if (t_end == n_tiles && p.S_final != nullptr) {
        float* Sf = p.S_final + (bh * DK) * (int64_t)dv + col0 + colw + l16;
        const float ss = ss_fin;
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Sf[(int64_t)(32 * ks + 8 * g + 4 * hf + i) * dv + c * 16] = P[c][ks][hf][i] * ss;
    }
    if constexpr (NORM) {
        if (t_end == n_tiles && p.z_final != nullptr && jt == 0 && h == 0 && l16 == 0) {
            float* zf = p.z_final + bh * DK;
            const float ss = ss_fin;
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) zf[32 * ks + 8 * g + 4 * hf + i] = P[CPW][ks][hf][i] * ss;
        }
    }
}

// Output scaling exists for the scaled identity map without the normaliser
// only (normalised outputs are scale-free; pre-mapped inputs carry the scale).
template <int DK, int DVT, int CH, bool NORM, bool PHI, int DECAY>
hipError_t launch_fwd_pipe(const FwdParams& p, int64_t grid, hipStream_t s) {
    const dim3 block(4 * WAVE);
    if (p.out_scale != 1.0f) {
        if constexpr (NORM || PHI) {
            return hipErrorInvalidValue;
        } else {
            hipLaunchKernelGGL((chunked_fwd_pipe<DK, DVT, CH, true, false, false, DECAY>), dim3((unsigned)grid), block,
                               0, s, p);
        }
    } else {
        hipLaunchKernelGGL((chunked_fwd_pipe<DK, DVT, CH, false, NORM, PHI, DECAY>), dim3((unsigned)grid), block, 0, s,
                           p);
    }
    return hipGetLastError();
}

}  // namespace la
