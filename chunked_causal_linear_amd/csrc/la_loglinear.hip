// Log-linear attention on chunks of 64 rows (slide deck "Log-Linear
// Attention": the Fenwick-tree partition of the past, the hierarchical mask M
// and the chunkwise computation - inside a chunk directly, across chunks
// through bucket states, one per Fenwick level).
//
// Query t sees key s <= t at level 0 (s = t) or floor(log2(t XOR s)) + 1, with
// per-token weights lam[t, level].  For a chunk n of C = 2^c rows, keys in an
// earlier chunk n' sit at level c + floor(log2(n XOR n')) + 1, so the earlier
// chunks form buckets of 2^(m-1) whole chunks, one for each set bit m-1 of n:
// chunks [h - 2^(m-1), h), h = n with its bits below m-1 cleared.
//
//   * run_loglinear_pyramid: the bucket states.  Level 1 buckets are single
//     chunks (the per-chunk states of phase 1); level m >= 2 node j sums level
//     m-1 nodes 2j and 2j+1 (a pyramid of N/2 + N/4 + ... states; each thread
//     owns four consecutive state elements through every level).
//   * loglinear_fwd: one workgroup per (head, chunk, 64 value columns), four
//     waves of 16 query rows.  Intra part: S^T = K Q^T on the matrix cores, each
//     score times lam[query, level] (0 above the diagonal), then V^T S^T;
//     inter part: for every set bit of n, the bucket state goes through LDS as
//     bf16 (P^T, rows = value columns), O_m^T = P^T Q^T, and O += lam[t, c + m]
//     O_m.  Outputs come out transposed (a lane holds four consecutive columns
//     of one row) and are stored as 8-byte pieces.
//   * loglinear_step_kernel: one decode step, the Fenwick tree recurrence over
//     each stream's level states (below);
//   * loglinear_prefix_levels_kernel: the level states after a prefix, for a
//     decode that follows a forward (from the forward's own chunk states and
//     pyramid when it is asked for them).
#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

namespace {

constexpr int LL_C = 64;          // rows per chunk
constexpr int LL_CB = 6;          // log2 of it
constexpr int LL_DVT = 64;        // value columns per workgroup
constexpr int LL_NLMAX = 40;      // most levels (bit length of L - 1 plus one)

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

__device__ __forceinline__ uint2 tr_read_ll(const char* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p));
}

// 16-byte row operand: row r, elements k0 + 8g .. k0 + 8g + 7 of a row-major
// tile with a row stride of `stride` elements.
__device__ __forceinline__ bf16x8 row_operand(const u16* t, int stride, int r, int k0, int g) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(t + r * stride + k0 + 8 * g));
}

// Row r's elements k0 + 4g .. k0 + 4g + 3 and k0 + 16 + 4g .. k0 + 16 + 4g + 3:
// the order of the column operand below.
__device__ __forceinline__ bf16x8 row_operand_split(const u16* t, int stride, int r, int k0, int g) {
    const uint2 lo = *reinterpret_cast<const uint2*>(t + r * stride + k0 + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(t + r * stride + k0 + 16 + 4 * g);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Column operand over keys key0 .. key0 + 31 in the order the S^T accumulators
// come out in (lane group g: keys 4g..4g+3 and 16+4g..16+4g+3), column base + n
// for lane n of the group (transpose reads of four rows at a time).
__device__ __forceinline__ bf16x8 col_operand(const u16* t, int stride, int key0, int base, int lane) {
    const int g = lane >> 4, rr = (lane & 15) >> 2, c4 = 4 * (lane & 3);
    const char* p = reinterpret_cast<const char*>(t);
    const uint2 lo = tr_read_ll(p + ((key0 + 4 * g + rr) * stride + base + c4) * 2);
    const uint2 hi = tr_read_ll(p + ((key0 + 16 + 4 * g + rr) * stride + base + c4) * 2);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ int bit_length(unsigned x) { return x == 0 ? 0 : 32 - __builtin_clz(x); }

int bit_length_host(int64_t x) {
    int b = 0;
    for (; x > 0; x >>= 1) ++b;
    return b;
}

__device__ __forceinline__ float4 add4f(const float4& a, const float4& b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Level m >= 2 has floor(N / 2^(m-1)) nodes; node j is the sum of chunk
// states j 2^(m-1) .. (j + 1) 2^(m-1) - 1, stored in bf16 (the forward's
// products take bucket states in bf16, so it reads half the bytes).  Every
// node is summed in fp32 and rounded once.  A thread owns four state elements:
// it reads each whole group of eight chunk states once and sums its level-2,
// -3 and -4 nodes in registers; the level-4 nodes feed a binary carry (cy[i]:
// the waiting left node of level 4 + i) that completes the nodes of levels 5
// and up in the same pass; the chunks past the last whole group give the tail
// of levels 2 and 3.  With `lev`, a node that is a bucket of the state after
// token Tl (level m + 6 of that state when bit m + 5 of Tl is set: node
// (Tl >> (m + 5)) - 1) is also written there, in fp32.  NC >= floor(log2 N) - 3.
template <int NC>
__global__ __launch_bounds__(256) void loglinear_pyramid_kernel(const float4* __restrict__ S, uint2* __restrict__ T,
                                                                int64_t BH, int N, int n_pyr, int64_t E4,
                                                                float4* __restrict__ lev, int64_t Tl, int n_lev) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * E4) return;
    const int64_t bh = idx / E4, e = idx % E4;
    const float4* s1 = S + bh * N * E4 + e;  // level 1: the chunk states
    uint2* out = T + bh * (int64_t)n_pyr * E4 + e;
    // node j of level m at out[(off + j) E4], off = the nodes of levels 2 .. m - 1
    auto put = [&](int m, int64_t off, int64_t j, const float4& x) {
        out[(off + j) * E4] = make_uint2(pack2_bf16(x.x, x.y), pack2_bf16(x.z, x.w));
        if (lev != nullptr && ((Tl >> (m + 5)) & 1) && j == (Tl >> (m + 5)) - 1)
            lev[(bh * n_lev + m + 6) * E4 + e] = x;
    };
    const int64_t off3 = N >> 1, off4 = off3 + (N >> 2), off5 = off4 + (N >> 3);
    const int g8 = N / 8;  // whole groups of eight
    float4 cy[NC];
    for (int b = 0; b < g8; ++b) {
        float4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = s1[(int64_t)(8 * b + u) * E4];
        float4 y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            y[u] = add4f(x[2 * u], x[2 * u + 1]);
            put(2, 0, 4 * b + u, y[u]);
        }
        const float4 z0 = add4f(y[0], y[1]), z1 = add4f(y[2], y[3]);
        put(3, off3, 2 * b, z0);
        put(3, off3, 2 * b + 1, z1);
        float4 cur = add4f(z0, z1);
        put(4, off4, b, cur);
        // carry: a level-(4 + i) node with an even index waits; an odd one
        // completes node j / 2 of level 5 + i with the one waiting
        int64_t j = b, off = off5;
        bool go = true;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (go) {
                if ((j & 1) == 0) {
                    cy[i] = cur;
                    go = false;
                } else {
                    cur = add4f(cy[i], cur);
                    j >>= 1;
                    put(5 + i, off, j, cur);
                    off += N >> (4 + i);  // the nodes of level 5 + i
                }
            }
        }
    }
    const int rem = N - 8 * g8;  // chunks past the last whole group (0..7)
    if (rem >= 2) {
        float4 y[2];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            if (2 * u + 1 < rem) {
                const int64_t c = 8 * g8 + 2 * u;
                const float4 yu = add4f(s1[c * E4], s1[(c + 1) * E4]);
                put(2, 0, 4 * g8 + u, yu);
                if (u < 2) y[u] = yu;
            }
        }
        if (rem >= 4) put(3, off3, 2 * g8, add4f(y[0], y[1]));
    }
}

// Three workgroups share a CU (at most 168 VGPRs, 46 KB of LDS at d_k = 128):
// the bucket state tile reuses K's and V's LDS once the intra part is done (stored
// [a][j] by 8-byte writes, read back by transpose reads), and only the in-chunk level
// weights (levels 0..6) are staged; a bucket's weight is
// read per row from global memory.
template <int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void loglinear_fwd(LogLinParams p) {
    constexpr int QS = DK + 8, VS = LL_DVT + 8;  // padded row strides (elements)
    constexpr int NKA = DK / 32;
    constexpr int NLI = LL_CB + 2;               // in-chunk levels 0..LL_CB, padded
    constexpr int PS = LL_DVT + 8;               // the bucket state's row stride ([a][j], d_k rows)
    static_assert(DK * PS <= LL_C * (QS + VS), "the bucket state fits where K and V were");
    __shared__ __attribute__((aligned(16))) u16 Qs[LL_C * QS];
    __shared__ __attribute__((aligned(16))) u16 KV[LL_C * (QS + VS)];  // K and V, then the bucket state
    __shared__ float lam_s[LL_C * NLI];
    u16* const Ks = KV;
    u16* const Vs = KV + LL_C * QS;
    u16* const Ps = KV;

    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    int w = blockIdx.x;
    if (p.xcd_remap) w = (w & 7) * (gridDim.x >> 3) + (w >> 3);
    const int jt = w % p.n_dvt;
    const int n = (w / p.n_dvt) % p.N;
    const int64_t bh = w / (p.n_dvt * p.N);
    const int col0 = jt * LL_DVT;
    const int64_t r0 = (int64_t)n * LL_C;
    const int valid = (int)(p.L - r0 < LL_C ? p.L - r0 : LL_C);
    const int dv = p.dv;

    // Bucket states: level m (bit m - 1 of n set) holds chunks
    // [h - 2^(m-1), h) as node (n >> (m - 1)) - 1 of its level: level 1 is the
    // per-chunk states, levels 2.. the pyramid, level l starting after the
    // floor(N / 2^(j-1)) nodes of every level j in 2 .. l - 1.  Each state is
    // loaded into registers one level ahead (the first one before the chunk's
    // tiles), so its load overlaps the products of the level before.
    const int64_t E = (int64_t)DK * dv;
    auto next_level = [&](int m) {  // the first level above m whose bit is set in n, or 0
        for (int mm = m + 1; (1 << (mm - 1)) <= n; ++mm)
            if ((n >> (mm - 1)) & 1) return mm;
        return 0;
    };
    // A level-1 bucket is a chunk state (fp32); the pyramid's nodes are bf16.
    constexpr int NPT = DK * (LL_DVT / 4) / 256;  // four-element pieces of a state tile per thread
    float4 xf[NPT];                               // a level-1 bucket
    uint2 xb[NPT];                                // a node of level 2 or more, four bf16 packed
    auto load_state = [&](int m) {
        const int node = (n >> (m - 1)) - 1;
        if (m == 1) {
            const float* P = p.S + (bh * p.N + node) * E;
#pragma unroll
            for (int u = 0; u < NPT; ++u) {
                const int i = tid + u * 256;
                const int a = i / (LL_DVT / 4), j4 = (i % (LL_DVT / 4)) * 4;
                xf[u] = *reinterpret_cast<const float4*>(P + (int64_t)a * dv + col0 + j4);
            }
        } else {
            int base = 0;
            for (int l = 2; l < m; ++l) base += p.N >> (l - 1);
            const u16* P = p.T + (bh * p.n_pyr + base + node) * E;
#pragma unroll
            for (int u = 0; u < NPT; ++u) {
                const int i = tid + u * 256;
                const int a = i / (LL_DVT / 4), j4 = (i % (LL_DVT / 4)) * 4;
                xb[u] = *reinterpret_cast<const uint2*>(P + (int64_t)a * dv + col0 + j4);
            }
        }
    };
    int m = next_level(0);
    if (m != 0) load_state(m);

    // chunk tiles into LDS (rows past the end are zero)
    for (int i = tid; i < LL_C * (DK / 8); i += 256) {
        const int r = i / (DK / 8), cg = i % (DK / 8);
        uint4 qv = make_uint4(0, 0, 0, 0), kv = qv;
        if (r < valid) {
            qv = *reinterpret_cast<const uint4*>(p.q + (bh * p.L + r0 + r) * DK + cg * 8);
            kv = *reinterpret_cast<const uint4*>(p.k + (bh * p.L + r0 + r) * DK + cg * 8);
        }
        *reinterpret_cast<uint4*>(Qs + r * QS + cg * 8) = qv;
        *reinterpret_cast<uint4*>(Ks + r * QS + cg * 8) = kv;
    }
    for (int i = tid; i < LL_C * (LL_DVT / 8); i += 256) {
        const int r = i / (LL_DVT / 8), cg = i % (LL_DVT / 8);
        uint4 vv = make_uint4(0, 0, 0, 0);
        if (r < valid) vv = *reinterpret_cast<const uint4*>(p.v + (bh * p.L + r0 + r) * dv + col0 + cg * 8);
        *reinterpret_cast<uint4*>(Vs + r * VS + cg * 8) = vv;
    }
    for (int i = tid; i < LL_C * NLI; i += 256) {
        const int r = i / NLI, l = i % NLI;
        lam_s[i] = (r < valid && l < p.n_lev) ? p.lam[(bh * p.L + r0 + r) * p.n_lev + l] : 0.f;
    }
    __syncthreads();

    const int qr = wave * 16 + l16;  // this lane's query row in the chunk
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 O[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) O[c] = zero4;

    // ---- intra: scores of query block `wave` against key blocks kb <= wave
    {
        f32x4 St[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) St[kb] = zero4;
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) {
            const bf16x8 qa = row_operand(Qs, QS, qr, ks * 32, g);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                if (kb <= wave) St[kb] = mfma_bf16(row_operand(Ks, QS, kb * 16 + l16, ks * 32, g), qa, St[kb]);
        }
        // St[kb][i] = score of key 16 kb + 4g + i and query qr: weight by its level
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kb * 16 + 4 * g + i;
                const int lev = key == qr ? 0 : bit_length((unsigned)(key ^ qr));
                St[kb][i] = (kb <= wave && key <= qr) ? St[kb][i] * lam_s[qr * NLI + lev] : 0.f;
            }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (2 * kk > wave) break;
            const bf16x8 sb = pack_acc_bf16(St[2 * kk], St[2 * kk + 1]);
#pragma unroll
            for (int c = 0; c < 4; ++c) O[c] = mfma_bf16(col_operand(Vs, VS, kk * 32, c * 16, lane), sb, O[c]);
        }
    }

    // ---- inter: one bucket state per set bit of n
    const float* lam_row = p.lam + (bh * p.L + r0 + (qr < valid ? qr : 0)) * p.n_lev;
    while (m != 0) {
        const int mn = next_level(m);
        const float lw = qr < valid ? lam_row[LL_CB + m] : 0.f;
        __syncthreads();  // Ps free (the first time: K and V are no longer read)
#pragma unroll
        for (int u = 0; u < NPT; ++u) {
            const int i = tid + u * 256;
            const int a = i / (LL_DVT / 4), j4 = (i % (LL_DVT / 4)) * 4;
            const uint32_t ab = m == 1 ? pack2_bf16(xf[u].x, xf[u].y) : xb[u].x;
            const uint32_t cd = m == 1 ? pack2_bf16(xf[u].z, xf[u].w) : xb[u].y;
            *reinterpret_cast<uint2*>(Ps + a * PS + j4) = make_uint2(ab, cd);
        }
        if (mn != 0) load_state(mn);
        __syncthreads();
        f32x4 Om[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) Om[c] = zero4;
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) {
            // P^T's rows by transpose reads over a = 32 ks .. 32 ks + 31 in the column
            // operand's order; the query operand takes the same order of a
            const bf16x8 qb = row_operand_split(Qs, QS, qr, ks * 32, g);
#pragma unroll
            for (int c = 0; c < 4; ++c) Om[c] = mfma_bf16(col_operand(Ps, PS, ks * 32, c * 16, lane), qb, Om[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) O[c] += lw * Om[c];
        m = mn;
    }

    // ---- output: lane holds columns 16c + 4g .. +3 of row qr
    if (qr < valid) {
        u16* o = p.o + (bh * p.L + r0 + qr) * dv + col0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<uint2*>(o + c * 16 + 4 * g) =
                make_uint2(pack2_bf16(O[c][0], O[c][1]), pack2_bf16(O[c][2], O[c][3]));
    }
}

// One decode step (the slides' Fenwick tree recurrence): the level states
// S[l] of a stream (the sum of k_s^T v_s over level l's bucket) advance to the
// token at position t.  With b the position of t's lowest set bit (t > 0),
// the buckets of levels 0..b merge into level b + 1 and levels 1..b empty;
// level 0 takes k_t^T v_t; then o = sum_l lam[l] q_t S[l].  After the step,
// level l >= 1 is non-empty only when bit l - 1 of t is set, so the output
// reads just those (besides level 0 and the merged level, which it forms
// itself).  One workgroup per (stream, DVS value columns): the columns of o
// are independent, so the slices need no reduction between workgroups.
// Thread t owns four columns (j4 = t % (DVS / 4)) of the rows
// a = t / (DVS / 4) + AG r, r < RPT, through every level; each level's RPT
// 16-byte loads go out together, and each element's merge, update and output
// share are formed in one pass.  The row partial sums of o reduce through LDS.
template <int DK, int DVS>
__global__ __launch_bounds__(256) void loglinear_step_kernel(LogLinStepParams p) {
    constexpr int NT = 256, J4 = DVS / 4, AG = NT / J4;
    constexpr int RPT = DK > AG ? DK / AG : 1;  // rows per thread (threads past DK idle)
    static_assert(J4 * AG == NT, "thread layout");
    __shared__ float qs[DK], ks[DK], vs[DVS], lw[LL_NLMAX];
    __shared__ float red[AG][DVS + 4];
    const int tid = threadIdx.x;
    const int j4 = tid % J4, ag = tid / J4;
    const int n_sl = p.dv / DVS;
    const int64_t st = blockIdx.x / n_sl;
    const int col0 = (blockIdx.x % n_sl) * DVS;
    const int dv = p.dv, nl = p.n_lev;
    const int64_t t = p.t;
    for (int i = tid; i < DK; i += NT) {
        qs[i] = bf2f(p.q[st * DK + i]);
        ks[i] = bf2f(p.k[st * DK + i]);
    }
    for (int i = tid; i < DVS; i += NT) vs[i] = bf2f(p.v[st * dv + col0 + i]);
    for (int i = tid; i < nl; i += NT) lw[i] = p.lam[st * nl + i];
    __syncthreads();
    // b = the lowest set bit of t (-1 at t = 0: nothing merges)
    const int b = t > 0 ? __builtin_ctzll((unsigned long long)t) : -1;
    const int64_t lev = (int64_t)DK * dv / 4;  // float4s per level
    float4* S = reinterpret_cast<float4*>(p.S) + st * nl * lev;
    const bool live = ag < DK;
    // element r of this thread: row ag + AG r, columns col0 + 4 j4 ..
    int64_t e[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) e[r] = (int64_t)(live ? ag + AG * r : 0) * (dv / 4) + col0 / 4 + j4;
    const float4 v4 = make_float4(vs[4 * j4], vs[4 * j4 + 1], vs[4 * j4 + 2], vs[4 * j4 + 3]);
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    auto fma4 = [](float w, const float4& x, const float4& y) {
        return make_float4(fmaf(w, x.x, y.x), fmaf(w, x.y, y.y), fmaf(w, x.z, y.z), fmaf(w, x.w, y.w));
    };
    float4 s0[RPT], acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float ka = live ? ks[ag + AG * r] : 0.f;
        s0[r] = make_float4(ka * v4.x, ka * v4.y, ka * v4.z, ka * v4.w);
        acc[r] = fma4(lw[0], s0[r], zero);
    }
    if (live) {
        if (b >= 0) {
            float4 merged[RPT];
#pragma unroll
            for (int r = 0; r < RPT; ++r) merged[r] = S[e[r]];
            for (int l = 1; l <= b; ++l) {
                float4 x[RPT];
#pragma unroll
                for (int r = 0; r < RPT; ++r) x[r] = S[l * lev + e[r]];
#pragma unroll
                for (int r = 0; r < RPT; ++r) merged[r] = add4f(merged[r], x[r]);
            }
            const float w = lw[b + 1];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                acc[r] = fma4(w, merged[r], acc[r]);
                S[(b + 1) * lev + e[r]] = merged[r];
            }
            for (int l = 1; l <= b; ++l)
#pragma unroll
                for (int r = 0; r < RPT; ++r) S[l * lev + e[r]] = zero;
        }
        // the untouched levels that hold keys: bit l - 1 of t set, l > b + 1
        for (int l = b + 2; l < nl; ++l) {
            if (((t >> (l - 1)) & 1) == 0) continue;
            float4 x[RPT];
#pragma unroll
            for (int r = 0; r < RPT; ++r) x[r] = S[l * lev + e[r]];
            const float w = lw[l];
#pragma unroll
            for (int r = 0; r < RPT; ++r) acc[r] = fma4(w, x[r], acc[r]);
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) S[e[r]] = s0[r];
    }
    float4 part = zero;
    if (live)
#pragma unroll
        for (int r = 0; r < RPT; ++r) part = fma4(qs[ag + AG * r], acc[r], part);
    red[ag][4 * j4] = part.x;
    red[ag][4 * j4 + 1] = part.y;
    red[ag][4 * j4 + 2] = part.z;
    red[ag][4 * j4 + 3] = part.w;
    __syncthreads();
    for (int c = tid; c < DVS; c += NT) {
        float sum = 0.f;
        for (int r = 0; r < AG; ++r) sum += red[r][c];
        if (p.out_f32)
            reinterpret_cast<float*>(p.o)[st * dv + col0 + c] = sum;
        else
            reinterpret_cast<u16*>(p.o)[st * dv + col0 + c] = f2bf(sum);
    }
}

// The level states after token T = L - 1: level 0 = k_T^T v_T; level l >= 1
// = the sum of k_s^T v_s over its bucket [h - 2^(l-1), h), h = T with its bits
// below l - 1 cleared, when bit l - 1 of T is set, else zero.  A bucket of
// 64 rows or more (l >= 7) is a run of whole chunks before T's chunk: the sum
// of their states, in chunk order (after a forward, the levels of two chunks
// or more are written by its pyramid and left alone here); the smaller
// buckets lie in T's chunk and are summed from the rows.  One workgroup per (head,
// level, 256 float4s of the state); a thread owns one float4 and keeps sixteen
// chunk loads in flight.
__global__ __launch_bounds__(256) void loglinear_prefix_levels_kernel(LogLinPrefixParams p) {
    const int64_t E4 = (int64_t)p.dk * p.dv / 4;
    const int64_t nblk = (E4 + 255) / 256;
    const int64_t blk = blockIdx.x % nblk;
    const int l = (int)((blockIdx.x / nblk) % p.n_lev);
    const int64_t bh = blockIdx.x / (nblk * p.n_lev);
    const int64_t T = p.L - 1;
    const int dv4 = p.dv / 4;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    float4* out = reinterpret_cast<float4*>(p.S) + (bh * p.n_lev + l) * E4;
    const bool present = l == 0 || ((T >> (l - 1)) & 1);
    int64_t r0 = T, r1 = T + 1;  // level 0: row T
    if (l > 0) {
        const int64_t h = (T >> (l - 1)) << (l - 1);
        r0 = h - ((int64_t)1 << (l - 1));
        r1 = h;
    }
    const u16* kh = p.k + bh * p.L * p.dk;
    const u16* vh = p.v + bh * p.L * p.dv;
    const int64_t e = blk * 256 + threadIdx.x;
    if (e >= E4 || (present && l >= 8 && p.pyr_written)) return;
    float4 sum = zero;
    if (present) {
        if (r1 - r0 >= 64) {
            const float4* ch = reinterpret_cast<const float4*>(p.chunks) + bh * p.n_chunks * E4 + e;
#pragma unroll 16
            for (int64_t c = r0 / 64; c < r1 / 64; ++c) sum = add4f(sum, ch[c * E4]);
        } else {
            const int a = (int)(e / dv4), c4 = (int)(e % dv4) * 4;
#pragma unroll 8
            for (int64_t r = r0; r < r1; ++r) {
                const float ka = bf2f(kh[r * p.dk + a]);
                const u16* vr = vh + r * p.dv + c4;
                sum.x = fmaf(ka, bf2f(vr[0]), sum.x);
                sum.y = fmaf(ka, bf2f(vr[1]), sum.y);
                sum.z = fmaf(ka, bf2f(vr[2]), sum.z);
                sum.w = fmaf(ka, bf2f(vr[3]), sum.w);
            }
        }
    }
    out[e] = sum;
}

}  // namespace

hipError_t run_loglinear_pyramid(const float* S, unsigned short* T, int64_t BH, int N, int n_pyr, int64_t E,
                                 float* lev, int64_t Tl, int n_lev, hipStream_t s) {
    if (N < 2 || T == nullptr) return hipSuccess;
    if (E % 4 != 0 || (lev != nullptr && (Tl < 0 || n_lev < bit_length_host(Tl) + 1))) return hipErrorInvalidValue;
    const int64_t E4 = E / 4;
    const int64_t blocks = (BH * E4 + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const int lg = bit_length_host(N) - 1;  // floor(log2 N)
    const float4* S4 = reinterpret_cast<const float4*>(S);
    uint2* T2 = reinterpret_cast<uint2*>(T);
    float4* L4 = reinterpret_cast<float4*>(lev);
    if (lg - 3 <= 4)
        hipLaunchKernelGGL(loglinear_pyramid_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, S4, T2, BH, N, n_pyr,
                           E4, L4, Tl, n_lev);
    else if (lg - 3 <= 8)
        hipLaunchKernelGGL(loglinear_pyramid_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, S4, T2, BH, N, n_pyr,
                           E4, L4, Tl, n_lev);
    else if (lg - 3 <= 16)
        hipLaunchKernelGGL(loglinear_pyramid_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, S4, T2, BH, N,
                           n_pyr, E4, L4, Tl, n_lev);
    else
        hipLaunchKernelGGL(loglinear_pyramid_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, S4, T2, BH, N,
                           n_pyr, E4, L4, Tl, n_lev);
    return hipGetLastError();
}

hipError_t run_loglinear_fwd(const LogLinParams& p, int64_t grid, hipStream_t s) {
    if (p.n_lev > LL_NLMAX || p.dv % LL_DVT != 0) return hipErrorInvalidValue;
    switch (p.dk) {
        case 64: hipLaunchKernelGGL(loglinear_fwd<64>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
        case 128: hipLaunchKernelGGL(loglinear_fwd<128>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace la

namespace la {

hipError_t run_loglinear_step(const LogLinStepParams& p, hipStream_t s) {
    if (p.n < 1 || p.n > 0x7FFFFFFFLL || p.dk < 1 || p.dk > 256 || p.n_lev < 1 || p.n_lev > LL_NLMAX || p.t < 0)
        return hipErrorInvalidValue;
    // the merged level (lowest set bit of t, plus one) and every level that
    // holds keys after the step (up to the bit length of t) must exist
    const int bits = p.t > 0 ? 64 - __builtin_clzll((unsigned long long)p.t) : 0;
    if (p.n_lev < bits + 1) return hipErrorInvalidValue;
    // value columns per workgroup: 32 (16 when there are only 16)
    const int dvs = p.dv < 32 ? p.dv : 32;
    if (p.dv % dvs != 0 || p.n * (p.dv / dvs) > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.n * (p.dv / dvs)));
    switch (p.dk * 1000 + dvs) {
        case 16016: hipLaunchKernelGGL((loglinear_step_kernel<16, 16>), grid, dim3(256), 0, s, p); break;
        case 32016: hipLaunchKernelGGL((loglinear_step_kernel<32, 16>), grid, dim3(256), 0, s, p); break;
        case 64016: hipLaunchKernelGGL((loglinear_step_kernel<64, 16>), grid, dim3(256), 0, s, p); break;
        case 128016: hipLaunchKernelGGL((loglinear_step_kernel<128, 16>), grid, dim3(256), 0, s, p); break;
        case 256016: hipLaunchKernelGGL((loglinear_step_kernel<256, 16>), grid, dim3(256), 0, s, p); break;
        case 16032: hipLaunchKernelGGL((loglinear_step_kernel<16, 32>), grid, dim3(256), 0, s, p); break;
        case 32032: hipLaunchKernelGGL((loglinear_step_kernel<32, 32>), grid, dim3(256), 0, s, p); break;
        case 64032: hipLaunchKernelGGL((loglinear_step_kernel<64, 32>), grid, dim3(256), 0, s, p); break;
        case 128032: hipLaunchKernelGGL((loglinear_step_kernel<128, 32>), grid, dim3(256), 0, s, p); break;
        case 256032: hipLaunchKernelGGL((loglinear_step_kernel<256, 32>), grid, dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace la

namespace la {

hipError_t run_loglinear_prefix_levels(const LogLinPrefixParams& p, hipStream_t s) {
    if (p.BH < 1 || p.L < 1 || p.dk < 1 || p.dv < 4 || p.dv % 4 != 0 || p.n_lev < 1 || p.n_lev > LL_NLMAX)
        return hipErrorInvalidValue;
    const int64_t T = p.L - 1;
    if ((T >> 6) > p.n_chunks || ((T >> 6) > 0 && p.chunks == nullptr)) return hipErrorInvalidValue;
    const int64_t E4 = (int64_t)p.dk * p.dv / 4;
    const int64_t grid = p.BH * p.n_lev * ((E4 + 255) / 256);
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(loglinear_prefix_levels_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace la
