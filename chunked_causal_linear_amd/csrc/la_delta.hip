// The delta rule and its gated form (page "Kimi K3 と Qwen 3.8 の Attention 機構
// 比較分析": section 3.1, equation (14) - look up what the current key maps to,
// erase that old prediction along the key, write the new value; section 2.4 -
// the gated form adds a global decay of the state).  With the state S (d_k x
// d_v, read as o = q S), the write strength beta_t and the gate alpha_t:
//     u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t),  S_t = alpha_t S_{t-1} + k_t u_t^T,
//     o_t = q_t^T S_t  (read after the update).
//
// Three kernels:
//  * delta_step_kernel: one decode step for many states (a read-modify-write
//    stream over fp32 states; k^T S and q^T S in one pass, then the update);
//  * delta_transform_kernel: per chunk of 64 rows, T = (I + A)^-1 diag(beta)
//    with A[i][j] = beta_i (k_i . k_j) g_i / g_j for j < i (g_i the product of
//    the chunk's gates up to row i): K K^T on the matrix cores, the unit
//    lower-triangular inverse blockwise in fp32 (the four 16 x 16 diagonal
//    blocks by forward substitution, the blocks below them on the fp32 matrix
//    cores), stored as bf16 with its columns in the matrix-core operand order
//    of delta_fwd_kernel; also log2 g per row;
//  * delta_fwd_kernel: the chunks of one head in order, carrying the state
//    (state waves) beside waves that move the data and form the score tile.
//    Per chunk (P the state before it, n = 64 rows):
//        R = V - diag(g) K P,  U = T R,
//        O = diag(g) Q P + (tril(Q K^T) * G) U,     G[i][j] = g_i / g_j,
//        P <- g_n P + K^T diag(g_n / g) U,
//    the chunkwise form the recurrence unrolls to inside a chunk.
#include "la_fwd_pipe.hpp"

namespace la {

namespace {

constexpr float kMinGateLog2 = -100.0f;  // a zero gate acts as 2^-100

}  // namespace

// ---------------------------------------------------------------------------
// decode step
// ---------------------------------------------------------------------------
// Thread t owns four value columns (j4 = t % (DV / 4)) of the rows
// a = t / (DV / 4) + AG i: every S access is a coalesced 16-byte vector.  With
// at most 16 rows per thread the state stays in registers between the
// reductions and the update; otherwise it is read a second time.
template <int DK, int DV>
__global__ __launch_bounds__(256) void delta_step_kernel(DeltaStepParams p) {
    constexpr int NT = 256;
    constexpr int J4 = DV / 4;
    constexpr int AG = NT / J4;
    constexpr int RPT = DK / AG > 0 ? DK / AG : 1;
    constexpr bool KEEP = RPT <= 16;
    static_assert(AG * J4 == NT, "thread layout");

    __shared__ float qs[DK], ks[DK];
    __shared__ float redw[AG][DV + 1], redy[AG][DV + 1];
    __shared__ float uu[DV];
    __shared__ float qk_s;

    const int tid = threadIdx.x;
    const int j4 = tid % J4, ag = tid / J4;
    const int64_t st = blockIdx.x;
    for (int i = tid; i < DK; i += NT) {
        qs[i] = bf2f(p.q[st * DK + i]);
        ks[i] = bf2f(p.k[st * DK + i]);
    }
    __syncthreads();
    if (tid < WAVE) {
        float a = 0.f;
        for (int i = tid; i < DK; i += WAVE) a = fmaf(qs[i], ks[i], a);
        for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o);
        if (tid == 0) qk_s = a;
    }
    const float alpha = p.alpha != nullptr ? p.alpha[st] : 1.0f;
    const float beta = p.beta[st];

    float4* S = reinterpret_cast<float4*>(p.S + st * DK * DV);
    float4 cur[KEEP ? RPT : 1];
    float4 aw = make_float4(0.f, 0.f, 0.f, 0.f), ay = aw;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int a = ag + AG * i;
        if (a < DK) {
            const float4 x = S[a * J4 + j4];
            if constexpr (KEEP) cur[i] = x;
            const float kk = ks[a], qq = qs[a];
            aw.x = fmaf(kk, x.x, aw.x);
            aw.y = fmaf(kk, x.y, aw.y);
            aw.z = fmaf(kk, x.z, aw.z);
            aw.w = fmaf(kk, x.w, aw.w);
            ay.x = fmaf(qq, x.x, ay.x);
            ay.y = fmaf(qq, x.y, ay.y);
            ay.z = fmaf(qq, x.z, ay.z);
            ay.w = fmaf(qq, x.w, ay.w);
        }
    }
    redw[ag][4 * j4] = aw.x;
    redw[ag][4 * j4 + 1] = aw.y;
    redw[ag][4 * j4 + 2] = aw.z;
    redw[ag][4 * j4 + 3] = aw.w;
    redy[ag][4 * j4] = ay.x;
    redy[ag][4 * j4 + 1] = ay.y;
    redy[ag][4 * j4 + 2] = ay.z;
    redy[ag][4 * j4 + 3] = ay.w;
    __syncthreads();
    if (tid < DV) {
        float w = 0.f, y = 0.f;
        for (int r = 0; r < AG; ++r) {
            w += redw[r][tid];
            y += redy[r][tid];
        }
        // the value minus the old prediction at k (of the decayed state), and
        // the read q^T S' = alpha q^T S + (q . k) u
        const float u = beta * (bf2f(p.v[st * DV + tid]) - alpha * w);
        uu[tid] = u;
        const float o = fmaf(alpha, y, qk_s * u);
        if (p.out_f32)
            reinterpret_cast<float*>(p.o)[st * DV + tid] = o;
        else
            reinterpret_cast<u16*>(p.o)[st * DV + tid] = f2bf(o);
    }
    __syncthreads();
    const float4 u4 = make_float4(uu[4 * j4], uu[4 * j4 + 1], uu[4 * j4 + 2], uu[4 * j4 + 3]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int a = ag + AG * i;
        if (a < DK) {
            float4 x;
            if constexpr (KEEP)
                x = cur[i];
            else
                x = S[a * J4 + j4];
            const float kk = ks[a];
            x.x = fmaf(kk, u4.x, alpha * x.x);
            x.y = fmaf(kk, u4.y, alpha * x.y);
            x.z = fmaf(kk, u4.z, alpha * x.z);
            x.w = fmaf(kk, u4.w, alpha * x.w);
            S[a * J4 + j4] = x;
        }
    }
}

template <int DK>
static hipError_t delta_step_dv(const DeltaStepParams& p, hipStream_t s) {
    const dim3 grid((unsigned)p.n), block(256);
    switch (p.dv) {
        case 16: hipLaunchKernelGGL((delta_step_kernel<DK, 16>), grid, block, 0, s, p); break;
        case 32: hipLaunchKernelGGL((delta_step_kernel<DK, 32>), grid, block, 0, s, p); break;
        case 64: hipLaunchKernelGGL((delta_step_kernel<DK, 64>), grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL((delta_step_kernel<DK, 128>), grid, block, 0, s, p); break;
        case 256: hipLaunchKernelGGL((delta_step_kernel<DK, 256>), grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t run_delta_step(const DeltaStepParams& p, hipStream_t s) {
    switch (p.dk) {
        case 16: return delta_step_dv<16>(p, s);
        case 32: return delta_step_dv<32>(p, s);
        case 64: return delta_step_dv<64>(p, s);
        case 128: return delta_step_dv<128>(p, s);
        case 256: return delta_step_dv<256>(p, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// chunk transform: one wave per chunk of 64 rows
// ---------------------------------------------------------------------------
// A in 16 x 16 blocks (ib, jb), jb <= ib (index ib (ib + 1) / 2 + jb), rows
// of 20 floats: a lane's 16-byte slice of row l16 at columns 4g .. 4g + 3 and
// the element writes of a column both meet distinct banks.
constexpr int TB_ROW = 20, TB_BLK = 16 * TB_ROW;
__device__ __forceinline__ constexpr int tblk(int ib, int jb) { return (ib * (ib + 1) / 2 + jb) * TB_BLK; }

// acc += X Y for 16 x 16 blocks on the fp32 matrix cores (four 16x16x4 steps):
// `a` is the lane's slice X[l16][4g .. 4g + 3], `b` Y in the accumulator
// layout (lane (g, l16) element i = Y[4g + i][l16]); step i multiplies column
// 4g + i of X by row 4g + i of Y, each lane group g supplying its k index.
__device__ __forceinline__ f32x4 mm16(const float4& a, const f32x4& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b[3], acc, 0, 0, 0);
    return acc;
}

template <int DK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void delta_transform_kernel(DeltaPrepParams p) {
    constexpr int NKA = DK / 32;
    __shared__ __attribute__((aligned(16))) float Ab[10 * TB_BLK];
    __shared__ __attribute__((aligned(16))) float lgs[64], bes[64];

    const int lane = threadIdx.x, l16 = lane % 16, g = lane / 16;
    const int64_t chunk = blockIdx.x;  // bh * N + n
    const int64_t bh = chunk / p.N, n = chunk % p.N;
    const int64_t L = p.L;
    const int64_t r0 = n * 64;
    const int valid = (int)(L - r0 < 64 ? L - r0 : 64);

    // K K^T on the matrix cores with the operands straight from memory: lane
    // (l16, g) of block b takes row 16 b + l16, elements 32 ks + 8 g .. + 7
    // (rows past the end: zero).  Blocks (ib, jb), jb <= ib: lane holds row
    // 16 ib + 4 g + e, column 16 jb + l16.
    const u16* kg = p.k + (bh * L + r0) * DK;
    f32x4 acc[10];
#pragma unroll
    for (int b = 0; b < 10; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKA; ++ks) {
        bf16x8 kr[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = 16 * b + l16;
            kr[b] = as_bf16x8(r < valid ? *reinterpret_cast<const uint4*>(kg + (int64_t)r * DK + 32 * ks + 8 * g)
                                        : make_uint4(0, 0, 0, 0));
        }
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb) acc[ib * (ib + 1) / 2 + jb] = mfma_bf16(kr[ib], kr[jb], acc[ib * (ib + 1) / 2 + jb]);
    }

    // log2 of the gates' product over rows 0..lane (rows past the end: gate 1)
    float lg = 0.f;
    if (p.alpha != nullptr && lane < valid) lg = fmaxf(__log2f(p.alpha[bh * L + r0 + lane]), kMinGateLog2);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(lg, o);
        if (lane >= o) lg += t;
    }
    p.lg[chunk * 64 + lane] = lg;
    const float beta = lane < valid ? p.beta[bh * L + r0 + lane] : 0.f;

    lgs[lane] = lg;
    bes[lane] = beta;
    __syncthreads();

    // A[i][j] = beta_i g_i / g_j (k_i . k_j) for j < i, 0 on and above the
    // diagonal, into its blocks (lane (g, l16): rows 16 ib + 4g + e, column 16 jb + l16)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
        const float4 lgi = *reinterpret_cast<const float4*>(&lgs[16 * ib + 4 * g]);
        const float4 bi = *reinterpret_cast<const float4*>(&bes[16 * ib + 4 * g]);
        const float lgi4[4] = {lgi.x, lgi.y, lgi.z, lgi.w}, bi4[4] = {bi.x, bi.y, bi.z, bi.w};
#pragma unroll
        for (int jb = 0; jb <= ib; ++jb) {
            const int j = 16 * jb + l16;
            const float lgj = lgs[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ib + 4 * g + e;
                Ab[tblk(ib, jb) + (4 * g + e) * TB_ROW + l16] =
                    j < i ? bi4[e] * __builtin_amdgcn_exp2f(lgi4[e] - lgj) * acc[ib * (ib + 1) / 2 + jb][e] : 0.f;
            }
        }
    }
    __syncthreads();

    // The diagonal blocks' inverses X_bb = (I + A_bb)^-1 by forward
    // substitution, lane (b = g, c = l16) solving for column c of block b:
    // x_i = [i == c] - sum_{j < i} A_bb[i][j] x_j (A_bb's entries from i on are zero).
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.f;
    {
        const float* Abb = Ab + tblk(g, g);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float sacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j4 = 0; j4 < (i + 3) / 4; ++j4) {
                const float4 a = *reinterpret_cast<const float4*>(Abb + i * TB_ROW + 4 * j4);
                sacc[0] = fmaf(a.x, x[4 * j4], sacc[0]);
                sacc[1] = fmaf(a.y, x[4 * j4 + 1], sacc[1]);
                sacc[2] = fmaf(a.z, x[4 * j4 + 2], sacc[2]);
                sacc[3] = fmaf(a.w, x[4 * j4 + 3], sacc[3]);
            }
            x[i] = (i == l16 ? 1.f : 0.f) - ((sacc[0] + sacc[1]) + (sacc[2] + sacc[3]));
        }
    }
    __syncthreads();  // every lane has read its A_bb
    // X_bb in place of A_bb
#pragma unroll
    for (int i = 0; i < 16; ++i) Ab[tblk(g, g) + i * TB_ROW + l16] = x[i];
    __syncthreads();

    // The blocks below the diagonal, by distance from it:
    //   X_ij = -X_ii Y_ij,  Y_ij = sum_{k = j .. i - 1} A_ik X_kj.
    auto slice = [&](int blk) __attribute__((always_inline)) {  // X[l16][4g .. 4g + 3] of a block
        return *reinterpret_cast<const float4*>(Ab + blk + l16 * TB_ROW + 4 * g);
    };
    auto dlay = [&](int blk) __attribute__((always_inline)) {  // a block in the accumulator layout
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = Ab[blk + (4 * g + e) * TB_ROW + l16];
        return r;
    };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // one distance at a time, each stage's operands loaded where it starts
    const f32x4 X00 = dlay(tblk(0, 0));
    f32x4 X10, X21, X32, X20, X31, X30;
    {
        const f32x4 X11 = dlay(tblk(1, 1)), X22 = dlay(tblk(2, 2));
        X10 = -mm16(slice(tblk(1, 1)), mm16(slice(tblk(1, 0)), X00, z4), z4);
        X21 = -mm16(slice(tblk(2, 2)), mm16(slice(tblk(2, 1)), X11, z4), z4);
        X32 = -mm16(slice(tblk(3, 3)), mm16(slice(tblk(3, 2)), X22, z4), z4);
        __builtin_amdgcn_sched_barrier(0);
        X20 = -mm16(slice(tblk(2, 2)), mm16(slice(tblk(2, 1)), X10, mm16(slice(tblk(2, 0)), X00, z4)), z4);
        X31 = -mm16(slice(tblk(3, 3)), mm16(slice(tblk(3, 2)), X21, mm16(slice(tblk(3, 1)), X11, z4)), z4);
    }
    __builtin_amdgcn_sched_barrier(0);
    X30 = -mm16(slice(tblk(3, 3)),
                mm16(slice(tblk(3, 2)), X20, mm16(slice(tblk(3, 1)), X10, mm16(slice(tblk(3, 0)), X00, z4))), z4);
    // this lane's column of its diagonal block, for T
    float xd[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xd[i] = Ab[tblk(g, g) + i * TB_ROW + l16];
    __syncthreads();  // A and X_bb are read: the blocks' area takes T

    // T = X diag(beta) in bf16 into LDS (row i, column j at its permuted
    // position), then out in whole rows of 16-byte pieces
    u16* Ts = reinterpret_cast<u16*>(Ab);
#pragma unroll
    for (int k = 0; k < 8; ++k) reinterpret_cast<uint4*>(Ts)[k * 64 + lane] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    {
        const float bc = bes[16 * g + l16];  // diagonal block g, column 16 g + l16
#pragma unroll
        for (int i = 0; i < 16; ++i) Ts[(16 * g + i) * 64 + pipe::perm_pos(16 * g + l16)] = f2bf(xd[i] * bc);
    }
    auto put = [&](int ib, int jb, const f32x4& X) __attribute__((always_inline)) {
        const int j = 16 * jb + l16;
        const float bj = bes[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) Ts[(16 * ib + 4 * g + e) * 64 + pipe::perm_pos(j)] = f2bf(X[e] * bj);
    };
    put(1, 0, X10);
    put(2, 1, X21);
    put(3, 2, X32);
    put(2, 0, X20);
    put(3, 1, X31);
    put(3, 0, X30);
    __syncthreads();
    uint4* T = reinterpret_cast<uint4*>(p.T + chunk * 64 * 64);
#pragma unroll
    for (int k = 0; k < 8; ++k) T[k * 64 + lane] = reinterpret_cast<const uint4*>(Ts)[k * 64 + lane];
}

template <int DK>
static hipError_t delta_transform_dk(const DeltaPrepParams& p, hipStream_t s) {
    hipLaunchKernelGGL((delta_transform_kernel<DK>), dim3((unsigned)(p.BH * p.N)), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t run_delta_transform(const DeltaPrepParams& p, hipStream_t s) {
    switch (p.dk) {
        case 64: return delta_transform_dk<64>(p, s);
        case 128: return delta_transform_dk<128>(p, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// forward: one workgroup per (head, 64 value columns), chunks in order
// ---------------------------------------------------------------------------
template <int DK>
struct alignas(16) DeltaStage {
    u16 q[64 * DK];
    u16 k[64 * DK];
    u16 v[64 * 64];  // V columns of the tile; each wave's output replaces its own 16 columns
    u16 t[64 * 64];  // T of the chunk (columns in operand order)
    float lg[64];    // log2 of the gates' product up to each row
};

// Eight waves, two per SIMD.  Waves 0-3 (state waves) own 16 value columns of
// the state each and run the chain that depends on it; waves 4-7 (prep waves)
// do everything that does not: every copy and output store, and the shared
// score tile (tril(Q K^T) * G) of the chunk, on the same SIMDs, so each
// SIMD has a second wave to issue while the other waits.  Two barriers per
// chunk n:
//   B1(n): chunk n has landed; the state waves are done with chunk n - 1 (its
//          output rows are in its stage, the score tile is free);
//   B2(n): the score tile of chunk n is complete.
// Between B1(n) and B2(n) the state waves compute K P, Q P, R and U = T R
// while the prep waves compute the score tile; between B2(n) and B1(n + 1)
// the state waves finish the chunk (intra product, outputs, state update)
// while the prep waves store the outputs of chunk n - 1, refill its stage with
// chunk n + NSTAGE - 1 and wait for chunk n + 1.
template <int DK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void delta_fwd_kernel(DeltaFwdParams p) {
    using namespace pipe;
    constexpr int QSEG = DK / 8, NKA = DK / 32;
    typedef DeltaStage<DK> StageT;
    constexpr int SBYTES = 64 * 64 * 2;
    constexpr int NFIT = (int)((160 * 1024 - SBYTES) / sizeof(StageT));
    constexpr int NSTAGE = NFIT < 4 ? NFIT : 4;
    constexpr int NQ = QSEG / 4;  // copy instructions per chunk and prep wave: Q (and K)
    constexpr int NV = 2, NTR = 2;  // V, T
    constexpr int NL = 2 * NQ + NV + NTR + 1;  // + the gate logs
    static_assert(NSTAGE >= 2 && (NSTAGE - 2) * NL < 64, "stages and vmcnt range");

    __shared__ StageT st[NSTAGE];
    __shared__ __attribute__((aligned(16))) u16 stile[64 * 64];  // (tril(Q K^T) * G), columns in operand order

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);  // wave-uniform
    const bool prep = wave >= 4;
    const int pw = wave & 3;  // prep waves: share of the copies and score blocks; state waves: column block
    const int lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int wi = work_index(p.xcd_remap);
    const int jt = wi % p.n_dvt;
    const int64_t bh = wi / p.n_dvt;
    const int col0 = jt * 64, cw = 16 * pw;
    const int64_t L = p.L, N = p.N;
    const int dv = p.dv;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    auto valid_of = [&](int64_t n) -> int { return (int)(L - n * 64 < 64 ? L - n * 64 : 64); };

    if (prep) {
        // ================= prep wave pw =================
        // this wave's share of the copies of chunk n (rows past the end clamped to the last row)
        auto issue = [&](int64_t n, StageT& s) __attribute__((always_inline)) {
            const int64_t r0 = n * 64;
            const int last = (int)(L - 1 - r0);
            const u16* qb = p.q + (bh * L + r0) * DK;
            const u16* kb = p.k + (bh * L + r0) * DK;
            const u16* vb = p.v + (bh * L + r0) * dv + col0;
            const u16* tb = p.T + (bh * N + n) * 64 * 64;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int b = pw * NQ + i, slot = b * WAVE + lane;
                const int r = slot / QSEG, seg = (slot % QSEG) ^ (r & (QSEG - 1));
                const uint32_t off = (uint32_t)(((r < last ? r : last) * DK + seg * 8) * 2);
                dma16(qb, off, lds_addr(s.q) + b * WAVE * 16);
                dma16(kb, off, lds_addr(s.k) + b * WAVE * 16);
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int b = pw * NV + i, slot = b * WAVE + lane;
                const int r = slot / 8, seg = (slot % 8) ^ (r & 7);
                dma16(vb, (uint32_t)(((r < last ? r : last) * dv + seg * 8) * 2), lds_addr(s.v) + b * WAVE * 16);
            }
#pragma unroll
            for (int i = 0; i < NTR; ++i) {
                const int b = pw * NTR + i, slot = b * WAVE + lane;
                const int r = slot / 8, seg = (slot % 8) ^ (r & 7);
                dma16(tb, (uint32_t)((r * 64 + seg * 8) * 2), lds_addr(s.t) + b * WAVE * 16);
            }
            // 256 bytes of gate logs: four 16-byte pieces per prep wave
            if (lane < 4) dma16(p.lg + (bh * N + n) * 64, (uint32_t)((pw * 4 + lane) * 16), lds_addr(s.lg) + pw * 64);
        };
        // wait until this wave's copies of chunk n have landed (loads complete in
        // order; later chunks' copies and the output stores may be in flight)
        auto land = [&](int64_t n) __attribute__((always_inline)) {
            const int64_t issued = n + NSTAGE - 2 < N - 1 ? n + NSTAGE - 2 : N - 1;  // newest chunk issued
            const int after = (int)(issued - n);
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
        // output rows of a chunk from the V tile of its stage: piece (pw * 2 + i) * 64 + lane
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        auto read_out = [&](const StageT& s, u32x4 (&ob)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int piece = (pw * 2 + i) * WAVE + lane, r = piece / 8, seg = piece % 8;
                ob[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(s.v) + tile_off<8>(r, seg * 8));
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage may be refilled
        };
        auto store_out = [&](int64_t n, const u32x4 (&ob)[2]) __attribute__((always_inline)) {
            const int valid = valid_of(n);
            u16* o = p.o + (bh * L + n * 64) * dv + col0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int piece = (pw * 2 + i) * WAVE + lane, r = piece / 8, seg = piece % 8;
                if (r < valid)
                    __builtin_nontemporal_store(ob[i], reinterpret_cast<u32x4*>(o + (int64_t)r * dv + seg * 8));
            }
        };
        // (tril(Q K^T) * G) blocks (ib, jb), jb <= ib: blocks b = pw, pw + 4,
        // pw + 8 of the ten, three independent chains.  The intra product reads
        // 32 keys at a time, so query blocks 0 and 2 also read the blocks above
        // the diagonal (0, 1) and (2, 3): prep waves 2 and 3, which have only two
        // blocks, write those as zeros (their third chain repeats a block of
        // their own and is not stored).
        auto score_tile = [&](const StageT& s) __attribute__((always_inline)) {
            int ib3[3], jb3[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int b = t < 2 || pw < 2 ? pw + 4 * t : pw;
                ib3[t] = b < 1 ? 0 : (b < 3 ? 1 : (b < 6 ? 2 : 3));
                jb3[t] = b - ib3[t] * (ib3[t] + 1) / 2;
            }
            f32x4 acc[3] = {zero4, zero4, zero4};
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks) {
                bf16x8 qa[3], kb[3];
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    qa[t] = row_op<QSEG>(s.q, 16 * ib3[t] + l16, 32 * ks, g);
                    kb[t] = row_op<QSEG>(s.k, 16 * jb3[t] + l16, 32 * ks, g);
                }
#pragma unroll
                for (int t = 0; t < 3; ++t) acc[t] = mfma_bf16(qa[t], kb[t], acc[t]);
            }
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const bool zero_block = t == 2 && pw >= 2;
                const int ib = zero_block ? (pw == 2 ? 0 : 2) : ib3[t];
                const int j = zero_block ? 16 * (ib + 1) + l16 : 16 * jb3[t] + l16;
                const float lgj = s.lg[j];
                const float4 lgi = *reinterpret_cast<const float4*>(s.lg + 16 * ib + 4 * g);
                const float li[4] = {lgi.x, lgi.y, lgi.z, lgi.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * ib + 4 * g + e;
                    const float val = !zero_block && j <= i ? acc[t][e] * __builtin_amdgcn_exp2f(li[e] - lgj) : 0.f;
                    *reinterpret_cast<u16*>(reinterpret_cast<char*>(stile) + tile_off<8>(i, perm_pos(j))) = f2bf(val);
                }
            }
        };

#pragma unroll
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (s0 < N) issue(s0, st[s0]);
        land(0);
        int si = 0;  // stage of chunk n
        for (int64_t n = 0; n < N; ++n) {
            const int sp = si == 0 ? NSTAGE - 1 : si - 1;  // stage of chunk n - 1 (and of chunk n + NSTAGE - 1)
            __syncthreads();  // B1(n)
            score_tile(st[si]);
            __syncthreads();  // B2(n)
            u32x4 ob[2];
            if (n > 0) read_out(st[sp], ob);
            if (n + NSTAGE - 1 < N) issue(n + NSTAGE - 1, st[sp]);
            if (n > 0) store_out(n - 1, ob);
            if (n + 1 < N) land(n + 1);
            si = si == NSTAGE - 1 ? 0 : si + 1;
        }
        __syncthreads();  // B1(N): the last chunk's output is in its stage
        const int sl = si == 0 ? NSTAGE - 1 : si - 1;
        u32x4 ob[2];
        read_out(st[sl], ob);
        store_out(N - 1, ob);
        return;
    }

    // ================= state wave pw: value columns cw .. cw + 15 =================
    const int c8 = 8 * (lane & 3);
    // P[ks][hf] lane (l16, g) element e = P[a = 32 ks + 8 g + 4 hf + e][c = col0 + cw + l16]
    f32x4 P[NKA][2];
#pragma unroll
    for (int ks = 0; ks < NKA; ++ks) P[ks][0] = P[ks][1] = zero4;

    int si = 0;
    for (int64_t n = 0; n < N; ++n) {
        StageT& s = st[si];
        const int valid = valid_of(n);
        const char* vbytes = reinterpret_cast<const char*>(s.v);
        __syncthreads();  // B1(n)
        bf16x8 pst[NKA];
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) pst[ks] = pack_acc_bf16(P[ks][0], P[ks][1]);
        // K P and Q P for this wave's 16 columns: lane holds row 16 ib + 4g + e, column cw + l16
        f32x4 X[4], O[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) X[ib] = O[ib] = zero4;
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                X[ib] = mfma_bf16(row_op<QSEG>(s.k, 16 * ib + l16, 32 * ks, g), pst[ks], X[ib]);
                O[ib] = mfma_bf16(row_op<QSEG>(s.q, 16 * ib + l16, 32 * ks, g), pst[ks], O[ib]);
            }
        // R = V - diag(g) K P; the inter part times g_i
        f32x4 R[4];
        float gl[4][4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            const float4 l4 = *reinterpret_cast<const float4*>(s.lg + 16 * ib + 4 * g);
            gl[ib][0] = l4.x;
            gl[ib][1] = l4.y;
            gl[ib][2] = l4.z;
            gl[ib][3] = l4.w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ib + 4 * g + e;
                const float gi = __builtin_amdgcn_exp2f(gl[ib][e]);
                const float vv = bf2f(*reinterpret_cast<const u16*>(vbytes + tile_off<8>(i, cw + l16)));
                R[ib][e] = fmaf(-gi, X[ib][e], vv);
                O[ib][e] *= gi;
            }
        }
        // U = T R (T lower triangular: key steps up to the query block's own)
        const bf16x8 Rp[2] = {pack_acc_bf16(R[0], R[1]), pack_acc_bf16(R[2], R[3])};
        f32x4 U[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            U[ib] = zero4;
#pragma unroll
            for (int ks = 0; ks <= ib / 2; ++ks) U[ib] = mfma_bf16(row_op<8>(s.t, 16 * ib + l16, 32 * ks, g), Rp[ks], U[ib]);
        }
        __syncthreads();  // B2(n): the score tile is complete
        // O += (tril(Q K^T) * G) U
        const bf16x8 Up[2] = {pack_acc_bf16(U[0], U[1]), pack_acc_bf16(U[2], U[3])};
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int ks = 0; ks <= ib / 2; ++ks) O[ib] = mfma_bf16(row_op<8>(stile, 16 * ib + l16, 32 * ks, g), Up[ks], O[ib]);
        // the output rows into this wave's own V columns (its last V read is above)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<u16*>(reinterpret_cast<char*>(s.v) + tile_off<8>(16 * ib + 4 * g + e, cw + l16)) =
                    f2bf(O[ib][e]);
        // P <- g_n P + K^T diag(g_n / g) U (rows past the end weigh 0)
        const float lgn = s.lg[63];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ib + 4 * g + e;
                U[ib][e] *= i < valid ? __builtin_amdgcn_exp2f(lgn - gl[ib][e]) : 0.f;
            }
        const bf16x8 Uw[2] = {pack_acc_bf16(U[0], U[1]), pack_acc_bf16(U[2], U[3])};
        const float gn = __builtin_amdgcn_exp2f(lgn);
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks) {
            P[ks][0] *= gn;
            P[ks][1] *= gn;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    P[ks][hf] = mfma_bf16(col_op<QSEG>(s.k, 32 * kk, 32 * ks + c8 + 4 * hf, lane), Uw[kk], P[ks][hf]);
        si = si == NSTAGE - 1 ? 0 : si + 1;
    }
    __syncthreads();  // B1(N)
    if (p.S_final != nullptr) {
        float* Sf = p.S_final + (bh * DK) * (int64_t)dv + col0 + cw + l16;
#pragma unroll
        for (int ks = 0; ks < NKA; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sf[(int64_t)(32 * ks + 8 * g + 4 * hf + e) * dv] = P[ks][hf][e];
    }
}

hipError_t run_delta_fwd(const DeltaFwdParams& p, hipStream_t s) {
    const int64_t grid = p.BH * p.n_dvt;
    switch (p.dk) {
        case 64:
            hipLaunchKernelGGL((delta_fwd_kernel<64>), dim3((unsigned)grid), dim3(512), 0, s, p);
            break;
        case 128:
            hipLaunchKernelGGL((delta_fwd_kernel<128>), dim3((unsigned)grid), dim3(512), 0, s, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace la
