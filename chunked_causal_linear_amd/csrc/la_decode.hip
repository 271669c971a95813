// One recurrent decode step for many independent states:
//     S = gamma S + phi(k) v^T ;  z = gamma z + phi(k) ;  o = phi(q)^T S [/ phi(q)^T z]
// (update, then read: the RNN view on the page "Linear Attention /
// Performerの理論と実装" and the token-by-token form on the page "attention
// と線形の間", section ②; gamma < 1 is the decayed recurrence the first page
// gives for Retention, gamma = 1 plain linear attention).
//
// The step is a read-modify-write stream over the fp32 states; a workgroup of
// 256 threads walks NS states, keeping the FAVOR+ projection W in LDS for all
// of them.  For one state, thread t owns four value columns (j4 = t % (DV/4))
// of the rows a = t / (DV/4) + AG * i, so every S access is a coalesced
// 16-byte vector and the row partial sums of o reduce through LDS.
#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

// WIN: the largest FAVOR+ input width the LDS copy of W holds (64 or 128;
// the smaller copy lets four workgroups share a CU instead of two)
template <int DK, int DV, bool FAV, int WIN>
__global__ __launch_bounds__(256) void recurrent_step_kernel(DecodeParams p, int ns_per_block) {
    constexpr int NT = 256;
    constexpr int J4 = DV / 4;          // float4 column groups
    constexpr int AG = NT / J4;         // row groups
    constexpr int RPT = DK / AG > 0 ? DK / AG : 1;  // rows per thread
    constexpr int DINMAX = 256;
    constexpr int WMAX = FAV ? DK * WIN : 8;  // FAVOR+ projection, d_in <= WIN
    static_assert(AG * J4 == NT, "thread layout");

    __shared__ float fq[DK], fk[DK], vv[DV];
    __shared__ float xq[DINMAX], xk[DINMAX];
    __shared__ float red[AG][DV + 1];
    __shared__ float sums[4];
    __shared__ u16 Ws[WMAX];  // FAVOR+ projection (m x d_in)

    const int tid = threadIdx.x;
    const float gam = p.gamma;  // 1 without the decay
    const int j4 = tid % J4, ag = tid / J4;
    const int din = p.d_in;
    const float s = p.in_scale;

    if (FAV) {
        for (int i = tid; i < p.dk * din; i += NT) Ws[i] = p.W[i];
    }

    for (int it = 0; it < ns_per_block; ++it) {
        const int64_t st = (int64_t)blockIdx.x * ns_per_block + it;
        if (st >= p.n) break;
        __syncthreads();
        for (int i = tid; i < din; i += NT) {
            xq[i] = s * bf2f(p.q[st * din + i]);
            xk[i] = s * bf2f(p.k[st * din + i]);
        }
        for (int i = tid; i < DV; i += NT) vv[i] = bf2f(p.v[st * DV + i]);
        if (tid < 4) sums[tid] = 0.f;
        __syncthreads();
        if (FAV) {
            // |x|^2 / 2 for q (wave 0) and k (wave 1)
            if (tid < 128) {
                const float* x = tid < 64 ? xq : xk;
                float acc = 0.f;
                for (int i = tid % 64; i < din; i += 64) acc += x[i] * x[i];
                for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
                if ((tid % 64) == 0) sums[tid / 64] = 0.5f * acc;
            }
            __syncthreads();
            const float inv_sqrt_m = 1.0f / sqrtf((float)DK);
            for (int a = tid; a < DK; a += NT) {
                float pq = 0.f, pk = 0.f;
                for (int c = 0; c < din; ++c) {
                    const float wv = bf2f(Ws[a * din + c]);
                    pq += wv * xq[c];
                    pk += wv * xk[c];
                }
                fq[a] = __expf(pq - sums[0]) * inv_sqrt_m;
                fk[a] = __expf(pk - sums[1]) * inv_sqrt_m;
            }
        } else {
            for (int a = tid; a < DK; a += NT) {
                fq[a] = p.fmap == 1 ? elu1(xq[a]) : xq[a];
                fk[a] = p.fmap == 1 ? elu1(xk[a]) : xk[a];
            }
        }
        __syncthreads();

        // S update and partial read
        float4* S = reinterpret_cast<float4*>(p.S + st * DK * DV);
        const float4 v4 = make_float4(vv[4 * j4], vv[4 * j4 + 1], vv[4 * j4 + 2], vv[4 * j4 + 3]);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 cur[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int a = ag + AG * i;
            if (a < DK) cur[i] = S[a * J4 + j4];
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int a = ag + AG * i;
            if (a < DK) {
                const float kk = fk[a], qq = fq[a];
                float4 x = cur[i];
                x.x = fmaf(kk, v4.x, gam * x.x);
                x.y = fmaf(kk, v4.y, gam * x.y);
                x.z = fmaf(kk, v4.z, gam * x.z);
                x.w = fmaf(kk, v4.w, gam * x.w);
                S[a * J4 + j4] = x;
                acc.x += qq * x.x;
                acc.y += qq * x.y;
                acc.z += qq * x.z;
                acc.w += qq * x.w;
            }
        }
        red[ag][4 * j4] = acc.x;
        red[ag][4 * j4 + 1] = acc.y;
        red[ag][4 * j4 + 2] = acc.z;
        red[ag][4 * j4 + 3] = acc.w;

        // z update and the denominator
        float dpart = 0.f;
        if (p.normalize && p.z != nullptr) {
            for (int a = tid; a < DK; a += NT) {
                const float zn = fmaf(gam, p.z[st * DK + a], fk[a]);
                p.z[st * DK + a] = zn;
                dpart += fq[a] * zn;
            }
            for (int o = 32; o > 0; o >>= 1) dpart += __shfl_xor(dpart, o);
            if ((tid % 64) == 0) atomicAdd(&sums[2], dpart);
        }
        __syncthreads();
        if (tid < DV) {
            float o = 0.f;
            for (int r = 0; r < AG; ++r) o += red[r][tid];
            if (p.normalize) o = o / sums[2];
            if (p.out_f32)
                reinterpret_cast<float*>(p.o)[st * DV + tid] = o;
            else
                reinterpret_cast<u16*>(p.o)[st * DV + tid] = f2bf(o);
        }
    }
}

template <int DK, int DV>
static void launch_decode(const DecodeParams& p, unsigned grid, int nsb, hipStream_t s) {
    if (p.fmap == 2 && p.d_in <= 64)
        hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, true, 64>), dim3(grid), dim3(256), 0, s, p, nsb);
    else if (p.fmap == 2)
        hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, true, 128>), dim3(grid), dim3(256), 0, s, p, nsb);
    else
        hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, false, 64>), dim3(grid), dim3(256), 0, s, p, nsb);
}

template <int DK>
static hipError_t decode_dv(const DecodeParams& p, unsigned grid, int nsb, hipStream_t s) {
    switch (p.dv) {
        case 16: launch_decode<DK, 16>(p, grid, nsb, s); break;
        case 32: launch_decode<DK, 32>(p, grid, nsb, s); break;
        case 64: launch_decode<DK, 64>(p, grid, nsb, s); break;
        case 128: launch_decode<DK, 128>(p, grid, nsb, s); break;
        case 256: launch_decode<DK, 256>(p, grid, nsb, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t run_recurrent_step(const DecodeParams& p, hipStream_t s) {
    // several states per workgroup amortise the W load (FAVOR+); otherwise one
    const int nsb = p.fmap == 2 ? 4 : 1;
    const unsigned grid = (unsigned)((p.n + nsb - 1) / nsb);
    switch (p.dk) {
        case 16: return decode_dv<16>(p, grid, nsb, s);
        case 32: return decode_dv<32>(p, grid, nsb, s);
        case 64: return decode_dv<64>(p, grid, nsb, s);
        case 128: return decode_dv<128>(p, grid, nsb, s);
        case 256: return decode_dv<256>(p, grid, nsb, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace la

namespace la {

// Exact int8 decode step (the int8 path of the forward, one token): S += k^T v
// and o = q S, every product and sum in wrapping 32-bit arithmetic, so the
// results are exact modulo 2^32 and therefore exact whenever they fit int32 -
// the int8 forward's convention.  One workgroup per state; thread t owns four
// value columns (j4 = t % (DV / 4)) of the rows t / (DV / 4) + AG i, so every
// state access is a 16-byte vector; the row partial sums of o reduce through
// LDS.
template <int DV>
__global__ __launch_bounds__(256) void recurrent_step_i8_kernel(DecodeParamsI8 p) {
    constexpr int NT = 256, J4 = DV / 4, AG = NT / J4;
    static_assert(J4 * AG == NT, "thread layout");
    __shared__ int qs[256], ks[256], vs[DV];
    __shared__ unsigned red[AG][DV + 4];
    const int tid = threadIdx.x;
    const int j4 = tid % J4, ag = tid / J4;
    const int64_t st = blockIdx.x;
    const int dk = p.dk;
    for (int i = tid; i < dk; i += NT) {
        qs[i] = p.q[st * dk + i];
        ks[i] = p.k[st * dk + i];
    }
    for (int i = tid; i < DV; i += NT) vs[i] = p.v[st * DV + i];
    __syncthreads();
    const unsigned v0 = (unsigned)vs[4 * j4], v1 = (unsigned)vs[4 * j4 + 1], v2 = (unsigned)vs[4 * j4 + 2],
                   v3 = (unsigned)vs[4 * j4 + 3];
    uint4* S = reinterpret_cast<uint4*>(p.S) + st * (int64_t)dk * J4;
    uint4 part = make_uint4(0u, 0u, 0u, 0u);
    for (int a = ag; a < dk; a += AG) {
        uint4 x = S[(int64_t)a * J4 + j4];
        const unsigned ka = (unsigned)ks[a], qa = (unsigned)qs[a];
        x.x += ka * v0;
        x.y += ka * v1;
        x.z += ka * v2;
        x.w += ka * v3;
        S[(int64_t)a * J4 + j4] = x;
        part.x += qa * x.x;
        part.y += qa * x.y;
        part.z += qa * x.z;
        part.w += qa * x.w;
    }
    red[ag][4 * j4] = part.x;
    red[ag][4 * j4 + 1] = part.y;
    red[ag][4 * j4 + 2] = part.z;
    red[ag][4 * j4 + 3] = part.w;
    __syncthreads();
    for (int c = tid; c < DV; c += NT) {
        unsigned sum = 0u;
        for (int r = 0; r < AG; ++r) sum += red[r][c];
        p.o[st * DV + c] = (int)sum;
    }
}

hipError_t run_recurrent_step_i8(const DecodeParamsI8& p, hipStream_t s) {
    if (p.n < 1 || p.n > 0x7FFFFFFFLL || p.dk < 1 || p.dk > 256) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.n);
    switch (p.dv) {
        case 16: hipLaunchKernelGGL(recurrent_step_i8_kernel<16>, grid, dim3(256), 0, s, p); break;
        case 32: hipLaunchKernelGGL(recurrent_step_i8_kernel<32>, grid, dim3(256), 0, s, p); break;
        case 64: hipLaunchKernelGGL(recurrent_step_i8_kernel<64>, grid, dim3(256), 0, s, p); break;
        case 128: hipLaunchKernelGGL(recurrent_step_i8_kernel<128>, grid, dim3(256), 0, s, p); break;
        case 256: hipLaunchKernelGGL(recurrent_step_i8_kernel<256>, grid, dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace la
