// Feature maps phi(in_scale * x), row by row (page "Linear Attention /
// Performerの理論と実装": the ELU feature map and FAVOR+ positive random
// features).
//
//  * identity and elu+1 are elementwise (8 bf16 per thread, fp32 math); with a
//    bf16 output they can also write the bf16 residual y - bf16(y).
//  * FAVOR+ is a small GEMM x W^T (k = d_in) on bf16 matrix cores with an
//    fp32 epilogue exp(proj - |x|^2 / 2) / sqrt(m).  W stays in LDS for the
//    life of the workgroup, which walks row tiles of 64.
#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

__global__ __launch_bounds__(256) void fmap_elementwise(FmapParams p) {
    const int64_t units = p.rows * p.d_in / 8;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * blockDim.x) {
        const uint4 raw = reinterpret_cast<const uint4*>(p.x)[u];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = p.in_scale * __uint_as_float(w[j] << 16);
            f[2 * j + 1] = p.in_scale * __uint_as_float(w[j] & 0xFFFF0000u);
        }
        if (p.fmap == 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = elu1(f[j]);
        }
        if (p.y_f32) {
            float4* y = reinterpret_cast<float4*>(p.y) + 2 * u;
            y[0] = make_float4(f[0], f[1], f[2], f[3]);
            y[1] = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            uint32_t hb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) hb[j] = pack2_bf16(f[2 * j], f[2 * j + 1]);
            reinterpret_cast<uint4*>(p.y)[u] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
            if (p.y_lo != nullptr) {
                // residual y - bf16(y), so that hi + lo carries y to about 2^-17
                uint32_t lb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lb[j] = pack2_bf16(f[2 * j] - __uint_as_float(hb[j] << 16),
                                       f[2 * j + 1] - __uint_as_float(hb[j] & 0xFFFF0000u));
                reinterpret_cast<uint4*>(p.y_lo)[u] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
            }
        }
    }
}

// FAVOR+: DINP = d_in padded to a multiple of 32 (columns past d_in are zero).
template <int DINP>
__global__ __launch_bounds__(256) void fmap_favor(FmapParams p) {
    constexpr int RT = 64;          // rows per tile
    constexpr int XS = DINP + 8;    // LDS row stride (elements)
    constexpr int MMAX = 256;
    constexpr int NKS = DINP / 32;
    __shared__ __attribute__((aligned(16))) u16 Ws[MMAX * XS];
    __shared__ __attribute__((aligned(16))) u16 Xs[RT * XS];
    __shared__ float half_sq[RT];

    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    const int m = p.m, din = p.d_in;
    const float s = p.in_scale;
    const float inv_sqrt_m = 1.0f / sqrtf((float)m);

    // W -> LDS (zero-padded columns)
    for (int idx = tid; idx < m * (DINP / 8); idx += 256) {
        const int r = idx / (DINP / 8), cg = idx % (DINP / 8);
        uint4 val = make_uint4(0, 0, 0, 0);
        if (cg * 8 < din) val = *reinterpret_cast<const uint4*>(p.W + (int64_t)r * din + cg * 8);
        *reinterpret_cast<uint4*>(Ws + r * XS + cg * 8) = val;
    }

    const int64_t n_tiles = (p.rows + RT - 1) / RT;
    for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        const int64_t r0 = tile * RT;
        __syncthreads();  // previous tile's readers done (and W written)
        for (int idx = tid; idx < RT * (DINP / 8); idx += 256) {
            const int r = idx / (DINP / 8), cg = idx % (DINP / 8);
            uint4 val = make_uint4(0, 0, 0, 0);
            if (r0 + r < p.rows && cg * 8 < din)
                val = *reinterpret_cast<const uint4*>(p.x + (r0 + r) * din + cg * 8);
            *reinterpret_cast<uint4*>(Xs + r * XS + cg * 8) = val;
        }
        __syncthreads();
        if (tid < RT) {
            float acc = 0.f;
            for (int c = 0; c < DINP; ++c) {
                const float xv = bf2f(Xs[tid * XS + c]);
                acc += xv * xv;
            }
            half_sq[tid] = 0.5f * s * s * acc;
        }
        __syncthreads();
        // wave w: rows 16w .. 16w+15, all m features
        bf16x8 a[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            a[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(Xs + (wave * 16 + l16) * XS + ks * 32 + g * 8));
        for (int nb = 0; nb < m / 16; ++nb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(Ws + (nb * 16 + l16) * XS + ks * 32 + g * 8));
                acc = mfma_bf16(a[ks], b, acc);
            }
            // acc[i] = x[row 16w + 4g + i] . W[feature 16nb + l16]
            const int feat = nb * 16 + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wave * 16 + g * 4 + i;
                if (r0 + r < p.rows) {
                    const float y = __expf(s * acc[i] - half_sq[r]) * inv_sqrt_m;
                    const int64_t off = (r0 + r) * m + feat;
                    if (p.y_f32) {
                        reinterpret_cast<float*>(p.y)[off] = y;
                    } else {
                        const u16 hb = f2bf(y);
                        reinterpret_cast<u16*>(p.y)[off] = hb;
                        if (p.y_lo != nullptr) p.y_lo[off] = f2bf(y - bf2f(hb));
                    }
                }
            }
        }
    }
}

hipError_t run_feature_map(const FmapParams& p, hipStream_t s) {
    if (p.fmap == 2) {
        const int64_t n_tiles = (p.rows + 63) / 64;
        const unsigned grid = (unsigned)(n_tiles < 2048 ? n_tiles : 2048);
        const int dinp = p.d_in <= 32 ? 32 : (p.d_in <= 64 ? 64 : 128);
        switch (dinp) {
            case 32: hipLaunchKernelGGL(fmap_favor<32>, dim3(grid), dim3(256), 0, s, p); break;
            case 64: hipLaunchKernelGGL(fmap_favor<64>, dim3(grid), dim3(256), 0, s, p); break;
            default: hipLaunchKernelGGL(fmap_favor<128>, dim3(grid), dim3(256), 0, s, p); break;
        }
    } else {
        const int64_t units = p.rows * p.d_in / 8;
        int64_t blocks = (units + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(fmap_elementwise, dim3((unsigned)blocks), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace la
