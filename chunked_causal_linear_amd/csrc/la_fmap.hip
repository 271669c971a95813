// Feature maps phi(in_scale * x), row by row (page "Linear Attention /
// Performerの理論と実装": the ELU feature map and FAVOR+ positive random
// features).
//
//  * identity and elu+1 are elementwise (8 bf16 per thread, fp32 math); with a
//    bf16 output they can also write the bf16 residual y - bf16(y).
//  * FAVOR+ is a small GEMM x W^T (k = d_in) on bf16 matrix cores with an
//    fp32 epilogue exp(proj - |x|^2 / 2) / sqrt(m) (one exp2 of a fused
//    multiply-add per feature).  W stays in LDS for the
//    life of the workgroup, whose waves walk slabs of 16 rows.
#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

__global__ __launch_bounds__(256) void fmap_elementwise(FmapParams p) {
    const int64_t units = p.rows * p.d_in / 8;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * blockDim.x) {
        const uint4 raw = load_nt(reinterpret_cast<const uint4*>(p.x) + u);
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
            store_nt(reinterpret_cast<uint4*>(p.y) + u, make_uint4(hb[0], hb[1], hb[2], hb[3]));
            if (p.y_lo != nullptr) {
                // residual y - bf16(y), so that hi + lo carries y to about 2^-17
                uint32_t lb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lb[j] = pack2_bf16(f[2 * j] - __uint_as_float(hb[j] << 16),
                                       f[2 * j + 1] - __uint_as_float(hb[j] & 0xFFFF0000u));
                store_nt(reinterpret_cast<uint4*>(p.y_lo) + u, make_uint4(lb[0], lb[1], lb[2], lb[3]));
            }
        }
    }
}

// FAVOR+: DINP = d_in padded to a multiple of 32 (columns past d_in are zero).
// W (m x d_in) stays in LDS; every wave walks slabs of 16 rows on its own
// (the next slab's rows are loaded while the current one is mapped): the
// slab's x rows go straight into registers as matrix-core operands, the
// product is taken as (W x^T) so that a lane ends with four consecutive
// features of one row (16 nb + 4g + i, row l16), and |x|^2 of the row is summed
// from the same operand registers.  bf16 results are staged per wave in LDS and
// leave as 16-byte stores with consecutive lanes on consecutive addresses
// (whole rows per instruction: a row's pieces spread over several instructions
// wrote at two thirds of the rate).  No barrier after W is in.
// M = m features (16 MB), fixed at compile time so the feature loop has no
// run-time bounds.
template <int DINP, int MB>
__global__ __launch_bounds__(256) void fmap_favor(FmapParams p) {
    constexpr int XS = DINP + 8;    // LDS row stride of W (elements)
    constexpr int M = 16 * MB;
    constexpr int NKS = DINP / 32;
    constexpr int YS = M + 8;       // staging row stride (elements)
    __shared__ __attribute__((aligned(16))) u16 Ws[M * XS];
    __shared__ __attribute__((aligned(16))) u16 Ys[4][16 * YS];

    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE, l16 = lane % 16, g = lane / 16;
    constexpr int m = M;
    const int din = p.d_in;
    const float s = p.in_scale;
    // exp(s w.x - s^2 |x|^2 / 2) / sqrt(m) = exp2(w.x sl - (s^2 |x|^2 / 2) log2(e) - log2(m) / 2):
    // one fused multiply-add and one exponential per feature
    constexpr float LOG2E = 1.4426950408889634f;
    const float sl = s * LOG2E;
    const float half_log2_m = 0.5f * log2f((float)m);
    u16* ys = Ys[wave];

    // W -> LDS (zero-padded columns)
    for (int idx = tid; idx < m * (DINP / 8); idx += 256) {
        const int r = idx / (DINP / 8), cg = idx % (DINP / 8);
        uint4 val = make_uint4(0, 0, 0, 0);
        if (cg * 8 < din) val = *reinterpret_cast<const uint4*>(p.W + (int64_t)r * din + cg * 8);
        *reinterpret_cast<uint4*>(Ws + r * XS + cg * 8) = val;
    }
    __syncthreads();

    const int64_t n_slabs = (p.rows + 15) / 16;
    const int64_t stride = (int64_t)gridDim.x * 4;
    // x[row][ks*32 + 8g .. +7] (zero past d_in or past the last row)
    auto load_x = [&](int64_t slab, uint4 (&u)[NKS]) {
        const int64_t row = slab * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u[ks] = make_uint4(0, 0, 0, 0);
            if (row < p.rows && ks * 32 + g * 8 < din) u[ks] = *reinterpret_cast<const uint4*>(p.x + row * din + ks * 32 + g * 8);
        }
    };
    // the staged 16 x m bf16 block of this slab to rows slab*16.. of dst
    constexpr int segs = M / 8;  // 16-byte pieces per row
    auto store_staged = [&](int64_t slab, u16* dst) {
        for (int e = lane; e < 16 * segs; e += WAVE) {
            const int r = e / segs, sg = e % segs;
            const int64_t row = slab * 16 + r;
            const uint4 val = *reinterpret_cast<const uint4*>(ys + r * YS + sg * 8);
            if (row < p.rows) store_nt(dst + row * m + sg * 8, val);
        }
    };

    int64_t slab = (int64_t)blockIdx.x * 4 + wave;
    uint4 xn[NKS];
    if (slab < n_slabs) load_x(slab, xn);
    for (; slab < n_slabs; slab += stride) {
        uint4 xc[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) xc[ks] = xn[ks];
        if (slab + stride < n_slabs) load_x(slab + stride, xn);
        const int64_t row = slab * 16 + l16;
        bf16x8 xb[NKS];
        float sq = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint32_t w[4] = {xc[ks].x, xc[ks].y, xc[ks].z, xc[ks].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = __uint_as_float(w[j] << 16), b = __uint_as_float(w[j] & 0xFFFF0000u);
                sq += a * a + b * b;
            }
            xb[ks] = as_bf16x8(xc[ks]);
        }
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        const float off = fmaf(0.5f * s * s * sq, LOG2E, half_log2_m);
        // y for features 16 nb + 4g + i of row l16 (kept in registers: the
        // residual pass reads them again)
        constexpr int NBM = MB;
        float y[NBM][4];
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 wb =
                    as_bf16x8(*reinterpret_cast<const uint4*>(Ws + (nb * 16 + l16) * XS + ks * 32 + g * 8));
                acc = mfma_bf16(wb, xb[ks], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) y[nb][i] = __builtin_amdgcn_exp2f(fmaf(acc[i], sl, -off));
        }
        if (p.y_f32) {
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb)
                if (row < p.rows)
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + row * m + nb * 16 + 4 * g) =
                        make_float4(y[nb][0], y[nb][1], y[nb][2], y[nb][3]);
            continue;
        }
        uint2 hb[NBM];
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            hb[nb] = make_uint2(pack2_bf16(y[nb][0], y[nb][1]), pack2_bf16(y[nb][2], y[nb][3]));
            *reinterpret_cast<uint2*>(ys + l16 * YS + nb * 16 + 4 * g) = hb[nb];
        }
        store_staged(slab, reinterpret_cast<u16*>(p.y));
        if (p.y_lo != nullptr) {
            // residual y - bf16(y), so that hi + lo carries y to about 2^-17
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb) {
                const uint2 h = hb[nb];
                *reinterpret_cast<uint2*>(ys + l16 * YS + nb * 16 + 4 * g) = make_uint2(
                    pack2_bf16(y[nb][0] - __uint_as_float(h.x << 16), y[nb][1] - __uint_as_float(h.x & 0xFFFF0000u)),
                    pack2_bf16(y[nb][2] - __uint_as_float(h.y << 16), y[nb][3] - __uint_as_float(h.y & 0xFFFF0000u)));
            }
            store_staged(slab, p.y_lo);
        }
    }
}

template <int DINP, int MB>
static void launch_favor(const FmapParams& p, hipStream_t s) {
    // four 16-row slabs per workgroup and round; as many workgroups as fit
    // the CUs at once (by LDS, at most four per CU), so W is loaded once per
    // resident workgroup
    constexpr int64_t lds = 2 * (16 * MB * (DINP + 8) + 4 * 16 * (16 * MB + 8));
    constexpr int64_t per_cu = 160 * 1024 / lds < 4 ? 160 * 1024 / lds : 4;
    const int64_t n_groups = (p.rows + 63) / 64;
    const int64_t cap = 256 * per_cu;
    const unsigned grid = (unsigned)(n_groups < cap ? n_groups : cap);
    hipLaunchKernelGGL((fmap_favor<DINP, MB>), dim3(grid), dim3(256), 0, s, p);
}

template <int DINP>
static void launch_favor_m(const FmapParams& p, hipStream_t s) {
    switch (p.m) {
        case 16: launch_favor<DINP, 1>(p, s); break;
        case 32: launch_favor<DINP, 2>(p, s); break;
        case 64: launch_favor<DINP, 4>(p, s); break;
        case 128: launch_favor<DINP, 8>(p, s); break;
        default: launch_favor<DINP, 16>(p, s); break;
    }
}

hipError_t run_feature_map(const FmapParams& p, hipStream_t s) {
    if (p.fmap == 2) {
        // m is a power of two in 16..256 (checked by the caller)
        const int dinp = p.d_in <= 32 ? 32 : (p.d_in <= 64 ? 64 : 128);
        switch (dinp) {
            case 32: launch_favor_m<32>(p, s); break;
            case 64: launch_favor_m<64>(p, s); break;
            default: launch_favor_m<128>(p, s); break;
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
