// Phase 2: exclusive prefix of the per-chunk states over chunks.
//
// P_0 = 0, P_n = P_{n-1} + S_{n-1}, done in place, plus the total (the state
// after the last chunk) - page "attention と線形の間", section ②: chunk n reads
// the state carried from every chunk before it, starting from zero.
//
// Elementwise-parallel over (head, state element); each thread walks the N
// chunks of four consecutive elements in order (a deterministic sum).  The
// loads of eight chunks are issued before their adds so that several reads are
// in flight per thread: the kernel is a pure HBM stream (read and write every
// per-chunk state once).  State sets larger than the caches are streamed with
// the non-temporal hint (6 % faster at 1 GB); smaller ones, which phase 1 has
// just written, are left to the caches.
#include <type_traits>

#include "la_common.hpp"
#include "la_kernels.hpp"

namespace la {

template <typename V4>
__device__ __forceinline__ V4 add4(const V4& a, const V4& b) {
    V4 r;
    r.x = a.x + b.x;
    r.y = a.y + b.y;
    r.z = a.z + b.z;
    r.w = a.w + b.w;
    return r;
}

// 16-byte state vectors, with the non-temporal hint when NT
template <bool NT, typename V4>
__device__ __forceinline__ V4 ld4(const V4* p) {
    if constexpr (NT) {
        const uint4 u = load_nt(p);
        return __builtin_bit_cast(V4, u);
    } else {
        return *p;
    }
}
template <bool NT, typename V4>
__device__ __forceinline__ void st4(V4* p, const V4& v) {
    if constexpr (NT)
        store_nt(p, __builtin_bit_cast(uint4, v));
    else
        *p = v;
}

// One launch scans two state sets of the same heads and chunk count: threads
// [0, BH E4) walk S (E4 vectors per chunk), the next BH Ez4 walk z (Ez4 per
// chunk; Ez4 = 0 when there is none).
template <typename V4, typename E, bool NT>
__global__ __launch_bounds__(256) void state_scan_kernel(V4* __restrict__ S, V4* __restrict__ total, int64_t E4,
                                                          V4* __restrict__ Z, V4* __restrict__ ztotal, int64_t Ez4,
                                                          int64_t N, int64_t BH) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * E4) {
        idx -= BH * E4;
        if (idx >= BH * Ez4) return;
        S = Z;
        total = ztotal;
        E4 = Ez4;
    }
    const int64_t bh = idx / E4, e = idx % E4;
    V4* base = S + bh * N * E4 + e;
    V4 run;
    run.x = run.y = run.z = run.w = E(0);
    constexpr int U = 8;
    int64_t n = 0;
    for (; n + U <= N; n += U) {
        V4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = ld4<NT>(base + (n + u) * E4);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            st4<NT>(base + (n + u) * E4, run);
            run = add4(run, x[u]);
        }
    }
    for (; n < N; ++n) {
        const V4 x = ld4<NT>(base + n * E4);
        st4<NT>(base + n * E4, run);
        run = add4(run, x);
    }
    if (total != nullptr) total[bh * E4 + e] = run;
}

// The decayed prefix (page "Linear Attention / Performerの理論と実装", the
// decayed recurrence): chunk n's state as it stands at the chunk's end enters
// after the carried state has decayed over the chunk's rows,
// P_n = gamma^len(n-1) P_{n-1} + S_{n-1}, len(n) = clamp(L - n Cs, 0, Cs).
// (S and z in one launch, split over the threads as above)
__global__ __launch_bounds__(256) void state_scan_decay_kernel(float4* __restrict__ S, float4* __restrict__ total,
                                                               int64_t E4, float4* __restrict__ Z,
                                                               float4* __restrict__ ztotal, int64_t Ez4, int64_t N,
                                                               int64_t BH, float lg, int64_t L, int64_t Cs) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * E4) {
        idx -= BH * E4;
        if (idx >= BH * Ez4) return;
        S = Z;
        total = ztotal;
        E4 = Ez4;
    }
    const int64_t bh = idx / E4, e = idx % E4;
    float4* base = S + bh * N * E4 + e;
    float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
    auto decay_of = [&](int64_t n) {
        int64_t len = L - n * Cs;
        len = len < 0 ? 0 : (len > Cs ? Cs : len);
        return __builtin_amdgcn_exp2f((float)len * lg);
    };
    constexpr int U = 8;
    int64_t n = 0;
    for (; n + U <= N; n += U) {
        float4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = base[(n + u) * E4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            base[(n + u) * E4] = run;
            const float a = decay_of(n + u);
            run = make_float4(fmaf(a, run.x, x[u].x), fmaf(a, run.y, x[u].y), fmaf(a, run.z, x[u].z),
                              fmaf(a, run.w, x[u].w));
        }
    }
    for (; n < N; ++n) {
        const float4 x = base[n * E4];
        base[n * E4] = run;
        const float a = decay_of(n);
        run = make_float4(fmaf(a, run.x, x.x), fmaf(a, run.y, x.y), fmaf(a, run.z, x.z), fmaf(a, run.w, x.w));
    }
    if (total != nullptr) total[bh * E4 + e] = run;
}

// Wrapping int32 adds (unsigned arithmetic) so overflow is defined.
struct WrapInt4 {
    unsigned x, y, z, w;
};

hipError_t run_state_scan(const ScanParams& p, int64_t BH, hipStream_t s) {
    const int64_t E4 = p.E / 4, Ez4 = p.z != nullptr ? p.Ez / 4 : 0;
    const int64_t threads = BH * (E4 + Ez4);
    const int64_t blocks = (threads + 255) / 256;
    if (p.log2_gamma != 0.0f && !p.is_int)
        hipLaunchKernelGGL(state_scan_decay_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<float4*>(p.S), reinterpret_cast<float4*>(p.S_final), E4,
                           reinterpret_cast<float4*>(p.z), reinterpret_cast<float4*>(p.z_final), Ez4, p.N, BH,
                           p.log2_gamma, p.L, p.Cs);
    else if (p.is_int)
        hipLaunchKernelGGL((state_scan_kernel<WrapInt4, unsigned, false>), dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<WrapInt4*>(p.S), reinterpret_cast<WrapInt4*>(p.S_final), E4,
                           reinterpret_cast<WrapInt4*>(p.z), reinterpret_cast<WrapInt4*>(p.z_final), Ez4, p.N, BH);
    else if (BH * p.N * (p.E + (Ez4 ? p.Ez : 0)) * 4 > (int64_t)512 << 20)  // larger than the last-level cache
        hipLaunchKernelGGL((state_scan_kernel<float4, float, true>), dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<float4*>(p.S), reinterpret_cast<float4*>(p.S_final), E4,
                           reinterpret_cast<float4*>(p.z), reinterpret_cast<float4*>(p.z_final), Ez4, p.N, BH);
    else
        hipLaunchKernelGGL((state_scan_kernel<float4, float, false>), dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<float4*>(p.S), reinterpret_cast<float4*>(p.S_final), E4,
                           reinterpret_cast<float4*>(p.z), reinterpret_cast<float4*>(p.z_final), Ez4, p.N, BH);
    return hipGetLastError();
}

}  // namespace la
