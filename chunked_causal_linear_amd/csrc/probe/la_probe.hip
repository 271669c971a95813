// Matrix-core rate and read bandwidth probes (see include/la_probe.h).
//
// Matrix cores: eight independent
// accumulators per wave, each updated once per round, so consecutive
// instructions never depend on each other and the matrix core never waits
// for a result.  The operands come from the thread index, so nothing folds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/la_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int NACC = 8;

__global__ __launch_bounds__(256) void probe_bf16(int64_t iters, float* out) {
    const int tid = threadIdx.x;
    const float x = 1.0f + 1e-3f * (float)(tid & 63);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(x * (float)(i + 1) * 1e-3f);
        b[i] = (__bf16)(x * (float)(8 - i) * 1e-3f);
    }
    f32x4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(int64_t)blockIdx.x * 256 + tid] = s;
}

__global__ __launch_bounds__(256) void probe_i8(int64_t iters, float* out) {
    const int tid = threadIdx.x;
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = 0x01010101 * ((tid + i) & 3);
        b[i] = 0x01010101 * ((tid + 2 * i) & 3);
    }
    i32x4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = i32x4{0, 0, 0, 0};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(int64_t)blockIdx.x * 256 + tid] = (float)s;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// grid-stride 16-byte reads of x, reps passes, folded per thread
__global__ __launch_bounds__(256) void probe_read(const u32x4* __restrict__ x, int64_t n16, int64_t reps, float* out) {
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x, stride = (int64_t)gridDim.x * 256;
    unsigned acc = 0;
    for (int64_t r = 0; r < reps; ++r)
        for (int64_t i = i0; i < n16; i += stride) {
            const u32x4 v = x[i];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    out[i0] = (float)acc;
}

}  // namespace

extern "C" int la_probe_mfma(int kind, int64_t iters, int64_t grid, float* out, struct ihipStream_t* stream) {
    if (iters < 1 || grid < 1 || grid > 0x7FFFFFFFLL || out == nullptr || (kind != 0 && kind != 1)) return -1;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        hipLaunchKernelGGL(probe_bf16, dim3((unsigned)grid), dim3(256), 0, s, iters, out);
    else
        hipLaunchKernelGGL(probe_i8, dim3((unsigned)grid), dim3(256), 0, s, iters, out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

extern "C" int la_probe_read(const void* x, int64_t n16, int64_t reps, int64_t grid, float* out,
                             struct ihipStream_t* stream) {
    if (x == nullptr || out == nullptr || n16 < 1 || reps < 1 || grid < 1 || grid > 0x7FFFFFFFLL / 256 ||
        (reinterpret_cast<uintptr_t>(x) & 15) != 0)
        return -1;
    hipLaunchKernelGGL(probe_read, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(x), n16, reps, out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}
