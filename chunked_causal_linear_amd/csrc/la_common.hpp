// Device helpers shared by the liblinattn kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  The fp32 -> bf16 direction uses the hardware conversion
// (round to nearest even) through the compiler's vector convert.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ u16 f2bf(float x) { return (u16)(pack2_bf16(x, 0.f) & 0xFFFFu); }

// 16-byte global loads and stores with the non-temporal hint, for data a
// kernel streams through once.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const void* p) {
    const u32x4_nt r = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void store_nt(void* p, const uint4& v) {
    __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_nt*>(p));
}

// ---------------------------------------------------------------------------
// Matrix-core wrappers.  16x16x32 bf16 -> fp32: lane l holds A[m = l%16][k = 8*(l/16) .. +7],
// B[k = 8*(l/16) .. +7][n = l%16] and C/D[m = 4*(l/16) + i][n = l%16], i = 0..3.
// 16x16x64 int8 -> int32: the same with 16 k-values per lane, k = 16*(l/16) .. +15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 mfma_i8(const i32x4& a, const i32x4& b, const i32x4& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 bf16x8_from2(const uint2& lo, const uint2& hi) {
    uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    return __builtin_bit_cast(bf16x8, u);
}

// fp32 accumulator pair -> 8 bf16 operand (first four from a, last four from b)
__device__ __forceinline__ bf16x8 pack_acc_bf16(const f32x4& a, const f32x4& b) {
    uint4 u = make_uint4(pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]), pack2_bf16(b[0], b[1]),
                         pack2_bf16(b[2], b[3]));
    return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------------------
// 4 x 8 transpose of 16-bit elements held as four rows of 8 (uint4 each).
// Output column c (0..7) as 4 elements (rows 0..3) packed in a uint2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t perm_lo(uint32_t hi_src, uint32_t lo_src) {
    // (lo_src.low16) | (hi_src.low16 << 16)
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t hi_src, uint32_t lo_src) {
    // (lo_src.high16) | (hi_src.high16 << 16)
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}

__device__ __forceinline__ uint32_t word(const uint4& u, int j) {
    return j == 0 ? u.x : (j == 1 ? u.y : (j == 2 ? u.z : u.w));
}

__device__ __forceinline__ void transpose4x8(const uint4 r[4], uint2 out[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t a = word(r[0], j), b = word(r[1], j), c = word(r[2], j), d = word(r[3], j);
        out[2 * j] = make_uint2(perm_lo(b, a), perm_lo(d, c));
        out[2 * j + 1] = make_uint2(perm_hi(b, a), perm_hi(d, c));
    }
}

// elu(x) + 1 with alpha = 1
__device__ __forceinline__ float elu1(float x) { return x >= 0.f ? x + 1.f : __expf(x); }

// elu+1 of in_scale * x for the eight bf16 values of u, in fp32: for
// s = |in_scale| and t = x s log2(e), elu+1(s x) is s x + 1 when t > 0 and
// exp2(t) = exp(s x) otherwise (1 at 0); a negative in_scale flips the sign
// of x first.  One multiply feeds both the test and the exponential.
struct Elu1Scale {
    float s, sl;
    uint32_t flip;  // sign bits of both halves of a bf16 pair, or 0
};
__device__ __forceinline__ Elu1Scale elu1_scale(float in_scale) {
    const float s = fabsf(in_scale);
    return Elu1Scale{s, s * 1.4426950408889634f, in_scale < 0.f ? 0x80008000u : 0u};
}
__device__ __forceinline__ void elu1_f32x8(const uint4& u, const Elu1Scale& e, float (&f)[8]) {
    const uint32_t w[4] = {u.x ^ e.flip, u.y ^ e.flip, u.z ^ e.flip, u.w ^ e.flip};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float a = __uint_as_float(w[j] << 16), b = __uint_as_float(w[j] & 0xFFFF0000u);
        const float ta = a * e.sl, tb = b * e.sl;
        f[2 * j] = ta > 0.f ? fmaf(a, e.s, 1.f) : __builtin_amdgcn_exp2f(ta);
        f[2 * j + 1] = tb > 0.f ? fmaf(b, e.s, 1.f) : __builtin_amdgcn_exp2f(tb);
    }
}

// Apply phi (elu+1 of in_scale * x) to 8 bf16 values in place.
__device__ __forceinline__ uint4 elu1_bf16x8(const uint4& u, float in_scale) {
    float f[8];
    elu1_f32x8(u, elu1_scale(in_scale), f);
    return make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]),
                      pack2_bf16(f[6], f[7]));
}

// elu+1 of in_scale * x for 8 bf16 values, as a bf16 pair (hi, lo) with
// hi = bf16(phi) and lo = bf16(phi - hi): hi + lo carries phi to about 2^-17
// relative, which keeps long state sums free of the bf16 rounding of phi.
__device__ __forceinline__ void elu1_split_bf16x8(const uint4& u, float in_scale, uint4& hi, uint4& lo,
                                                  float mul = 1.0f) {
    float f[8];
    elu1_f32x8(u, elu1_scale(in_scale), f);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] *= mul;
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = pack2_bf16(f[2 * j], f[2 * j + 1]);
        l[j] = pack2_bf16(f[2 * j] - __uint_as_float(h[j] << 16), f[2 * j + 1] - __uint_as_float(h[j] & 0xFFFF0000u));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

}  // namespace la
