// Device helpers shared by the GEMM kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a16 {
namespace dev {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint16_t f32_to_bf16_rne(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float bf16_round(float x) {
    return __uint_as_float(static_cast<uint32_t>(f32_to_bf16_rne(x)) << 16);
}

// silu(g) * u with g and u first rounded to bf16 (the rounding of a gate/up
// output that is stored and then activated).  silu(g) = g / (1 + e^-g) is
// evaluated as g / (1 + t) for g >= 0 and g t / (1 + t) for g < 0, with t =
// e^-|g|, so nothing overflows (e^-g would below g = -88.7, where g e^g is
// still a normal bf16).  The hardware exp2 flushes subnormal results, so t is
// formed as 2^64 t (normal down to g = -131) and the 2^-64 is applied after
// the division, by an exact power-of-two multiply.  The divisor lies in
// [1, 2]: the quotient is the hardware reciprocal's product refined by one
// Newton step (within an ulp of fp32, far below the bf16 rounding after),
// with the dividend's sign.
__device__ inline float silu_mul_bf16(float g, float u) {
    g = bf16_round(g);
    u = bf16_round(u);
    const float ts = __builtin_amdgcn_exp2f(64.0f - __builtin_fabsf(g) * 1.44269504088896341f);
    const float den = 1.0f + ts * 0x1p-64f;
    const float num = g >= 0.0f ? g : g * ts;
    const float r = __builtin_amdgcn_rcpf(den);
    float q = num * r;
    q = __builtin_fmaf(__builtin_fmaf(-den, q, num), r, q);
    q = __builtin_copysignf(q, num);   // the refinement would turn -0 into +0
    return (g >= 0.0f ? q : q * 0x1p-64f) * u;
}

// Buffer loads address the packed weights and the activations with a scalar
// resource and a 32-bit per-lane offset; a K position goes into the scalar
// offset, so loops do no per-lane address arithmetic.  Reads past a
// resource's size return zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint64_t bytes) {
    const uint32_t n = bytes < 0xFFFFFFFFull ? static_cast<uint32_t>(bytes) : 0xFFFFFFFFu;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(n),
                                             0x00020000);
}

constexpr int kNonTemporal = 2;   // cache-policy bits of a streaming load
constexpr int kDeviceScope = 16;  // cache-policy bits of a device-coherent access

}  // namespace dev
}  // namespace w4a16
