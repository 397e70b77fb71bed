// MXFP8 activations for A8W4: bf16 rows -> E4M3 codes with one E8M0 scale
// per block of 32 along the row.
//
// news.ainew.jp, "vLLM publishes Kimi K3 production support", MXFP4 MoE: the
// AMD operators include A8W4, 8-bit activations on the 4-bit weights.  The
// activations take the OCP microscaling form of the weights: per block, the
// scale is 2^(floor(log2 amax) - 8) (8: the exponent of E4M3's largest
// normal, 448 = 1.75 * 2^8), kept in E8M0's range, and each element is the
// E4M3 value nearest to x / scale (ties to the even mantissa, saturating at
// +-448).  An all-zero block takes scale byte 0 and +0 codes.
//
// One thread per block of 32: four 16-byte loads of the bf16 values, the
// block maximum, then two 16-byte stores of codes and one scale byte.  Bound:
// HBM (2 bytes read, 1 + 1/32 written per element).

#include "device_common.h"
#include "internal.h"

namespace w4a16 {

namespace {

using namespace dev;

// E4M3 code of v (finite), nearest value with ties to the even mantissa,
// magnitudes above 448 saturating to 448.  Below 2^-6 the grid is the
// subnormal step 2^-9, so the magnitude code is round(|v| * 2^9) (8 being the
// smallest normal, whose code is also 8).  From 2^-6 up, rounding the fp32
// significand to 3 bits is an integer add on the bits (the carry moves into
// the exponent), and the E4M3 code is the fp32 exponent and top mantissa bits
// rebased from bias 127 to bias 7: (bits >> 20) - (120 << 3).
__device__ inline uint32_t e4m3_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = __builtin_fminf(__builtin_fabsf(v), 448.0f);
    uint32_t x = __float_as_uint(a);
    uint32_t mag;
    if (x < 0x3C800000u) {   // 2^-6
        mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
    } else {
        x += 0x7FFFFu + ((x >> 20) & 1u);
        mag = (x >> 20) - (120u << 3);
    }
    return sign | mag;
}

// floor(log2 a) of a positive finite fp32 value (exponent field, or for a
// subnormal the position of the top mantissa bit).
__device__ inline int floor_log2(float a) {
    const uint32_t x = __float_as_uint(a);
    const int e = static_cast<int>((x >> 23) & 0xFFu);
    return e != 0 ? e - 127 : -118 - static_cast<int>(__builtin_clz(x & 0x7FFFFFu));
}

__global__ void __launch_bounds__(256) k_quant_mxfp8(const uint16_t* __restrict__ x, int64_t rows,
                                                     const int32_t* rows_dev, int K,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
    int64_t n = rows;
    if (rows_dev) {
        const int64_t d = rows_dev[0];
        n = d < n ? (d > 0 ? d : 0) : n;
    }
    const int bpr = K / 32;
    const int64_t blocks = n * bpr;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < blocks;
         b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 32);
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 w = src[q];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * q + 2 * h] = __uint_as_float(ww[h] << 16);
                v[8 * q + 2 * h + 1] = __uint_as_float(ww[h] & 0xFFFF0000u);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        uint32_t sb = 0;
        u32x4 c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
        if (amax > 0.0f) {
            int bb = floor_log2(amax) + 119;   // floor(log2 amax) - 8 + 127
            bb = bb < 0 ? 0 : (bb > 254 ? 254 : bb);
            sb = static_cast<uint32_t>(bb);
            const int sh = 127 - bb;
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                w[q] = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[q] |= e4m3_code(__builtin_ldexpf(v[4 * q + i], sh)) << (8 * i);
            }
            c0 = u32x4{w[0], w[1], w[2], w[3]};
            c1 = u32x4{w[4], w[5], w[6], w[7]};
        }
        u32x4* dst = reinterpret_cast<u32x4*>(codes + b * 32);
        dst[0] = c0;
        dst[1] = c1;
        scales[b] = static_cast<uint8_t>(sb);
    }
}

}  // namespace

void launch_quant_mxfp8(const uint16_t* x, int64_t rows, const int32_t* rows_dev, int K,
                        uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const int64_t blocks = rows * (K / 32);
    int64_t g = (blocks + 255) / 256;
    g = g < 1 ? 1 : (g > 8192 ? 8192 : g);
    k_quant_mxfp8<<<dim3(static_cast<unsigned>(g)), dim3(256), 0, s>>>(x, rows, rows_dev, K, codes,
                                                                      scales);
}

}  // namespace w4a16
