// Grouped W4A16 GEMM for few routed rows per expert (decode-sized tiles of at
// most 16*MT rows): a weight-streaming kernel for CDNA4.
//
//   out[p, n] = sum_c A[row(p), c] * (q[e,n,c] - 8) * s[e,n,c/32]
//
// Chord page, "H200 and Blackwell indexed decode": with a few routed rows per
// expert the path is bound by weight traffic; the dequantised weights take the
// wide side of the matrix instruction and the tokens the narrow side; the
// INT4 subtract-then-scale is fused into nibble extraction.  "H200 prefill and
// TP8": deep-K gate/up keeps a split of K (stream-K) where the M x N grid
// alone cannot fill the machine.
//
// CDNA4 design (one wavefront = one packed chunk of CW output columns over a
// K range; four wavefronts per workgroup on neighbouring chunks of one tile):
//   * every lane fetches its codes for one K group of 32 with 16-byte loads
//     (CW/16 words) and its CW/16 group scales: the packed layout makes each
//     wavefront's stream contiguous, and a ring of D groups is kept in flight;
//   * the activation fragments (8 bf16 per lane per 16-row M tile) come
//     straight from L2 (the activations are small and shared by every chunk);
//   * a code q becomes the bf16 value 128 + q by OR-ing the exponent pattern
//     0x43 above it, two codes per VALU op; v_mfma_f32_16x16x32_bf16 (K = 32 =
//     one scale group) then yields P = sum x (128 + q); the offset
//     -136 * sum x is produced once per M tile by one MFMA against a constant
//     operand and fed as the accumulator input, so the MFMA returns
//     sum x (q - 8) exactly as the group's partial; the fp32 group scale is
//     applied with one FMA per accumulator element.  Weights are never
//     rounded: the products and the within-group sums are exact.

#include "internal.h"

namespace w4a16 {

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// B operand for one 16-column block: the word's eight codes as bf16 128 + q,
// in MFMA K order (nibble order 0,2,4,6,1,3,5,7 puts offsets 2p and 2p+1 in
// the two halves of (w >> 4p) & 0x000F000F).
__device__ inline bf16x8 codes_to_b(uint32_t w) {
    u32x4 d;
    d.x = (w & 0x000F000Fu) | 0x43004300u;
    d.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    d.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    d.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, d);
}

template <int MT, int WPL>
struct Frag {
    u32x4 w[WPL / 4];      // codes: WPL words
    uint32_t s[WPL / 2];   // scales: WPL bf16
    u32x4 a[MT];           // activation fragments
};

template <int MT, int WPL>
__device__ inline void load_frag(Frag<MT, WPL>& f, const uint32_t* cp, const uint16_t* sp,
                                 const uint16_t* const* ap, int ks, int mt_active) {
    const u32x4* c4 = reinterpret_cast<const u32x4*>(cp + static_cast<int64_t>(ks) * 64 * WPL);
#pragma unroll
    for (int i = 0; i < WPL / 4; ++i) f.w[i] = __builtin_nontemporal_load(c4 + i);
    const uint16_t* s = sp + static_cast<int64_t>(ks) * 16 * WPL;
    if constexpr (WPL == 4) {
        u32x2 v = *reinterpret_cast<const u32x2*>(s);
        f.s[0] = v.x;
        f.s[1] = v.y;
    } else {
        u32x4 v = *reinterpret_cast<const u32x4*>(s);
        f.s[0] = v.x;
        f.s[1] = v.y;
        f.s[2] = v.z;
        f.s[3] = v.w;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
        if (t < mt_active) f.a[t] = *reinterpret_cast<const u32x4*>(ap[t] + ks * 32);
}

template <int MT, int WPL>
__device__ inline void compute_frag(const Frag<MT, WPL>& f, f32x4 (&acc)[MT][WPL],
                                    int mt_active) {
    const bf16x8 c136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u,
                                                         0xC308C308u, 0xC308C308u});  // -136
    bf16x8 b[WPL];
    float sc[WPL];
#pragma unroll
    for (int i = 0; i < WPL / 4; ++i) {
        b[4 * i + 0] = codes_to_b(f.w[i].x);
        b[4 * i + 1] = codes_to_b(f.w[i].y);
        b[4 * i + 2] = codes_to_b(f.w[i].z);
        b[4 * i + 3] = codes_to_b(f.w[i].w);
    }
#pragma unroll
    for (int i = 0; i < WPL / 2; ++i) {
        sc[2 * i] = __uint_as_float(f.s[i] << 16);
        sc[2 * i + 1] = __uint_as_float(f.s[i] & 0xFFFF0000u);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t < mt_active) {
            bf16x8 a = __builtin_bit_cast(bf16x8, f.a[t]);
            f32x4 off = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, c136, zero, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < WPL; ++j) {
                f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], off, 0, 0, 0);
                acc[t][j] += sc[j] * d;
            }
        }
    }
}

}  // namespace

// One (row tile, column chunk, K split) of the GEMM for this wavefront.
template <int MT, int WPL>
__device__ void gemm_tile(const GemmArgs& a, int e, int p0, int nrows, int chunk, int lane) {
    constexpr int D = 4;  // groups of K kept in flight per wavefront
    const int mt_active = (nrows + 15) >> 4;
    const bool slot_rows = a.tile_src != TILE_MASKED;

    // ---- activation row of each of this lane's MFMA A rows
    const uint16_t* ap[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int r = 16 * t + (lane & 15);
        int rr = r < nrows ? r : 0;
        int64_t row = p0 + rr;
        if (slot_rows && a.arow != W4A16_AROW_POSITION) {
            int f = a.sorted_ids[p0 + rr];
            if (f < 0 || f >= a.num_slots) f = a.sorted_ids[p0];
            if (f < 0 || f >= a.num_slots) f = 0;
            row = (a.arow == W4A16_AROW_TOKEN) ? f / a.top_k : f;
        }
        row = row < a.A_rows ? row : a.A_rows - 1;
        ap[t] = a.A + row * a.K + 8 * (lane >> 4);
    }

    // ---- K range of this split
    const int s = blockIdx.z;
    const int ks0 = static_cast<int>(static_cast<int64_t>(s) * a.KS / a.split_k);
    const int ks1 = static_cast<int>(static_cast<int64_t>(s + 1) * a.KS / a.split_k);
    const int64_t cbase = static_cast<int64_t>(e) * a.NC + chunk;
    const uint32_t* cp = a.codes + (cbase * a.KS) * 64 * WPL + lane * WPL;
    const uint16_t* sp = a.scales + (cbase * a.KS) * 16 * WPL + (lane & 15) * WPL;

    f32x4 acc[MT][WPL];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < WPL; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Frag<MT, WPL> fr[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (ks0 + i < ks1) load_frag<MT, WPL>(fr[i], cp, sp, ap, ks0 + i, mt_active);
    for (int ks = ks0; ks < ks1; ks += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (ks + i < ks1) {
                compute_frag<MT, WPL>(fr[i], acc, mt_active);
                if (ks + i + D < ks1) load_frag<MT, WPL>(fr[i], cp, sp, ap, ks + i + D, mt_active);
            }
        }
    }

    // ---- epilogue: lane holds rows 16t + 4*(lane/16) + i of column 16j + lane%16
    const int col0 = chunk * a.CW + (lane & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= mt_active) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * t + 4 * (lane >> 4) + i;
            if (r >= nrows) continue;
            int64_t orow = p0 + r;
            if (slot_rows && (a.tile_src == TILE_BLOCKS || a.orow == W4A16_OROW_SLOT)) {
                int f = a.sorted_ids[p0 + r];
                if (f < 0 || f >= a.num_slots) continue;
                if (a.orow == W4A16_OROW_SLOT && a.out_kind != OUT_PARTIAL) orow = f;
            }
            if (a.out_kind == OUT_BF16) {
                uint16_t* o = static_cast<uint16_t*>(a.out) + orow * a.N + col0;
#pragma unroll
                for (int j = 0; j < WPL; ++j) o[16 * j] = f32_to_bf16_rne(acc[t][j][i]);
            } else {
                float* o = static_cast<float*>(a.out) +
                           (a.out_kind == OUT_PARTIAL ? s * a.ws_stride : 0) + orow * a.N + col0;
#pragma unroll
                for (int j = 0; j < WPL; ++j) o[16 * j] = acc[t][j][i];
            }
        }
    }
}

// Tiles are walked grid-stride along grid.y, so any device-side tile count is
// fully covered whatever the grid size; every wavefront leaves the loop once
// its tile index passes the count.
template <int MT, int WPL>
__global__ void __launch_bounds__(256) k_gemm_small(GemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int chunk = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (chunk >= a.NC) return;
    for (int ty = blockIdx.y;; ty += gridDim.y) {
        int e, p0, nrows;
        if (a.tile_src == TILE_TABLE) {
            if (ty >= a.tile_count[0]) return;
            const int4 t = reinterpret_cast<const int4*>(a.tiles)[ty];
            e = t.x;
            p0 = t.y;
            nrows = t.z;
        } else if (a.tile_src == TILE_BLOCKS) {
            p0 = ty * a.block_m;
            if (p0 >= a.ntp[0]) return;
            e = a.expert_ids[ty];
            nrows = a.sorted_cap - p0 < a.block_m ? a.sorted_cap - p0 : a.block_m;
        } else {
            if (ty >= a.grid_tiles_total) return;
            const int g = ty / a.chunks_per_expert;
            const int r0 = (ty % a.chunks_per_expert) * a.tile_m;
            const int cnt = a.masked_m[g];
            if (r0 >= cnt) continue;
            e = g;
            p0 = g * a.max_m + r0;
            nrows = cnt - r0 < a.tile_m ? cnt - r0 : a.tile_m;
        }
        if (e < 0 || e >= a.E || nrows <= 0) continue;
        gemm_tile<MT, WPL>(a, e, p0, nrows, chunk, lane);
    }
}

void launch_gemm_small(const GemmArgs& a, int mt, hipStream_t st) {
    const dim3 grid((a.NC + 3) / 4, a.grid_tiles, a.split_k), block(256);
    if (a.CW == 64) {
        switch (mt) {
            case 1: k_gemm_small<1, 4><<<grid, block, 0, st>>>(a); break;
            case 2: k_gemm_small<2, 4><<<grid, block, 0, st>>>(a); break;
            case 3: k_gemm_small<3, 4><<<grid, block, 0, st>>>(a); break;
            default: k_gemm_small<4, 4><<<grid, block, 0, st>>>(a); break;
        }
    } else {
        switch (mt) {
            case 1: k_gemm_small<1, 8><<<grid, block, 0, st>>>(a); break;
            case 2: k_gemm_small<2, 8><<<grid, block, 0, st>>>(a); break;
            case 3: k_gemm_small<3, 8><<<grid, block, 0, st>>>(a); break;
            default: k_gemm_small<4, 8><<<grid, block, 0, st>>>(a); break;
        }
    }
}

}  // namespace w4a16
