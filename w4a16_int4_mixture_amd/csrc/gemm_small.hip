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
// (x & mask) | bits: with mask and bits arriving as kernel arguments rather
// than literals, the compiler emits a single v_and_or_b32 per pair.
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
    return (x & mask) | bits;
}

__device__ inline bf16x8 codes_to_b(uint32_t w, uint32_t mask, uint32_t bits) {
    u32x4 d;
    d.x = and_or(w, mask, bits);
    d.y = and_or(w >> 4, mask, bits);
    d.z = and_or(w >> 8, mask, bits);
    d.w = and_or(w >> 12, mask, bits);
    return __builtin_bit_cast(bf16x8, d);
}

// Codes and scales of one K group for one wavefront (WPL words + WPL scales
// per lane).
template <int WPL>
struct WFrag {
    u32x4 w[WPL / 4];
    uint32_t s[WPL / 2];
};

template <int WPL>
__device__ inline void load_w(WFrag<WPL>& f, const uint32_t* cp, const uint16_t* sp, int ks) {
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
}

// One K group: MT row blocks x WPL column blocks; A fragments come from LDS.
template <int MT, int WPL>
__device__ inline void compute_group(const WFrag<WPL>& f, const u32x4* a_lds,
                                     f32x4 (&acc)[MT][WPL], uint32_t mask, uint32_t bits) {
    const bf16x8 c136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u,
                                                         0xC308C308u, 0xC308C308u});  // -136
    u32x4 av[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) av[t] = a_lds[t * 64];
    bf16x8 b[WPL];
    float sc[WPL];
#pragma unroll
    for (int i = 0; i < WPL / 4; ++i) {
        b[4 * i + 0] = codes_to_b(f.w[i].x, mask, bits);
        b[4 * i + 1] = codes_to_b(f.w[i].y, mask, bits);
        b[4 * i + 2] = codes_to_b(f.w[i].z, mask, bits);
        b[4 * i + 3] = codes_to_b(f.w[i].w, mask, bits);
    }
#pragma unroll
    for (int i = 0; i < WPL / 2; ++i) {
        sc[2 * i] = __uint_as_float(f.s[i] << 16);
        sc[2 * i + 1] = __uint_as_float(f.s[i] & 0xFFFF0000u);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, av[t]);
        const f32x4 off = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, c136, zero, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < WPL; ++j) {
            const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], off, 0, 0, 0);
            acc[t][j] += sc[j] * d;
        }
    }
}

// Activation staging: a stage covers SG groups of K; its fragments (SG x MT,
// 1 KB each: 64 lanes x 16 bytes in MFMA A-operand order) are loaded by the
// four wavefronts of the workgroup (wavefront w takes the groups g = w mod 4)
// and read by all of them from LDS.
constexpr int kSG = 8;

template <int MT>
struct AStage {
    u32x4 v[kSG / 4][MT];
};

template <int MT>
__device__ inline void load_a_stage(AStage<MT>& st, const uint16_t* const* ap, int ks_stage,
                                    int ks_min, int wave) {
#pragma unroll
    for (int i = 0; i < kSG / 4; ++i) {
        int g = ks_stage + 4 * i + wave;
        g = g < ks_min ? ks_min : g;
#pragma unroll
        for (int t = 0; t < MT; ++t) st.v[i][t] = *reinterpret_cast<const u32x4*>(ap[t] + g * 32);
    }
}

template <int MT>
__device__ inline void store_a_stage(const AStage<MT>& st, u32x4* buf, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kSG / 4; ++i)
#pragma unroll
        for (int t = 0; t < MT; ++t) buf[((4 * i + wave) * MT + t) * 64 + lane] = st.v[i][t];
}

}  // namespace

// The K loop of one workgroup tile with MT active 16-row blocks.  Weights and
// scales run through a register ring kSG groups deep (one 16-byte code load
// per WPL/4 words per group, issued kSG groups ahead); activations are staged
// through LDS one stage ahead, double-buffered, one barrier per stage.  The
// first (K range mod kSG) groups are done before the ring starts.
template <int MT, int WPL>
__device__ void stream_loop(const uint32_t* cp, const uint16_t* sp, const uint16_t* const* ap,
                            int ks0, int ks1, int wave, int lane, u32x4* lds,
                            f32x4 (&acc)[MT][WPL], uint32_t mask, uint32_t bits) {
    constexpr int D = kSG;
    if (ks1 <= ks0) return;
    u32x4* buf0 = lds;
    u32x4* buf1 = lds + kSG * MT * 64;
    // Stages are aligned to the end of the K range: the first stage starts
    // `pad` groups early; those slots re-read group ks0 and have their scales
    // zeroed, so they add exactly zero.  Every stage then runs the same code.
    const int pad = (kSG - (ks1 - ks0) % kSG) % kSG;
    const int kb = ks0 - pad;
    const int nst = (ks1 - kb) / kSG;

    // first activation stage is issued before the weight ring so that storing
    // it to LDS does not wait for the ring's loads
    WFrag<WPL> ring[D];
    {
        AStage<MT> a0;
        load_a_stage<MT>(a0, ap, kb, ks0, wave);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < D; ++i) {
            load_w<WPL>(ring[i], cp, sp, kb + i < ks0 ? ks0 : kb + i);
            if (kb + i < ks0) {
#pragma unroll
                for (int j = 0; j < WPL / 2; ++j) ring[i].s[j] = 0u;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        store_a_stage<MT>(a0, buf0, wave, lane);
    }
    __syncthreads();
    for (int st = 0; st < nst - 1; ++st) {
        u32x4* cur = (st & 1) ? buf1 : buf0;
        u32x4* nxt = (st & 1) ? buf0 : buf1;
        const int base = kb + st * kSG;
        AStage<MT> an;
        load_a_stage<MT>(an, ap, base + kSG, ks0, wave);
        __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads ahead of the ring refills
#pragma unroll
        for (int g = 0; g < kSG; ++g) {
            compute_group<MT, WPL>(ring[g], cur + g * MT * 64 + lane, acc, mask, bits);
            load_w<WPL>(ring[g], cp, sp, base + kSG + g);
            __builtin_amdgcn_sched_barrier(0);
        }
        store_a_stage<MT>(an, nxt, wave, lane);
        __syncthreads();
    }
    {
        u32x4* cur = ((nst - 1) & 1) ? buf1 : buf0;
#pragma unroll
        for (int g = 0; g < kSG; ++g) compute_group<MT, WPL>(ring[g], cur + g * MT * 64 + lane, acc, mask, bits);
    }
}

// One (row tile, 4 column chunks, K split) with MT active row blocks.
template <int MT, int WPL>
__device__ void gemm_tile_mt(const GemmArgs& a, int e, int p0, int nrows, int chunk, int wave,
                             int lane, u32x4* lds) {
    const bool slot_rows = a.tile_src != TILE_MASKED;
    const bool active = chunk < a.NC;

    // activation row of each of this lane's MFMA A rows (rows past the tile
    // reuse its first row: MFMA rows are independent and are not stored)
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

    const int s = blockIdx.z;
    const int ks0 = static_cast<int>(static_cast<int64_t>(s) * a.KS / a.split_k);
    const int ks1 = static_cast<int>(static_cast<int64_t>(s + 1) * a.KS / a.split_k);
    // a wavefront past the last chunk re-streams the last chunk (cache hits,
    // only when N / CW is not a multiple of 4) and stores nothing: the loop
    // stays free of wavefront-dependent branches
    const int64_t cbase = static_cast<int64_t>(e) * a.NC + (active ? chunk : a.NC - 1);
    const uint32_t* cp = a.codes + (cbase * a.KS) * 64 * WPL + lane * WPL;
    const uint16_t* sp = a.scales + (cbase * a.KS) * 16 * WPL + (lane & 15) * WPL;

    f32x4 acc[MT][WPL];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < WPL; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the exponent pattern lives in a VGPR so that (x & mask) | bits is one
    // v_and_or_b32 (a VALU op reads at most one scalar operand); the empty asm
    // only pins the register class and emits nothing
    uint32_t vbits = a.unpack_bits;
    asm volatile("" : "+v"(vbits));
    stream_loop<MT, WPL>(cp, sp, ap, ks0, ks1, wave, lane, lds, acc, a.unpack_mask, vbits);
    if (!active) return;

    // epilogue: lane holds rows 16t + 4*(lane/16) + i of column 16j + lane%16
    const int col0 = chunk * a.CW + (lane & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
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

template <int MT, int WPL>
__device__ void gemm_tile(const GemmArgs& a, int e, int p0, int nrows, int chunk, int wave,
                          int lane, u32x4* lds) {
    const int mt_active = (nrows + 15) >> 4;
    if (mt_active <= 1) gemm_tile_mt<1, WPL>(a, e, p0, nrows, chunk, wave, lane, lds);
    else if (MT >= 2 && mt_active == 2) gemm_tile_mt<(MT >= 2 ? 2 : 1), WPL>(a, e, p0, nrows, chunk, wave, lane, lds);
    else if (MT >= 3 && mt_active == 3) gemm_tile_mt<(MT >= 3 ? 3 : 1), WPL>(a, e, p0, nrows, chunk, wave, lane, lds);
    else if (MT >= 4) gemm_tile_mt<(MT >= 4 ? 4 : 1), WPL>(a, e, p0, nrows, chunk, wave, lane, lds);
}

// Tiles are walked grid-stride along grid.y, so any device-side tile count is
// fully covered whatever the grid size; every wavefront leaves the loop once
// its tile index passes the count.
template <int MT, int WPL>
__global__ void __launch_bounds__(256) k_gemm_small(GemmArgs a) {
    __shared__ u32x4 lds[2 * kSG * MT * 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int chunk = blockIdx.x * 4 + wave;
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
        gemm_tile<MT, WPL>(a, e, p0, nrows, chunk, wave, lane, lds);
        __syncthreads();  // the next tile reuses the staging buffers
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
