// Grouped W4A16 GEMM for many routed rows per expert (tiles of up to 256
// rows): an MFMA-bound kernel for CDNA4.
//
//   out[p, n] = sum_c A[row(p), c] * bf16((q[e,n,c] - 8) * s[e,n,c/32])
//
// Chord page, "H200 prefill and TP8": with many routed rows per expert the
// path is bound by the matrix units and the dequant; the dequant (subtract,
// then scale) is amortised over the rows of a tile, and block M follows the
// routed rows per expert.
//
// CDNA4 design.  A workgroup is four wavefronts on a tile of up to 256 rows
// (MB row blocks of 16) and 256 columns (two 128-column chunks of the prefill
// profile).  Wavefront w works on chunk 2 * blockIdx.x + w / 2 and, inside
// it, on the 16-column blocks {2h, 2h+1, 2h+4, 2h+5} (h = w % 2), for every
// row of the tile; with the gate/up interleave those are two gate blocks and
// their two up blocks, so SiLU * gate can run on the accumulators.
//   * Weights: per K group each lane loads its four words (8 codes each) and
//     four scales and dequantises them once for the whole tile: a code q
//     becomes bf16 128 + q (one v_and_or_b32 per pair), then fp32, then
//     (128 + q) * s - 136 * s in one exact FMA, then bf16 (one rounding of
//     (q - 8) * s).  The B operands stay in registers; a ring keeps the
//     weights of the next four groups in flight.
//   * Activations: stages of two K groups (up to 256 rows x 64 K = 32 KB)
//     go through LDS, double-buffered, one barrier per stage; each stage is
//     loaded into registers one stage ahead and read back in MFMA A-operand
//     order.
//   * v_mfma_f32_16x16x32_bf16, one per (row block, column block, group);
//     256 fp32 accumulators per lane live in the accumulation registers.

#include "device_common.h"
#include "internal.h"

namespace w4a16 {

namespace {

using namespace dev;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWPL = 8;          // words per lane per group in a 128-column chunk
constexpr int kRecWords = 576 * kWPL;
constexpr int kBlocks = 4;       // 16-column blocks per wavefront
constexpr int kRing = 4;         // groups of weights in flight

// The weights of one K group for one lane: words and scales of its four
// column blocks (block order 2h, 2h+1, 2h+4, 2h+5).
struct WGroup {
    u32x2 w_lo, w_hi;   // words of blocks 2h, 2h+1 and 2h+4, 2h+5
    uint32_t s_lo, s_hi;  // bf16 scale pairs of the same blocks
};

__device__ inline uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// B operand of one column block: the word's eight codes dequantised with the
// scale s (c = -136 s), in MFMA K order (the packed nibble order puts K
// offsets 2p and 2p+1 in the two 16-bit halves of (w >> 4p) & 0x000F000F).
__device__ inline bf16x8 dequant_block(uint32_t w, float s, float c, uint32_t mask,
                                       uint32_t bits) {
    u32x4 d;
    uint32_t x[4] = {w, w >> 4, w >> 8, w >> 12};
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t v = (x[p] & mask) | bits;            // bf16 (128 + q) pair
        const float lo = __uint_as_float(v << 16);
        const float hi = __uint_as_float(v & 0xFFFF0000u);
        o[p] = pk_bf16(__builtin_fmaf(lo, s, c), __builtin_fmaf(hi, s, c));
    }
    d.x = o[0];
    d.y = o[1];
    d.z = o[2];
    d.w = o[3];
    return __builtin_bit_cast(bf16x8, d);
}

__device__ inline void dequant_group(const WGroup& g, uint32_t mask, uint32_t bits,
                                     bf16x8 (&b)[kBlocks]) {
    const float s0 = __uint_as_float(g.s_lo << 16), s1 = __uint_as_float(g.s_lo & 0xFFFF0000u);
    const float s2 = __uint_as_float(g.s_hi << 16), s3 = __uint_as_float(g.s_hi & 0xFFFF0000u);
    b[0] = dequant_block(g.w_lo.x, s0, -136.0f * s0, mask, bits);
    b[1] = dequant_block(g.w_lo.y, s1, -136.0f * s1, mask, bits);
    b[2] = dequant_block(g.w_hi.x, s2, -136.0f * s2, mask, bits);
    b[3] = dequant_block(g.w_hi.y, s3, -136.0f * s3, mask, bits);
}

// Loads group ks of the chunk for this lane: words at (slot * 64 + lane) * 8
// + {2h, 2h+1} and + {2h+4, 2h+5}; scales (bf16) after the record's codes at
// (slot * 16 + lane % 16) * 8 + the same block indices.
__device__ inline void load_wgroup(WGroup& g, __amdgpu_buffer_rsrc_t w, uint32_t code_off,
                                   uint32_t scale_off, int ks) {
    const int soff = ((ks >> 3) * kRecWords + (ks & 7) * (64 * kWPL)) * 4;
    const int ssoff = ((ks >> 3) * kRecWords + 512 * kWPL) * 4 + (ks & 7) * (16 * kWPL * 2);
    g.w_lo = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(w, code_off, soff, kNonTemporal));
    g.w_hi = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(w, code_off + 16, soff, kNonTemporal));
    g.s_lo = __builtin_amdgcn_raw_buffer_load_b32(w, scale_off, ssoff, kNonTemporal);
    g.s_hi = __builtin_amdgcn_raw_buffer_load_b32(w, scale_off + 8, ssoff, kNonTemporal);
}

// Activation stage: rows [0, 16 * MB) x 64 K (groups 2s, 2s+1), 8 x 16 bytes
// per thread per 256 rows.  Thread i takes K chunk kc = i % 8 (group kc / 4,
// K offset 8 * (kc % 4)) of rows i / 8 + 32 * pass.
template <int MB>
struct AStage {
    u32x4 v[MB / 2];
};

// soff = 128 s bytes (uniform); delta (<= 0, per lane) moves a K chunk of a
// padding group back onto the last real group.
template <int MB>
__device__ inline void load_astage(AStage<MB>& st, __amdgpu_buffer_rsrc_t x,
                                   const uint32_t (&row_off)[MB / 2], int soff, int delta) {
#pragma unroll
    for (int i = 0; i < MB / 2; ++i)
        st.v[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(x, row_off[i] + delta, soff, 0));
}

// LDS layout of a stage: [group (2)][row block (16)][lane (64)] x 16 bytes,
// lane = 16 * (K offset / 8) + row % 16 (the MFMA A-operand order).
template <int MB>
__device__ inline void store_astage(const AStage<MB>& st, u32x4* buf, int tid) {
    const int kc = tid & 7;
    const int g = kc >> 2;
#pragma unroll
    for (int i = 0; i < MB / 2; ++i) {
        const int r = (tid >> 3) + 32 * i;
        buf[(g * 16 + (r >> 4)) * 64 + (kc & 3) * 16 + (r & 15)] = st.v[i];
    }
}

constexpr int kStageU4 = 2 * 16 * 64;  // u32x4 per LDS stage

}  // namespace

// One tile (expert e, positions [p0, p0 + nrows), nrows <= 16 * MB) for the
// two chunks of blockIdx.x.
template <int MB>
__device__ __forceinline__ void large_tile(const GemmArgs& a, int e, int p0, int nrows,
                                           int wave, int lane, u32x4* lds) {
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x * 2 + (wave >> 1);
    const int h = wave & 1;
    const bool active = chunk < a.NC;
    const bool slot_rows = a.tile_src != TILE_MASKED;

    // activation rows this thread stages: rows tid / 8 + 32 i (rows past the
    // tile reuse its first row: they are computed, never stored)
    uint32_t row_off[MB / 2];
#pragma unroll
    for (int i = 0; i < MB / 2; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int rr = r < nrows ? r : 0;
        int64_t row = p0 + rr;
        if (slot_rows && a.arow != W4A16_AROW_POSITION) {
            int f = a.sorted_ids[p0 + rr];
            if (f < 0 || f >= a.num_slots) f = a.sorted_ids[p0];
            if (f < 0 || f >= a.num_slots) f = 0;
            row = (a.arow == W4A16_AROW_TOKEN) ? f / a.top_k : f;
        }
        row = row < a.A_rows ? row : a.A_rows - 1;
        // A_rows * K * 2 < 2^32 is checked on the host
        row_off[i] = static_cast<uint32_t>(row * a.K * 2 + (tid & 7) * 16);
    }
    const __amdgpu_buffer_rsrc_t x = make_rsrc(a.A, static_cast<uint64_t>(a.A_rows) * a.K * 2);
    // K chunk kc of stage s lies in group 2s + kc / 4; in the stages that
    // reach past K (padding groups, zero weights) such a chunk re-reads the
    // last real group, so that nothing outside the row is read
    const int kgrp_half = (tid & 7) >> 2;
    auto a_delta = [&](int s) {
        const int g = 2 * s + kgrp_half;
        return g < a.KS ? 0 : (a.KS - 1 - g) * 64;
    };

    const int64_t cbase = static_cast<int64_t>(e) * a.NC + (active ? chunk : a.NC - 1);
    const __amdgpu_buffer_rsrc_t w =
        make_rsrc(a.packed + cbase * a.chunk_words, static_cast<uint64_t>(a.chunk_words) * 4);
    const uint32_t code_off = static_cast<uint32_t>((lane * kWPL + 2 * h) * 4);
    const uint32_t scale_off = static_cast<uint32_t>(((lane & 15) * kWPL + 2 * h) * 2);
    const uint32_t mask = a.unpack_mask;
    const uint32_t bits = a.unpack_bits;

    f32x4 acc[MB][kBlocks];
#pragma unroll
    for (int t = 0; t < MB; ++t)
#pragma unroll
        for (int j = 0; j < kBlocks; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ngroups = a.KSP;         // a multiple of 8
    const int nst = ngroups / 2;       // a multiple of 4

    WGroup ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) load_wgroup(ring[i], w, code_off, scale_off, i);
    AStage<MB> ast;
    load_astage<MB>(ast, x, row_off, 0, 2 * 0 + 1 < a.KS ? 0 : a_delta(0));
    store_astage<MB>(ast, lds, tid);
    __syncthreads();

    // Two stages per iteration, so that ring slots and LDS buffers are static
    // (nst is a multiple of 4).  The body has no branches: past the end, the
    // last stage and the last group are loaded again and never used, so the
    // compiler can count the loads in flight and wait only for the oldest.
    for (int s = 0; s < nst; s += 2) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int st = s + half;
            const u32x4* cur = lds + half * kStageU4;
            {
                const int sn = st + 1 < nst ? st + 1 : nst - 1;
                load_astage<MB>(ast, x, row_off, 128 * sn, 2 * sn + 1 < a.KS ? 0 : a_delta(sn));
            }
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const int slot = 2 * half + gg;
                const int g = 2 * st + gg;
                bf16x8 b[kBlocks];
                dequant_group(ring[slot], mask, bits, b);
                load_wgroup(ring[slot], w, code_off, scale_off,
                            g + kRing < ngroups ? g + kRing : ngroups - 1);
#pragma unroll
                for (int t = 0; t < MB; ++t) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, cur[(gg * 16 + t) * 64 + lane]);
#pragma unroll
                    for (int j = 0; j < kBlocks; ++j)
                        acc[t][j] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[j], acc[t][j], 0, 0, 0);
                    // keep at most four row blocks of A fragments in registers
                    if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);
                }
            }
            store_astage<MB>(ast, lds + (1 - half) * kStageU4, tid);
            __syncthreads();
        }
    }
    if (!active) return;

    // epilogue: lane holds rows 16t + 4*(lane/16) + i of column 16 J[j] +
    // lane%16, J = {2h, 2h+1, 2h+4, 2h+5}
#pragma unroll
    for (int t = 0; t < MB; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * t + 4 * (lane >> 4) + i;
            if (r >= nrows) continue;
            int64_t orow = p0 + r;
            if (slot_rows && (a.tile_src == TILE_BLOCKS || a.orow == W4A16_OROW_SLOT)) {
                const int f = a.sorted_ids[p0 + r];
                if (f < 0 || f >= a.num_slots) continue;
                if (a.orow == W4A16_OROW_SLOT) orow = f;
            }
            if (a.out_kind == OUT_SILU) {
                // blocks 2h, 2h+1 are gate columns, 2h+4, 2h+5 the matching up
                uint16_t* o = static_cast<uint16_t*>(a.out) + orow * (a.N / 2) + chunk * 64 +
                              32 * h + (lane & 15);
                o[0] = f32_to_bf16_rne(silu_mul_bf16(acc[t][0][i], acc[t][2][i]));
                o[16] = f32_to_bf16_rne(silu_mul_bf16(acc[t][1][i], acc[t][3][i]));
            } else {
                const int64_t c0 = orow * a.N + chunk * 128 + 32 * h + (lane & 15);
                if (a.out_kind == OUT_BF16) {
                    uint16_t* o = static_cast<uint16_t*>(a.out) + c0;
                    o[0] = f32_to_bf16_rne(acc[t][0][i]);
                    o[16] = f32_to_bf16_rne(acc[t][1][i]);
                    o[64] = f32_to_bf16_rne(acc[t][2][i]);
                    o[80] = f32_to_bf16_rne(acc[t][3][i]);
                } else {
                    float* o = static_cast<float*>(a.out) + c0;
                    o[0] = acc[t][0][i];
                    o[16] = acc[t][1][i];
                    o[64] = acc[t][2][i];
                    o[80] = acc[t][3][i];
                }
            }
        }
    }
}

// Tiles are walked grid-stride along grid.y (the decision is uniform across
// the workgroup, so every barrier is reached by all four wavefronts).  The
// row-block count is rounded up to a multiple of 4 per tile.
__global__ void __launch_bounds__(256) k_gemm_large(GemmArgs a) {
    __shared__ u32x4 lds[2 * kStageU4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
        nrows = nrows < 256 ? nrows : 256;
        const int mb = (nrows + 63) >> 6;   // quarters of 256 rows
        if (mb <= 1) large_tile<4>(a, e, p0, nrows, wave, lane, lds);
        else if (mb == 2) large_tile<8>(a, e, p0, nrows, wave, lane, lds);
        else if (mb == 3) large_tile<12>(a, e, p0, nrows, wave, lane, lds);
        else large_tile<16>(a, e, p0, nrows, wave, lane, lds);
        __syncthreads();  // the next tile reuses the staging buffers
    }
}

void launch_gemm_large(const GemmArgs& a, hipStream_t st) {
    const dim3 grid((a.NC + 1) / 2, a.grid_tiles, 1), block(256);
    k_gemm_large<<<grid, block, 0, st>>>(a);
}

}  // namespace w4a16
