// Internal declarations of the W4A16 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/w4a16moe.h"

namespace w4a16 {

// ---- errors ---------------------------------------------------------------

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define W4A16_CHECK_ARG(cond, ...)                                  \
    do {                                                            \
        if (!(cond)) {                                              \
            ::w4a16::set_error(__VA_ARGS__);                        \
            return W4A16_ERR_INVALID_ARG;                           \
        }                                                           \
    } while (0)

// Map the sticky launch status to W4A16_ERR_HIP after launching on a stream.
w4a16_status check_launch(const char* what);

// ---- packed weight geometry ------------------------------------------------
//
// Per expert e and chunk c of CW packed columns, K/32 groups are padded to
// KSP = round_up(K/32, 8) and cut into KSP/8 records ("stages") of 8 groups.
// A record is contiguous: first the codes, then the scales of its 8 groups.
// Both profiles use 576 * WPL words per record.
//
// DECODE (CW = 64, operands of v_mfma_f32_16x16x32_bf16):
//   codes : word (g8, lane, j) at  (g8 * 64 + lane) * WPL + j      (g8 < 8)
//           = the eight codes of column c*CW + 16*j + lane%16 (packed order)
//             for K = ks*32 + 8*(lane/16) + o, o = 0..7, with the code of
//             offset o in nibble i where o = 2*(i%4) + i/4 (order
//             0,2,4,6,1,3,5,7): (word >> 4p) & 0x000F000F then selects
//             offsets (2p, 2p+1) in the two 16-bit halves
//   scales: bf16 (g8, c16, j) at  512*WPL words + (g8 * 16 + c16) * WPL + j
//           = the scale of column c*CW + 16*j + c16, group ks
// PREFILL (CW = 128, operands of v_mfma_f32_32x32x16_bf16; 32-column blocks
// j = 0..3, half h = 0, 1 owns blocks h and h + 2):
//   codes : word (g8, h, lane, v) at ((g8 * 2 + h) * 64 + lane) * 4 + v
//           = the eight codes of column c*CW + 32*(h + 2*(v/2)) + lane%32 for
//             K = ks*32 + 16*(v%2) + 8*(lane/32) + o, o = 0..7, in the
//             canonical nibble order (nibble o = offset o)
//   scales: bf16 (h, c32, g8, jj) at 4096 words + ((h * 32 + c32) * 8 + g8) * 2 + jj
//           = the scale of column c*CW + 32*(h + 2*jj) + c32, group ks (a
//           lane's scales of the record's 8 groups are 32 contiguous bytes)
// DECODE, MXFP4 for MXFP8 activations (W4A16_PACK_MXFP8_ACT; operands of
// v_mfma_scale_f32_16x16x128_f8f6f4, B in E2M1: lane l holds column l%16 for
// K = 32*(l/16) + o, o = 0..31, nibble o of its 16 bytes, low nibble first;
// a record is two 128-K steps s):
//   codes : word (s, j, lane, w) at ((s * WPL + j) * 64 + lane) * 4 + w
//           = canonical word (K/8 index) r*32 + s*16 + 4*(lane/16) + w of
//             column c*CW + 16*j + lane%16 (record r): 32 consecutive codes
//   scales: word (s, lane) at 512*WPL words + s * 64 + lane; byte j = the
//           E8M0 scale of column c*CW + 16*j + lane%16, group r*8 + 4*s +
//           lane/16 (the B-scale operand of block j, selected by op_sel)
// Padding groups (ks >= K/32) hold zero codes and zero scales.
// WPL = CW / 16 words (and scales) per lane per group.
struct PackGeom {
    int E, N, K, CW, NC, KS, KSP, WPL;
    bool interleave;
    bool mxfp4;                          // E2M1 codes in canonical nibble order, E8M0 scales as bf16
    bool a8;                             // MXFP4 laid out for MXFP8 activations (block-scaled MFMA)
    uint64_t stage_words, chunk_words;   // 32-bit words per record / per chunk
    uint64_t stage_bytes, chunk_bytes, bytes;
};

__host__ __device__ inline int nibble_k_offset(int i) { return 2 * (i & 3) + (i >> 2); }

// Packed column -> canonical column (gate/up interleave: within each CW
// chunk, the first CW/2 packed columns are gate columns and the last CW/2 the
// matching up columns).
__host__ __device__ inline int canonical_column(int nn, int N, int CW, bool interleave) {
    if (!interleave) return nn;
    int c = nn / CW, w = nn % CW, half = CW / 2;
    return w < half ? c * half + w : N / 2 + c * half + (w - half);
}

int chunk_width_of(int profile);
w4a16_status make_geom(int profile, uint32_t flags, int E, int N, int K, int group,
                       PackGeom* g);
w4a16_status check_desc(const w4a16_desc* d);

// ---- launchers (defined next to their kernels) ------------------------------

void launch_prepack(const PackGeom& g, const uint32_t* codes, const void* scales,
                    void* packed, hipStream_t s);

struct AlignArgs {
    const int32_t* topk_ids;
    int T, top_k, E_global, E_local, block_m;
    const int32_t* expert_map;
    w4a16_routing r;
    int32_t* err_flag;  // device int or nullptr (validation)
    // router top-k first (logits != nullptr): float [T, E_global] in, ids_out
    // [T, top_k] and weights_out [T, top_k] written, then sorted
    const float* logits;
    int32_t* ids_out;
    float* weights_out;
};
void launch_align(const AlignArgs& a, hipStream_t s);
void launch_router_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s);
constexpr int kRouterMaxExperts = 1024;   // 16 logits per lane of a wavefront
constexpr int kRouterMaxTopK = 64;        // one lane per selected expert

// How a GEMM block finds its rows.
enum TileSrc { TILE_TABLE = 0, TILE_BLOCKS = 1, TILE_MASKED = 2, TILE_CONTIG = 3 };
// What the GEMM stores: bf16 [rows, N], fp32 [rows, N], or SiLU(gate) * up
// as bf16 [rows, N/2] from a gate/up-interleaved weight.
enum OutKind { OUT_BF16 = 0, OUT_F32 = 1, OUT_SILU = 2 };

struct GemmArgs {
    // rows
    int tile_src, arow, orow, top_k, num_slots;
    const uint16_t* A;
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    const int32_t* ntp;
    const int32_t* tiles;
    const int32_t* tile_count;
    int block_m, tile_m;
    const int32_t* masked_m;
    int max_m, chunks_per_expert;
    const int32_t* m_indices;   // contiguous: expert of each row (-1 padding)
    int grid_tiles;        // tiles the host expects (sizes the persistent grids)
    int tiles_cap;         // tile indices that may hold work (bound of the device count)
    int grid_tiles_total;  // masked: experts * chunks_per_expert
    // weights (packed records, see PackGeom)
    const uint32_t* packed;
    int64_t chunk_words, stage_words;
    int NC, KS, KSP, N, K, CW, E;
    int64_t A_rows;    // rows of A (row indices are clamped below it)
    int sorted_cap;    // entries of sorted_ids
    // output
    void* out;
    int out_kind;
    int split_k;
    // split-K (split_k > 1): fp32 partials [split_k][ws_stride] (rows of the
    // position-indexed space x N; ws_stride * 4 bytes < 4 GiB, checked on the
    // host) and one arrival counter per (tile, column group), zero between
    // calls
    float* partials;
    int32_t* counters;
    int64_t ws_stride;
    // fused top-k combine (comb_out != nullptr): arrival counters [comb_T]
    // [comb_groups] (zero between calls), one per token and 256 columns
    uint16_t* comb_out;
    const int32_t* comb_row_of;
    const float* comb_w;
    int32_t* comb_counters;
    int comb_T, comb_groups;
    uint32_t unpack_mask;  // 0x000F000F: one code in each 16-bit half
    uint32_t unpack_bits;  // 0x43004300: bf16 exponent of 128 in each half
    uint32_t nib_mask;     // 0x0F0F0F0F: one code in each byte
    int fp4;               // MXFP4 weights (E2M1 codes): streaming kernel only
    int a8;                // A8W4: A holds E4M3 bytes [A_rows, K], A_scales E8M0 [A_rows, K/32]
    const uint8_t* A_scales;
};
// wide: the 8-group code ring (three workgroups per CU up to two row blocks)
// instead of the 16-group one, for two-block tiles.
void launch_gemm_small(const GemmArgs& a, int mt, bool wide, hipStream_t s);
// A8W4 kernel (weights packed with W4A16_PACK_MXFP8_ACT, MXFP8 activations;
// tiles of up to 16 * mt rows, no K split).
void launch_gemm_mx(const GemmArgs& a, int mt, hipStream_t s);
// Large-M kernel (PREFILL profile only, tiles of up to 256 rows, no K split).
void launch_gemm_large(const GemmArgs& a, hipStream_t s);

// SiLU(gate) * up over positions p < rows (p < min(*rows_dev, rows) when
// rows_dev is given).  masked_m != nullptr: p is skipped when p % max_m >=
// masked_m[p / max_m] (counts cut to max_m).  sorted_ids != nullptr: p is
// skipped unless f = sorted_ids[p] is in [0, num_slots); its row is f when
// slot_rows, else p.
void launch_silu_mul(const uint16_t* y13, int64_t rows, const int32_t* rows_dev, int I,
                     const int32_t* masked_m, int max_m, const int32_t* sorted_ids, int num_slots,
                     bool slot_rows, uint16_t* z, hipStream_t s);
// MXFP8 conversion (A8W4 activations) of rows [0, min(*rows_dev, rows)) of
// x [rows, K] bf16 into codes [rows, K] and scale bytes [rows, K/32].
void launch_quant_mxfp8(const uint16_t* x, int64_t rows, const int32_t* rows_dev, int K,
                        uint8_t* codes, uint8_t* scales, hipStream_t s);
// Indexed -> masked placement from a routing sort made with block_m = 1
// (no padding): sorted position p of expert e has rank p - offsets[e].
struct MaskedPlaceArgs {
    const uint16_t* X;          // [T, H] bf16
    int H, top_k, num_slots;
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    const int32_t* ntp;
    int sorted_cap;
    const int32_t* offsets;     // [E + 1]
    const int32_t* row_of;      // slot -> position, -1 if not local
    int E, max_m;
    uint16_t* a3;               // [E * max_m, H]
    int32_t* masked_m;          // [E]
    int32_t* row_of_masked;     // [num_slots]
    int32_t* dropped;           // [1] or nullptr
};
void launch_to_masked(const MaskedPlaceArgs& a, hipStream_t s);

// Zero `bytes` (a multiple of 16) at p, 16-byte aligned, with a kernel.
void launch_zero(void* p, uint64_t bytes, hipStream_t s);
void launch_combine(const uint16_t* y, int64_t y_rows, int H, const int32_t* row_of,
                    const float* w, int T, int top_k, uint16_t* out, hipStream_t s);

}  // namespace w4a16
