/*
 * w4a16moe.h -- C ABI of the W4A16 INT4 Mixture-of-Experts expert path for
 * AMD Instinct MI355X (gfx950).
 *
 * Source page for every operation declared here ("Chord page"): "vLLM x Novita
 * AI: Chord W4A16 INT4 MoE kernels for Kimi K2.x" (novita.ai blog).  Section
 * names are given in English translation.
 *
 * The path: BF16 activations X [T, H]; INT4 expert weights with one BF16 scale
 * per group of 32 along K (TL;DR; "Grouped SM90 kernels", operator listing:
 * weight [G, N, K] uint4, scale [G, N, K/32] bf16); routed rows grouped by
 * expert in the indexed layout (sorted_ids / expert_ids / num_tokens_padded,
 * "Two kernel families") or the grouped masked layout (per-expert valid count
 * masked_m on the device plus a host hint expected_m, "Grouped SM90
 * kernels"); then gate/up GEMM -> SiLU(gate) * up -> down GEMM -> top-k
 * weighted combine.
 *
 * Conventions shared by every call
 *   - Device pointers point to GPU memory of the current HIP device; host
 *     pointers are marked "host".  The caller owns every buffer.  The library
 *     never allocates or frees device memory and keeps no pointer after a call
 *     returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call that
 *     launches work is asynchronous on that stream and never synchronises the
 *     host, except w4a16_moe_align with W4A16_ALIGN_VALIDATE set.
 *   - bf16 tensors are arrays of uint16 bit patterns; all tensors are dense,
 *     row-major, without padding between rows.
 *   - Every call returns a w4a16_status.  Argument checks run on the host
 *     before anything is launched; on failure nothing is launched and
 *     w4a16_last_error() describes the problem.  No call falls back to another
 *     implementation silently.
 *
 * Weight boundary format (what the caller hands to w4a16_prepack)
 *   codes  : int32 [E, N, K/8]; code c of a row sits in word c/8 at bits
 *            4*(c%8) .. 4*(c%8)+3 (low nibble = lowest K); the code q in
 *            0..15 stands for the signed value q - 8.
 *   scales : bf16 [E, N, K/32]; w[e][n][c] = (q - 8) * scales[e][n][c/32]
 *            (subtract, then scale: "H200 and Blackwell indexed decode").
 *   The gate projection is W13 rows [0, I), the up projection rows [I, 2I).
 */
#ifndef W4A16MOE_H
#define W4A16MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* Status codes                                                             */
/* ------------------------------------------------------------------------ */
typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, misaligned pointer, expected_m <= 0 */
    W4A16_ERR_UNSUPPORTED = 2,   /* group != 32, K or N not a multiple of the packing unit, profile */
    W4A16_ERR_MODE_MISMATCH = 3, /* prepared weight used in a mode it was not packed for */
    W4A16_ERR_CAPACITY = 4,      /* a caller buffer (routing, tiles, output, workspace) too small */
    W4A16_ERR_ROUTING = 5,       /* expert id out of range (reported only under VALIDATE) */
    W4A16_ERR_HIP = 6            /* a HIP runtime call or kernel launch failed */
} w4a16_status;

/* Thread-local, human-readable message for the last non-OK status of this
 * thread ("" when none).  The pointer stays valid until the next call. */
const char* w4a16_last_error(void);

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t w4a16_version(void);

/* ------------------------------------------------------------------------ */
/* Load time: prepacking (Chord page, "Indexed kernels" and Figure 2: the    */
/* profile and the weight layout are fixed when the model is loaded; the     */
/* token count only tunes the schedule inside a profile.  "vLLM             */
/* integration": unsupported quantisation schemes fail at load time.         */
/* "Grouped SM90 kernels": the mode is recorded in the prepared weight and   */
/* checked at dispatch).                                                     */
/* ------------------------------------------------------------------------ */
typedef enum {
    W4A16_PROFILE_DECODE = 1,  /* few routed rows per expert: weight streaming,
                                  64 output columns per wavefront chunk        */
    W4A16_PROFILE_PREFILL = 2  /* many routed rows per expert: MFMA-bound,
                                  128 output columns per wavefront chunk       */
} w4a16_profile;

/* Prepack flags. */
#define W4A16_PACK_GATE_UP_INTERLEAVE 0x1u /* W13 only: interleave gate and up
    column blocks so that one wavefront owns matching gate/up columns (allows
    the SiLU(gate)*up epilogue inside the gate/up GEMM) */

#define W4A16_PACK_MXFP4 0x2u /* set by w4a16_prepack_mxfp4 (recorded in the
    descriptor): the weights are MXFP4, E2M1 codes with one E8M0 scale per 32
    (news.ainew.jp, "vLLM publishes Kimi K3 production support", MXFP4 MoE:
    4-bit floating-point expert weights with shared power-of-two block
    scales).  DECODE profile only; the GEMM then runs the streaming kernel's
    MXFP4 variant */

#define W4A16_PACK_MXFP8_ACT 0x4u /* with W4A16_PACK_MXFP4 (w4a16_prepack_mxfp4,
    DECODE profile): A8W4, MXFP4 weights for MXFP8 activations (news.ainew.jp,
    "vLLM publishes Kimi K3 production support", MXFP4 MoE: A8W4 fused
    operators on AMD, 8-bit activations on 4-bit weights).  The weights are
    laid out for CDNA4's block-scaled matrix instruction (E4M3 x E2M1, 128 K
    per instruction, E8M0 scales applied by the hardware), and every GEMM on
    them takes MXFP8 activations (w4a16_gemm_args.A_scales) */

#define W4A16_DESC_MAGIC 0x4D413457u   /* "W4AM" as little-endian bytes */
#define W4A16_DESC_VERSION 1u

/* Plain-old-data record of a prepared weight.  Produced by w4a16_prepack,
 * passed back unchanged with the packed buffer to every GEMM call, where its
 * magic, version, profile, flags and shape are checked. */
typedef struct {
    uint32_t magic;          /* W4A16_DESC_MAGIC */
    uint32_t version;        /* W4A16_DESC_VERSION */
    int32_t profile;         /* w4a16_profile */
    uint32_t flags;          /* W4A16_PACK_* */
    int32_t E;               /* experts */
    int32_t N;               /* output columns (2I for W13, H for W2) */
    int32_t K;               /* reduction length (H for W13, I for W2) */
    int32_t group;           /* always 32 */
    int32_t chunk_n;         /* output columns per packed wavefront chunk */
    int32_t k_groups;        /* K/32 rounded up to a multiple of 8 (padding groups are zero) */
    uint64_t stage_bytes;    /* bytes of one 8-group record of one chunk (codes then scales) */
    uint64_t chunk_bytes;    /* bytes of one chunk over all of K */
    uint64_t bytes;          /* total bytes of the packed buffer */
} w4a16_desc;

/* Size of the packed buffer for a profile and shape (host call, no GPU).
 * UNSUPPORTED if group != 32, K % 32 != 0 or N is not a multiple of the
 * profile's chunk width (64 DECODE, 128 PREFILL).
 * Layout: for each expert and each chunk of chunk_n packed output columns,
 * K is cut into records of 8 groups of 32; a record holds the chunk's codes
 * for those groups (lane-major, in MFMA operand order) followed by their
 * scales, so one wavefront streams one contiguous region. */
w4a16_status w4a16_prepack_bytes(int32_t profile, uint32_t flags, int32_t E, int32_t N,
                                 int32_t K, int32_t group, uint64_t* bytes /* host out */);

/* Permute canonical codes and scales into the profile's device layout.
 *   codes  : device int32 [E, N, K/8], canonical format above
 *   scales : device bf16 [E, N, K/32]
 *   packed : device, caller-owned, >= w4a16_prepack_bytes(...) bytes, 256-byte aligned
 *   desc   : host out, filled on success
 * One launch on `stream`; a pure bit permutation (no arithmetic on values). */
w4a16_status w4a16_prepack(int32_t profile, uint32_t flags, const int32_t* codes,
                           const uint16_t* scales, int32_t E, int32_t N, int32_t K,
                           int32_t group, void* packed, uint64_t packed_bytes,
                           w4a16_desc* desc /* host out */, void* stream);

/* MXFP4 weights (W4A16_PACK_MXFP4): the same layout as w4a16_prepack's
 * DECODE profile, from
 *   codes       : device int32 [E, N, K/8]; code c of a row sits in word c/8 at
 *                 bits 4*(c%8) .. +3; the code is an E2M1 number (bit 3 sign,
 *                 bits 2..1 exponent, bit 0 mantissa: +-{0, 0.5, 1, 1.5, 2, 3,
 *                 4, 6})
 *   scales_e8m0 : device uint8 [E, N, K/32]; block scale 2^(b - 127), b = 255
 *                 NaN
 * so w[e][n][c] = e2m1(code) * 2^(b - 127).  Codes keep their canonical nibble
 * order (byte b of a word holds K offsets 2b and 2b + 1, the operand order of
 * the hardware E2M1 -> bf16 conversion); each scale is stored as the bf16
 * 2^(b - 127), which is exact.  UNSUPPORTED with the PREFILL profile.  flags
 * may hold W4A16_PACK_GATE_UP_INTERLEAVE; the descriptor records
 * W4A16_PACK_MXFP4.  w4a16_prepack and w4a16_prepack_host refuse the MXFP4
 * flag (their scales are bf16). */
w4a16_status w4a16_prepack_mxfp4(int32_t profile, uint32_t flags, const int32_t* codes,
                                 const uint8_t* scales_e8m0, int32_t E, int32_t N, int32_t K,
                                 int32_t group, void* packed, uint64_t packed_bytes,
                                 w4a16_desc* desc /* host out */, void* stream);

/* Host-side reference of w4a16_prepack_mxfp4 (host buffers). */
w4a16_status w4a16_prepack_mxfp4_host(int32_t profile, uint32_t flags, const int32_t* codes,
                                      const uint8_t* scales_e8m0, int32_t E, int32_t N,
                                      int32_t K, int32_t group, void* packed,
                                      uint64_t packed_bytes, w4a16_desc* desc);

/* Host-side reference of the same permutation (no GPU), for load-time
 * tooling and tests.  Buffers are host memory. */
w4a16_status w4a16_prepack_host(int32_t profile, uint32_t flags, const int32_t* codes,
                                const uint16_t* scales, int32_t E, int32_t N, int32_t K,
                                int32_t group, void* packed, uint64_t packed_bytes,
                                w4a16_desc* desc);

/* ------------------------------------------------------------------------ */
/* Routing metadata, indexed layout (Chord page, "Two kernel families": the  */
/* indexed family consumes vLLM's sorted_ids / expert_ids /                  */
/* num_tokens_padded; "vLLM integration": the over-allocated align buffers   */
/* are consumed without reading routing counts back to the host, which keeps */
/* the path graph-capturable; Figure 3: activations are never padded, the    */
/* routing indices carry the padding sentinels).                             */
/* ------------------------------------------------------------------------ */

/* Buffers written by w4a16_moe_align (all device memory, caller-owned). */
typedef struct {
    int32_t* sorted_ids;        /* [sorted_cap]: for each local expert e in
                                   ascending order, its routed slots f = t*k+j in
                                   ascending order, then the sentinel T*k up to a
                                   multiple of block_m; the tail after
                                   num_tokens_padded also holds the sentinel */
    int32_t sorted_cap;
    int32_t* expert_ids;        /* [blocks_cap]: local expert of each block_m
                                   block of sorted_ids; -1 past the last block */
    int32_t blocks_cap;
    int32_t* num_tokens_padded; /* [1]: padded total (sum of padded segments) */
    int32_t* row_of;            /* [T*k] or NULL: position of slot f in
                                   sorted_ids, -1 if f is not routed to a local
                                   expert */
    int32_t* tiles;             /* [tiles_cap][4] or NULL: GEMM row tiles
                                   {expert, first position, rows, 0}: each local
                                   expert's rows cut into pieces of at most tile_m
                                   rows (expert-major, ascending); entries past
                                   *tile_count are not written */
    int32_t tiles_cap;
    int32_t* tile_count;        /* [1] (required when tiles != NULL) */
    int32_t tile_m;             /* rows per tile, multiple of 16, <= 256 */
    int32_t* expert_offsets;    /* [E_local + 1] or NULL: start of each local
                                   expert's padded segment in sorted_ids, then
                                   num_tokens_padded */
} w4a16_routing;

#define W4A16_ALIGN_VALIDATE 0x1u  /* read routing back and report ROUTING for
                                      out-of-range expert ids (synchronises) */

/* Capacities that always suffice for T tokens, top_k, E_local experts. */
w4a16_status w4a16_moe_align_capacity(int32_t T, int32_t top_k, int32_t E_local,
                                      int32_t block_m, int32_t tile_m,
                                      int32_t* sorted_cap, int32_t* blocks_cap,
                                      int32_t* tiles_cap /* host outs */);

/* Stable counting sort of routed slots by local expert.
 *   topk_ids   : device int32 [T, top_k], global expert ids
 *   expert_map : device int32 [E_global] global -> local id or -1; NULL = identity
 *   Ids outside [0, E_global), or mapping outside [0, E_local), are skipped
 *   like non-local experts.  1 <= E_local <= 1024, 1 <= block_m <= 256.
 * Output is fully determined by the input (bit-reproducible). */
w4a16_status w4a16_moe_align(const int32_t* topk_ids, int32_t T, int32_t top_k,
                             int32_t E_global, const int32_t* expert_map, int32_t E_local,
                             int32_t block_m, const w4a16_routing* routing, uint32_t flags,
                             void* stream);

/* ------------------------------------------------------------------------ */
/* The step before the expert GEMMs: router top-k (the pages list an        */
/* optimised expert routing step ahead of the grouped GEMMs, outside their   */
/* timed unit; news.ainew.jp, "vLLM publishes Kimi K3 production support",   */
/* TL;DR), fused with the routing sort when the sort runs as one workgroup.  */
/*   logits : device float [T, E_global], finite                            */
/*   topk_ids [T, top_k] (written): the top_k experts with the largest        */
/*            logits, largest first, equal logits in ascending expert id     */
/*   topk_weights [T, top_k] (written): softmax over the selected logits,     */
/*            e^(l_j - l_0) / sum_i e^(l_i - l_0) in fp32, summed in j order  */
/* 1 <= E_global <= 1024, 1 <= top_k <= min(64, E_global); INVALID_ARG else. */
/* ------------------------------------------------------------------------ */
w4a16_status w4a16_moe_router_topk(const float* logits, int32_t T, int32_t E_global,
                                   int32_t top_k, int32_t* topk_ids, float* topk_weights,
                                   void* stream);

/* Router top-k, then w4a16_moe_align on its ids (same arguments, outputs
 * and errors).  One launch when the sort runs as one workgroup (up to 2047
 * routed slots at 16 wavefronts: decode sizes), else the router kernel then
 * the sort. */
w4a16_status w4a16_moe_route_align(const float* logits, int32_t T, int32_t E_global,
                                   int32_t top_k, const int32_t* expert_map, int32_t E_local,
                                   int32_t block_m, const w4a16_routing* routing,
                                   int32_t* topk_ids, float* topk_weights, uint32_t flags,
                                   void* stream);

/* Indexed routing -> grouped masked layout, on the device (Chord page,
 * "Grouped SM90 kernels": the masked dispatch takes rows already placed per
 * expert, [G, max_m, K], with each expert's valid count in masked_m; "vLLM
 * integration": routing counts stay on the device).  Local slots f = t*k + j
 * in ascending order: the i-th local slot of expert e goes to row e*max_m + i
 * when i < max_m, a3 row = X[f / k] and row_of[f] = e*max_m + i; non-local
 * slots and ranks i >= max_m get row_of[f] = -1 (the latter are dropped and
 * counted in *dropped); masked_m[e] = min(count_e, max_m).  Rows of a3 not
 * written keep their contents.
 *   X       : device bf16 [X_rows >= T, H], H % 8 == 0, 16-byte aligned
 *   scratch : caller-owned routing buffers for a sort with block_m = 1
 *             (capacities from w4a16_moe_align_capacity(T, top_k, E_local,
 *             1, 0)); row_of and expert_offsets required, tiles ignored;
 *             overwritten by the call
 *   a3      : device bf16 [E_local * max_m, H], 16-byte aligned
 *   masked_m: device int32 [E_local]; row_of: device int32 [T * top_k];
 *   dropped : device int32 [1] or NULL
 * Two launches on `stream` (the sort, then the placement). */
w4a16_status w4a16_moe_indexed_to_masked(const uint16_t* X, int64_t X_rows, int32_t H,
                                         const int32_t* topk_ids, int32_t T, int32_t top_k,
                                         int32_t E_global, const int32_t* expert_map,
                                         int32_t E_local, int32_t max_m,
                                         const w4a16_routing* scratch, uint16_t* a3,
                                         int32_t* masked_m, int32_t* row_of, int32_t* dropped,
                                         void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped W4A16 GEMM (Chord page, "H200 prefill and TP8", "H200 and        */
/* Blackwell indexed decode", "Grouped SM90 kernels").                       */
/*   out[p, n] = bf16( sum_c A[row(p), c] * (q[e,n,c] - 8) * s[e,n,c/32] )   */
/* with fp32 accumulation, for every routed row p of expert e.  The INT4     */
/* codes are unpacked and scaled in registers; no dequantised copy exists.   */
/* ------------------------------------------------------------------------ */
typedef enum {
    W4A16_LAYOUT_INDEXED = 0,    /* rows found through sorted_ids (vLLM routing) */
    W4A16_LAYOUT_MASKED = 1,     /* [G * max_m] rows, masked_m valid per expert */
    W4A16_LAYOUT_CONTIGUOUS = 2  /* [m] rows concatenated per expert, each expert's
                                    segment padded to a multiple of 128 rows, the
                                    expert of each row in m_indices (-1 on padding)
                                    ("Grouped SM90 kernels", contiguous prefill and
                                    Figure 3).  PREFILL-profile weights only */
} w4a16_layout;

/* How an indexed row position p finds its activation row. */
typedef enum {
    W4A16_AROW_TOKEN = 0,    /* A row = sorted_ids[p] / top_k (gate/up on X [T, K]) */
    W4A16_AROW_SLOT = 1,     /* A row = sorted_ids[p]         (A is [T*k, K])       */
    W4A16_AROW_POSITION = 2  /* A row = p                     (A is compact, e.g. Z) */
} w4a16_arow;

/* Where an indexed row position p writes its output row. */
typedef enum {
    W4A16_OROW_POSITION = 0, /* out row p (compact [sorted_cap, N]) */
    W4A16_OROW_SLOT = 1      /* out row sorted_ids[p] ([T*k, N]) */
} w4a16_orow;

typedef enum {
    W4A16_EPI_STORE = 0,     /* store bf16(acc) */
    W4A16_EPI_SILU_MUL = 1   /* W13 only: store bf16(silu(bf16(gate)) * bf16(up)),
                                out is [rows, N/2].  With a W13 packed with
                                GATE_UP_INTERLEAVE it is applied to the
                                accumulators in the GEMM kernel; with a plain
                                W13 the GEMM stages bf16 Y13 in the workspace
                                at the rows it would store (positions, or
                                slots with OROW_SLOT) and a second kernel
                                applies it to those rows (same result; padding
                                rows are skipped in both) */
} w4a16_epilogue;

#define W4A16_GEMM_F32_OUT 0x1u  /* store the fp32 accumulator (float) instead of
                                    bf16; EPI_STORE only (exactness tests) */

typedef struct {
    int32_t layout;                 /* w4a16_layout */
    int32_t epilogue;               /* w4a16_epilogue */
    uint32_t flags;                 /* W4A16_GEMM_* */
    int32_t split_k;                /* 0 = automatic; >1 forces K splits (INDEXED
                                       only: MASKED rejects it, MODE_MISMATCH).
                                       Each split keeps an fp32 partial of
                                       sorted_cap x N; a forced split whose
                                       partial reaches 4 GiB is UNSUPPORTED (the
                                       automatic choice then runs unsplit).
                                       Ignored (no split) with OROW_SLOT or
                                       F32_OUT and with a PREFILL weight */
    const uint16_t* A;              /* device bf16 activations, [A_rows, K];
                                       A_rows * K * 2 bytes must stay below
                                       4 GiB (else UNSUPPORTED) */
    int64_t A_rows;
    /* INDEXED */
    int32_t arow;                   /* w4a16_arow */
    int32_t orow;                   /* w4a16_orow */
    int32_t top_k;                  /* for AROW_TOKEN; sentinel = num_slots */
    int32_t num_slots;              /* T * top_k (the sentinel value) */
    const int32_t* sorted_ids;      /* device [sorted_cap] */
    int32_t sorted_cap;
    const int32_t* expert_ids;      /* device [blocks_cap]; used when tiles == NULL */
    int32_t blocks_cap;
    int32_t block_m;                /* align granule; tile height when tiles == NULL */
    const int32_t* num_tokens_padded; /* device [1] */
    const int32_t* tiles;           /* device [tiles_cap][4] from w4a16_moe_align, or NULL */
    int32_t tiles_cap;
    const int32_t* tile_count;      /* device [1] */
    int32_t tile_m;                 /* rows per tile: the tile_m the table was
                                       written with (w4a16_routing.tile_m).  A
                                       table entry with more rows than this is
                                       cut to tile_m rows; the rows past it are
                                       neither computed nor stored */
    int32_t rows_hint;              /* host: expected routed rows on this GPU (launch
                                       choice only; 0 = unknown) */
    /* MASKED */
    const int32_t* masked_m;        /* device int32 [G]: valid rows of each expert;
                                       a count above max_m counts as max_m, one
                                       <= 0 as no rows */
    int32_t max_m;                  /* rows reserved per expert; A is [G*max_m, K] */
    int32_t expected_m;             /* host hint > 0, launch choice only */
    /* weights */
    const void* packed;             /* device, from w4a16_prepack */
    const w4a16_desc* desc;         /* host */
    /* output */
    void* out;                      /* device; bf16 (or float with F32_OUT) */
    int64_t out_rows;               /* rows available in out */
    /* scratch: device, 256-byte aligned, >= w4a16_gemm_workspace_bytes(...).
       It starts with counters (split-K arrival counters; with a PREFILL
       weight, the 256-byte work-queue block), which must read zero when a
       call starts: allocate it zeroed.  A completed call leaves the counters
       it used at zero but may leave partial sums after them, so a workspace
       reused for a call of another shape, split or tile capacity must be
       zeroed again first.  Calls that share a workspace must not run
       concurrently. */
    void* workspace;
    uint64_t workspace_bytes;
    /* CONTIGUOUS: device int32 [A_rows]: expert of each row of A (and of out),
       -1 on padding.  Every expert's segment starts on a 128-row boundary, so
       a block of 128 (or 64) rows holds one expert: the expert of a block is
       that of its first row (a block starting with padding is skipped), and
       only the block's rows whose index equals it are stored.  A is [m, K] with
       m = A_rows; out is [m, N] (N/2 with SILU_MUL), out_rows >= m.  split_k
       overrides are refused (MODE_MISMATCH). */
    const int32_t* m_indices;
    /* Fused top-k weighted combine (the down GEMM's epilogue; Chord page,
       "Measurements": the expert outputs are merged per token after the down
       GEMM).  When comb_out != NULL the call also writes
         comb_out[t, n] = bf16( sum_{j<k, row_of[t*k+j] >= 0} w[t, j] * out[row_of[t*k+j], n] )
       in fp32, j ascending, on the bf16 rows it stores: the same bits as
       w4a16_moe_combine on those rows.  The last of a token's rows to be
       stored (per group of 256 columns) triggers its sum, so nothing waits
       and the order of the sum is fixed; tokens with no local slot get +0.
       Needs INDEXED with a tile table, OROW_POSITION, EPI_STORE, bf16 output
       (no F32_OUT); out then holds the compact rows [sorted_cap, N] the sums
       read.  Arrival counters (T * ceil(N / 256) ints) join the workspace's
       counters. */
    uint16_t* comb_out;             /* device bf16 [comb_T, N] */
    const int32_t* comb_row_of;     /* device int32 [comb_T * top_k]: row_of from w4a16_moe_align */
    const float* comb_weights;      /* device float [comb_T, top_k] */
    int32_t comb_T;                 /* tokens */
    /* A8W4 (a weight packed with W4A16_PACK_MXFP8_ACT; NULL otherwise, else
       MODE_MISMATCH): A then holds MXFP8 activations, E4M3 bytes [A_rows, K],
       and A_scales their E8M0 block scales, bytes [A_rows, K/32] (both as
       w4a16_quantize_mxfp8 writes them), so that
         out[p, n] = sum_c e4m3(A[row, c]) 2^(A_scales[row, c/32] - 127) * w[e][n][c]
       with fp32 accumulation inside the matrix instruction (an order the
       hardware fixes: the sum is exact whenever every partial sum is).
       INDEXED layout only, no K split (split_k overrides ignored), no fused
       combine (UNSUPPORTED); A_rows * K bytes below 4 GiB. */
    const uint8_t* A_scales;
} w4a16_gemm_args;

/* Workspace needed by this GEMM call (0 when none).  Host call. */
w4a16_status w4a16_gemm_workspace_bytes(const w4a16_gemm_args* args, uint64_t* bytes);

/* Run one grouped GEMM stage.  Checks the descriptor (magic, version, shape,
 * flags vs epilogue) before launching: a weight packed with gate/up
 * interleave used with EPI_STORE is a MODE_MISMATCH; so is any split_k
 * override under MASKED (the grouped dispatch owns its schedule).  Rows of
 * padding, rows past masked_m and experts with no rows are never stored;
 * experts with masked_m == 0 read no weights.  With a K split, each split
 * leaves an fp32 partial in the workspace and the split that finishes last
 * adds them in split order, inside the same kernel: results do not depend on
 * the order in which splits finish. */
w4a16_status w4a16_moe_w4a16_gemm(const w4a16_gemm_args* args, void* stream);

/* Allocation-free variant of w4a16_moe_w4a16_gemm, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, checks, kernels and
 * results; args->workspace and args->workspace_bytes are ignored.  Instead,
 * the call uses a static scratch array of the library (32 MiB per GPU, held
 * from the library's load until the process ends), whose device address is
 * looked up once per device on that device's first call.  A call whose
 * workspace (w4a16_gemm_workspace_bytes) exceeds 32 MiB returns CAPACITY
 * before anything is launched.  The call allocates and frees nothing.
 * Every call on one GPU shares that GPU's array: the call clears the part
 * that must start at zero (its counters) with a kernel on `stream`, and calls
 * that may overlap on one GPU (different streams, or different threads
 * without ordering) race on it and must be serialised by the caller. */
w4a16_status w4a16_moe_w4a16_gemm_noalloc(const w4a16_gemm_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Activation between the GEMMs (Chord page, "Measurements": the activation  */
/* is the step between the timed gate/up and down GEMMs; the path's          */
/* activation is SiLU of the gate half times the up half of the gate/up      */
/* output).                                                                  */
/*   Z[r, j] = bf16( silu(g) * u ), g = Y13[r, j], u = Y13[r, I + j],        */
/* silu(g) = g / (1 + exp(-g)), evaluated in fp32 without overflow: within  */
/* one bf16 ulp of the exact value for every finite bf16 g, and the same     */
/* function as the fused SILU_MUL epilogue.                                  */
/*   y13: device bf16 [rows, 2I]; z: device bf16 [rows, I]; I % 8 == 0.      */
/* Rows [0, min(*rows_dev, rows)) when rows_dev != NULL (device count, e.g.  */
/* num_tokens_padded), else [0, rows).  INVALID_ARG on null or misaligned    */
/* buffers (16 bytes) or a bad I.                                            */
/* ------------------------------------------------------------------------ */
w4a16_status w4a16_moe_silu_mul(const uint16_t* y13, int64_t rows, const int32_t* rows_dev,
                                int32_t I, uint16_t* z, void* stream);

/* ------------------------------------------------------------------------ */
/* MXFP8 activations for A8W4 (news.ainew.jp, "vLLM publishes Kimi K3        */
/* production support", MXFP4 MoE: A8W4 operators, 8-bit activations).  The */
/* OCP microscaling conversion of each block of 32 along a row:              */
/*   scale byte b = clamp(floor(log2 amax) - 8 + 127, 0, 254)  (8: exponent  */
/*   of E4M3's largest normal; an all-zero block takes b = 0)                */
/*   code_i = E4M3 nearest to x_i / 2^(b - 127), ties to the even mantissa,  */
/*            saturating at +-448                                            */
/*   x: device bf16 [rows, K], finite; codes: device uint8 [rows, K];        */
/*   scales: device uint8 [rows, K/32]; K a positive multiple of 32.         */
/* Rows [0, min(*rows_dev, rows)) when rows_dev != NULL (device count, e.g.  */
/* num_tokens_padded), else [0, rows).  INVALID_ARG on null or misaligned    */
/* buffers (x and codes 16 bytes) or a bad K.                                */
/* ------------------------------------------------------------------------ */
w4a16_status w4a16_quantize_mxfp8(const uint16_t* x, int64_t rows, const int32_t* rows_dev,
                                  int32_t K, uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------ */
/* Top-k weighted combine (Chord page, "Measurements": the expert outputs of */
/* the timed GEMMs are merged per token after the down GEMM, outside the     */
/* timed unit; the merge is the router's top-k weighted sum):                */
/*   out[t, h] = bf16( sum_{j<k, row_of[t*k+j] >= 0} w[t, j] * y[row_of[t*k+j], h] ) */
/* fp32, j ascending, each product and sum rounded separately; a token with */
/* no local slot gives +0.  y: device bf16 [y_rows, H]; row_of: device       */
/* int32 [T*k] (entries outside [0, y_rows) are skipped); topk_weights:      */
/* device float [T, k]; out: device bf16 [T, H].  INVALID_ARG on null or     */
/* misaligned buffers (16 bytes) or H not a positive multiple of 8.          */
/* ------------------------------------------------------------------------ */
w4a16_status w4a16_moe_combine(const uint16_t* y, int64_t y_rows, int32_t H,
                               const int32_t* row_of, const float* topk_weights, int32_t T,
                               int32_t top_k, uint16_t* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Schedule choice (Chord page, "H200 prefill and TP8": block-M from routed */
/* tokens per expert with an 80-rows/expert threshold and a 176-row cap;     */
/* shape-aware stream-K gating; "Grouped SM90 kernels": masked BM from       */
/* expected_m, wave-aware BN, latency-tuned buffered K).  Host only; the     */
/* constants are this library's own, measured on gfx950.                    */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t block_m;     /* align granule (sorted_ids padding) */
    int32_t tile_m;      /* rows per GEMM tile */
    int32_t split_k;     /* K splits (1 = none) */
    int32_t kernel;      /* 1 = small-M streaming kernel, 2 = large-M LDS kernel */
    int32_t ring_groups; /* streaming kernel: K groups of codes in flight per
                            wavefront, 8 (three workgroups per CU up to 32-row
                            tiles) or 16; 0 for the large-M kernel */
} w4a16_plan;

/* INDEXED: rows_hint = routed rows expected on this GPU (0 = unknown), tile_m
 * 0 = choose.  MASKED: expected_m > 0.  CONTIGUOUS (PREFILL profile, else
 * MODE_MISMATCH): rows_hint = m; block_m is the 128-row segment alignment,
 * tile_m is 128 when ceil(m / 128) blocks times the column pairs of the
 * large-M kernel fill the 256 compute units, else 64. */
w4a16_status w4a16_plan_gemm(const w4a16_desc* desc, int32_t layout, int32_t rows_hint,
                             int32_t expected_m, int32_t tile_m, w4a16_plan* plan /* host out */);

#ifdef __cplusplus
}
#endif

#endif /* W4A16MOE_H */
