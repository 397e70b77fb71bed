// C ABI entry points: argument checks, schedule choice, launches.
//
// Every check runs on the host before anything is launched (Chord page,
// "vLLM integration": unsupported schemes fail loudly instead of selecting a
// wrong kernel; "Grouped SM90 kernels": a weight prepared for one mode fails
// loudly in another, and the grouped dispatch owns its schedule and refuses
// tuning overrides).

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "internal.h"

namespace w4a16 {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = 0; }

w4a16_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: HIP launch failed: %s", what, hipGetErrorString(e));
        return W4A16_ERR_HIP;
    }
    return W4A16_OK;
}

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Largest tile height of the streaming kernel (DECODE profile, 4 MFMA row
// blocks) and of the large-M kernel (PREFILL profile, 8 row blocks of 32).
// The profile, fixed at load time, picks the kernel; the routed rows per
// expert pick the tile height inside it.
static constexpr int kSmallMaxTile = 64;
static constexpr int kLargeMaxTile = 256;

static int max_tile(const w4a16_desc* d) {
    return d->profile == W4A16_PROFILE_PREFILL ? kLargeMaxTile : kSmallMaxTile;
}

__device__ int32_t g_routing_errors;

// ---- schedule choice ---------------------------------------------------------
//
// The indexed rule follows the shape of the page's resolver (block height from
// routed rows per expert tok_e, not from the total), with CDNA4 constants:
// the tile is sized to hold an expert's rows in one pass, in 16-row MFMA
// steps: twice the mean up to 16 rows per expert (decode: every expert in one
// tile of at most 32 rows, so that a 48-expert share is one item per
// resident workgroup), 1.25 times the mean above.  The streaming kernel's
// code ring is one stage ("wide": three workgroups per CU) for tiles of up to
// two row blocks whose experts mostly fill one block, or whose K is a single
// record (latency-bound items, where occupancy hides more than depth), and
// two stages otherwise.  The masked rule
// sizes tiles to expected_m itself: a tile of up to 32 rows keeps two
// streaming workgroups per CU (three at 16), which is worth more than the
// extra weight pass of an expert above expected_m (on the Zipf EP32 share,
// 1.0x tiles beat 1.3x / 1.25x ones by a quarter on both GEMMs).  K splits are added until the grid holds
// enough wavefronts to keep every CU streaming (shape-aware split-K gating),
// but never below 8 groups of K per split.

// K splits are whole 8-group records; every split keeps at least 2 records.
// The streaming kernel runs four wavefronts per workgroup and (by its
// registers) two workgroups per CU for tiles of up to 32 rows; K splits are
// added only while the items still fit in one round of resident workgroups
// (more items are dealt evenly over several rounds by the persistent grid,
// and need no split to fill the machine).  Every extra split also writes and
// reads one fp32 [rows, N] partial: keep that under a quarter of the weight
// stream.
static constexpr int64_t kResidentWorkgroups = 512;   // 256 CUs x 2

static int choose_split(int64_t tiles_est, int64_t rows_est, int NC, int stages, int N,
                        int64_t weight_bytes) {
    const int64_t wgs = std::max<int64_t>(tiles_est, 1) * ((NC + 3) / 4);
    const int64_t partial_bytes = std::max<int64_t>(rows_est, 1) * N * 8;
    int split = 1;
    while (wgs * (split + 1) <= kResidentWorkgroups && stages / (split + 1) >= 2 &&
           partial_bytes * (split + 1) <= weight_bytes / 4)
        ++split;
    return split;
}

// Contiguous layout: blocks of 128 rows when the (block, column pair) items
// of the large-M kernel fill the machine's compute units once, else blocks of
// 64 rows (twice the items).  Chord page, "Grouped SM90 kernels": BM128 on
// large grids spreads the dequant over more rows; small problems fall back to
// BM64 so that the M tiles fill the machine.
static constexpr int64_t kComputeUnits = 256;

static int contig_block_m(int NC, int64_t m) {
    const int64_t pairs = (NC + 1) / 2;
    return ceil_div(std::max<int64_t>(m, 1), 128) * pairs >= kComputeUnits ? 128 : 64;
}

// rows_cap: rows of the position-indexed output space when the caller's
// buffers are known (0 = unknown); with no rows_hint it sizes the split-K
// partials.
static w4a16_status plan_impl(const w4a16_desc* d, int layout, int rows_hint, int expected_m,
                              int tile_m_in, int64_t rows_cap, w4a16_plan* p) {
    const int E = d->E;
    const int stages = d->k_groups / 8;
    const int NC = d->N / d->chunk_n;
    int tile_m;
    int64_t tiles_est;
    if (layout == W4A16_LAYOUT_CONTIGUOUS) {
        if (d->profile != W4A16_PROFILE_PREFILL) {
            set_error("the contiguous layout runs on weights packed with the PREFILL profile");
            return W4A16_ERR_MODE_MISMATCH;
        }
        p->block_m = 128;
        p->tile_m = contig_block_m(NC, rows_hint);
        p->kernel = 2;
        p->split_k = 1;
        return W4A16_OK;
    }
    if (layout == W4A16_LAYOUT_MASKED) {
        if (expected_m <= 0) {
            set_error("expected_m must be a positive integer (got %d)", expected_m);
            return W4A16_ERR_INVALID_ARG;
        }
        const int64_t want = expected_m;
        const int step = d->profile == W4A16_PROFILE_PREFILL ? 32 : 16;
        tile_m = static_cast<int>(
            std::min<int64_t>(std::max<int64_t>(round_up(want, step), step), max_tile(d)));
        tiles_est = E;
    } else {
        if (tile_m_in > 0) {
            tile_m = tile_m_in;
        } else {
            const double tok_e = rows_hint > 0 ? static_cast<double>(rows_hint) / E : 16.0;
            if (d->profile == W4A16_PROFILE_PREFILL) {
                // one tile holds an expert's rows up to ~1.4x the mean
                // (Poisson-like tails), in 32-row steps; the kernel computes
                // only the 32-row blocks a tile fills
                tile_m = static_cast<int>(std::min<int64_t>(
                    std::max<int64_t>(round_up(static_cast<int64_t>(1.4 * tok_e + 0.999), 32), 32),
                    kLargeMaxTile));
            } else {
                // the streaming kernel's work per K group grows with the row
                // blocks of a tile, while an expert cut into two tiles streams
                // its weights twice
                const double want = tok_e <= 16.0 ? 2.0 * tok_e : 1.25 * tok_e;
                tile_m = static_cast<int>(std::min<int64_t>(
                    std::max<int64_t>(round_up(static_cast<int64_t>(want + 0.999), 16), 16),
                    kSmallMaxTile));
            }
        }
        tiles_est = rows_hint > 0 ? ceil_div(rows_hint, tile_m) + E / 2 : E;
    }
    p->block_m = 16;
    p->tile_m = tile_m;
    p->kernel = d->profile == W4A16_PROFILE_PREFILL ? 2 : 1;
    const int64_t rows_est = layout == W4A16_LAYOUT_MASKED ? static_cast<int64_t>(E) * expected_m
                             : rows_hint > 0                ? std::max<int64_t>(rows_hint, E)
                             : rows_cap > 0                 ? rows_cap
                                                            : E;
    const int64_t active = std::min<int64_t>(E, std::max<int64_t>(tiles_est, 1));
    const int64_t weight_bytes = active * static_cast<int64_t>(d->N) * d->K * 18 / 32;
    p->split_k = p->kernel == 2 ? 1 : choose_split(tiles_est, rows_est, NC, stages, d->N, weight_bytes);
    if (p->kernel == 2) {
        p->ring_groups = 0;
    } else {
        const double mean = layout == W4A16_LAYOUT_MASKED ? static_cast<double>(expected_m)
                            : rows_hint > 0 ? static_cast<double>(rows_hint) / E : 16.0;
        const bool wide = tile_m <= 16 || (tile_m <= 32 && (mean <= 16.0 || stages == 1));
        p->ring_groups = wide ? 8 : 16;
    }
    return W4A16_OK;
}

// ---- GEMM ------------------------------------------------------------------

// Workspace: [arrival counters | fp32 split-K partials | bf16 gate/up staging],
// each part 256-byte aligned.  The counters must be zero before the first
// call; every call leaves them zero.
struct Resolved {
    GemmArgs g;
    int kernel;              // 1 streaming, 2 large-M
    int mt;
    bool wide;               // streaming kernel: the 8-group code ring
    int split;
    int64_t rows_cap;        // rows of the position-indexed output space
    int64_t tiles_bound;     // tile indices a launch can visit
    uint64_t ws_counters;    // bytes of arrival counters (split > 1) or work-queue counters
    uint64_t ws_partial;     // bytes of fp32 partials (split > 1)
    uint64_t ws_y13;         // bytes of the bf16 gate/up staging (SiLU not fused)
    bool silu_separate;      // run the SiLU kernel on staged Y13
    uint64_t ws_total() const { return ws_counters + ws_partial + ws_y13; }
};

static uint64_t round256(uint64_t b) { return (b + 255) / 256 * 256; }

static w4a16_status resolve(const w4a16_gemm_args* a, Resolved* r) {
    W4A16_CHECK_ARG(a, "null GEMM arguments");
    w4a16_status st = check_desc(a->desc);
    if (st != W4A16_OK) return st;
    const w4a16_desc* d = a->desc;
    W4A16_CHECK_ARG(a->packed && aligned(a->packed, 256), "packed weights null or not 256-byte aligned");
    W4A16_CHECK_ARG(a->A && aligned(a->A, 16), "activations null or not 16-byte aligned");
    W4A16_CHECK_ARG(a->out && aligned(a->out, 16), "output null or not 16-byte aligned");
    W4A16_CHECK_ARG(a->epilogue == W4A16_EPI_STORE || a->epilogue == W4A16_EPI_SILU_MUL,
                    "unknown epilogue %d", a->epilogue);
    W4A16_CHECK_ARG((a->flags & ~W4A16_GEMM_F32_OUT) == 0, "unknown GEMM flags 0x%x", a->flags);
    const bool f32_out = (a->flags & W4A16_GEMM_F32_OUT) != 0;
    const bool interleaved = (d->flags & W4A16_PACK_GATE_UP_INTERLEAVE) != 0;
    if (a->epilogue == W4A16_EPI_STORE && interleaved) {
        set_error("weight packed with gate/up interleave used with a plain store epilogue");
        return W4A16_ERR_MODE_MISMATCH;
    }
    W4A16_CHECK_ARG(!interleaved || d->chunk_n == 64 || d->chunk_n == 128,
                    "gate/up interleave needs 64- or 128-column chunks");
    W4A16_CHECK_ARG(!(f32_out && a->epilogue != W4A16_EPI_STORE), "F32_OUT needs EPI_STORE");
    W4A16_CHECK_ARG(a->epilogue != W4A16_EPI_SILU_MUL || d->N % 16 == 0,
                    "SiLU epilogue needs N %% 16 == 0");

    GemmArgs& g = r->g;
    g = GemmArgs{};
    g.A = a->A;
    g.packed = static_cast<const uint32_t*>(a->packed);
    g.stage_words = static_cast<int64_t>(d->stage_bytes / 4);
    g.chunk_words = static_cast<int64_t>(d->chunk_bytes / 4);
    g.N = d->N;
    g.K = d->K;
    g.CW = d->chunk_n;
    g.NC = d->N / d->chunk_n;
    g.KS = d->K / 32;
    g.KSP = d->k_groups;
    g.E = d->E;
    W4A16_CHECK_ARG(a->A_rows >= 1, "A_rows must be positive");
    if (static_cast<uint64_t>(a->A_rows) * static_cast<uint64_t>(d->K) * 2 > 0xFFFFFFFFull) {
        set_error("activations of %lld x %d bf16 exceed the 4 GiB a kernel addresses",
                  static_cast<long long>(a->A_rows), d->K);
        return W4A16_ERR_UNSUPPORTED;
    }
    g.A_rows = a->A_rows;

    w4a16_plan plan;
    if (a->layout == W4A16_LAYOUT_INDEXED) {
        W4A16_CHECK_ARG(a->sorted_ids && a->num_tokens_padded, "indexed layout needs sorted_ids and num_tokens_padded");
        W4A16_CHECK_ARG(a->sorted_cap >= 1, "sorted_cap must be positive");
        W4A16_CHECK_ARG(a->num_slots >= 1, "num_slots (T * top_k) must be positive");
        W4A16_CHECK_ARG(a->arow >= W4A16_AROW_TOKEN && a->arow <= W4A16_AROW_POSITION, "bad arow %d", a->arow);
        W4A16_CHECK_ARG(a->orow == W4A16_OROW_POSITION || a->orow == W4A16_OROW_SLOT, "bad orow %d", a->orow);
        W4A16_CHECK_ARG(a->arow != W4A16_AROW_TOKEN || a->top_k >= 1, "AROW_TOKEN needs top_k >= 1");
        W4A16_CHECK_ARG(a->split_k >= 0, "split_k must be >= 0");
        int tile_m;
        if (a->tiles) {
            W4A16_CHECK_ARG(a->tile_count && aligned(a->tiles, 16), "tile table needs tile_count and 16-byte alignment");
            W4A16_CHECK_ARG(a->tiles_cap >= 1, "tiles_cap must be positive");
            W4A16_CHECK_ARG(a->tile_m >= 16 && a->tile_m % 16 == 0, "tile_m must be a positive multiple of 16");
            if (a->tile_m > max_tile(d)) {
                set_error("tile_m %d exceeds the %d this weight profile supports", a->tile_m, max_tile(d));
                return W4A16_ERR_UNSUPPORTED;
            }
            tile_m = a->tile_m;
        } else {
            W4A16_CHECK_ARG(a->expert_ids && a->blocks_cap >= 1, "indexed layout without tiles needs expert_ids");
            W4A16_CHECK_ARG(a->block_m >= 16 && a->block_m % 16 == 0, "block_m must be a positive multiple of 16");
            if (a->block_m > max_tile(d)) {
                set_error("block_m %d exceeds the %d this weight profile supports", a->block_m, max_tile(d));
                return W4A16_ERR_UNSUPPORTED;
            }
            tile_m = a->block_m;
        }
        st = plan_impl(d, W4A16_LAYOUT_INDEXED, a->rows_hint, 0, tile_m, a->sorted_cap, &plan);
        if (st != W4A16_OK) return st;
        int split = a->split_k > 0 ? a->split_k : plan.split_k;
        // the large-M kernel runs unsplit: split_k applies to the streaming kernel
        if (a->orow == W4A16_OROW_SLOT || f32_out || plan.kernel == 2) split = 1;
        split = std::max(1, std::min(split, g.KSP / 8));
        r->kernel = plan.kernel;
        {
            const int64_t need_a = a->arow == W4A16_AROW_POSITION ? a->sorted_cap
                                   : a->arow == W4A16_AROW_SLOT   ? a->num_slots
                                                                  : ceil_div(a->num_slots, a->top_k);
            if (a->A_rows < need_a) {
                set_error("activations have %lld rows, this row mode needs %lld",
                          static_cast<long long>(a->A_rows), static_cast<long long>(need_a));
                return W4A16_ERR_CAPACITY;
            }
        }
        g.sorted_cap = a->sorted_cap;
        g.tile_src = a->tiles ? TILE_TABLE : TILE_BLOCKS;
        g.arow = a->arow;
        g.orow = a->orow;
        g.top_k = a->top_k;
        g.num_slots = a->num_slots;
        g.sorted_ids = a->sorted_ids;
        g.expert_ids = a->expert_ids;
        g.ntp = a->num_tokens_padded;
        g.tiles = a->tiles;
        g.tile_count = a->tile_count;
        g.block_m = a->block_m;
        g.tile_m = tile_m;
        if (a->tiles) {
            int64_t want = a->rows_hint > 0 ? ceil_div(a->rows_hint, tile_m) + d->E : a->tiles_cap;
            g.grid_tiles = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(a->tiles_cap, want)));
        } else {
            g.grid_tiles = a->blocks_cap;
        }
        r->tiles_bound = a->tiles ? a->tiles_cap : a->blocks_cap;
        r->mt = tile_m / 16;
        r->wide = plan.ring_groups == 8;
        r->split = split;
        r->rows_cap = a->sorted_cap;
        const int64_t need_rows = a->orow == W4A16_OROW_SLOT ? a->num_slots : a->sorted_cap;
        const int64_t out_w = a->epilogue == W4A16_EPI_SILU_MUL ? d->N / 2 : d->N;
        (void)out_w;
        if (a->out_rows < need_rows) {
            set_error("output has %lld rows, needs %lld", static_cast<long long>(a->out_rows),
                      static_cast<long long>(need_rows));
            return W4A16_ERR_CAPACITY;
        }
    } else if (a->layout == W4A16_LAYOUT_MASKED) {
        W4A16_CHECK_ARG(a->masked_m, "masked layout needs masked_m");
        W4A16_CHECK_ARG(a->max_m >= 1, "max_m must be positive");
        if (a->expected_m <= 0) {
            set_error("expected_m must be a positive integer (got %d)", a->expected_m);
            return W4A16_ERR_INVALID_ARG;
        }
        if (a->split_k != 0) {
            set_error("the grouped masked dispatch chooses its own schedule: split_k override refused");
            return W4A16_ERR_MODE_MISMATCH;
        }
        st = plan_impl(d, W4A16_LAYOUT_MASKED, 0, a->expected_m, 0,
                       static_cast<int64_t>(d->E) * a->max_m, &plan);
        if (st != W4A16_OK) return st;
        const int64_t rows = static_cast<int64_t>(d->E) * a->max_m;
        if (a->A_rows < rows) {
            set_error("masked activations have %lld rows, need E*max_m = %lld",
                      static_cast<long long>(a->A_rows), static_cast<long long>(rows));
            return W4A16_ERR_CAPACITY;
        }
        if (a->out_rows < rows) {
            set_error("masked output has %lld rows, needs %lld", static_cast<long long>(a->out_rows),
                      static_cast<long long>(rows));
            return W4A16_ERR_CAPACITY;
        }
        g.tile_src = TILE_MASKED;
        g.arow = W4A16_AROW_POSITION;
        g.orow = W4A16_OROW_POSITION;
        g.masked_m = a->masked_m;
        g.max_m = a->max_m;
        g.tile_m = plan.tile_m;
        g.chunks_per_expert = static_cast<int>(ceil_div(a->max_m, plan.tile_m));
        g.grid_tiles_total = d->E * g.chunks_per_expert;
        g.grid_tiles = g.grid_tiles_total;
        int split = f32_out || plan.kernel == 2 ? 1 : plan.split_k;
        r->kernel = plan.kernel;
        r->tiles_bound = g.grid_tiles_total;
        r->mt = plan.tile_m / 16;
        r->wide = plan.ring_groups == 8;
        r->split = std::max(1, std::min(split, g.KSP / 8));
        r->rows_cap = rows;
    } else if (a->layout == W4A16_LAYOUT_CONTIGUOUS) {
        W4A16_CHECK_ARG(a->m_indices, "contiguous layout needs m_indices");
        if (a->split_k != 0) {
            set_error("the grouped contiguous dispatch chooses its own schedule: split_k override refused");
            return W4A16_ERR_MODE_MISMATCH;
        }
        const int64_t m = a->A_rows;
        W4A16_CHECK_ARG(m < (1LL << 31), "contiguous layout: m must stay below 2^31 rows");
        st = plan_impl(d, W4A16_LAYOUT_CONTIGUOUS, static_cast<int>(m), 0, 0, m, &plan);
        if (st != W4A16_OK) return st;
        if (a->out_rows < m) {
            set_error("contiguous output has %lld rows, needs m = %lld",
                      static_cast<long long>(a->out_rows), static_cast<long long>(m));
            return W4A16_ERR_CAPACITY;
        }
        g.tile_src = TILE_CONTIG;
        g.arow = W4A16_AROW_POSITION;
        g.orow = W4A16_OROW_POSITION;
        g.m_indices = a->m_indices;
        g.tile_m = plan.tile_m;
        g.grid_tiles_total = static_cast<int>(ceil_div(m, plan.tile_m));
        g.grid_tiles = g.grid_tiles_total;
        r->kernel = 2;
        r->tiles_bound = g.grid_tiles_total;
        r->mt = plan.tile_m / 16;
        r->split = 1;
        r->rows_cap = m;
    } else {
        W4A16_CHECK_ARG(false, "unknown layout %d", a->layout);
    }
    // a split's fp32 partial [rows_cap, N] is addressed with 32-bit byte
    // offsets: below 4 GiB or no split (an explicit override is refused)
    if (r->split > 1 && static_cast<uint64_t>(r->rows_cap) * d->N * 4 >= 0xFFFFFFFFull) {
        if (a->layout == W4A16_LAYOUT_INDEXED && a->split_k > 1) {
            set_error("split_k %d: a split's fp32 partial of %lld x %d exceeds 4 GiB", a->split_k,
                      static_cast<long long>(r->rows_cap), d->N);
            return W4A16_ERR_UNSUPPORTED;
        }
        r->split = 1;
    }
    // A8W4: MXFP8 activations on a weight laid out for them, and only there
    const bool a8 = (d->flags & W4A16_PACK_MXFP8_ACT) != 0;
    if (a8 != (a->A_scales != nullptr)) {
        set_error(a8 ? "a weight packed for MXFP8 activations needs A_scales"
                     : "A_scales given for a weight not packed for MXFP8 activations");
        return W4A16_ERR_MODE_MISMATCH;
    }
    if (a8) {
        if (a->layout != W4A16_LAYOUT_INDEXED || a->comb_out) {
            set_error("A8W4 runs the indexed layout without the fused combine");
            return W4A16_ERR_UNSUPPORTED;
        }
        r->split = 1;
    }
    // fused top-k combine in the epilogue (the down GEMM of the indexed path)
    if (a->comb_out) {
        W4A16_CHECK_ARG(a->layout == W4A16_LAYOUT_INDEXED && a->tiles,
                        "the fused combine needs the indexed layout with a tile table");
        if (r->kernel != 1) {
            set_error("the fused combine runs in the streaming kernel (DECODE profile) only");
            return W4A16_ERR_UNSUPPORTED;
        }
        W4A16_CHECK_ARG(a->orow == W4A16_OROW_POSITION, "the fused combine needs OROW_POSITION");
        W4A16_CHECK_ARG(a->epilogue == W4A16_EPI_STORE && !f32_out,
                        "the fused combine needs EPI_STORE with bf16 output");
        W4A16_CHECK_ARG(a->comb_row_of && a->comb_weights && aligned(a->comb_out, 16),
                        "the fused combine needs row_of, weights and a 16-byte aligned output");
        W4A16_CHECK_ARG(a->top_k >= 1 && a->comb_T >= 0 &&
                            static_cast<int64_t>(a->comb_T) * a->top_k == a->num_slots,
                        "the fused combine needs comb_T * top_k == num_slots");
        if (static_cast<uint64_t>(a->sorted_cap) * d->N * 2 >= 0xFFFFFFFFull) {
            set_error("fused combine: rows of %d x %d bf16 exceed the 4 GiB a kernel addresses",
                      a->sorted_cap, d->N);
            return W4A16_ERR_UNSUPPORTED;
        }
    }
    g.split_k = r->split;
    g.tiles_cap = static_cast<int>(std::min<int64_t>(r->tiles_bound, 0x7FFFFFFF));
    g.unpack_mask = 0x000F000Fu;
    g.unpack_bits = 0x43004300u;
    g.nib_mask = 0x0F0F0F0Fu;
    g.fp4 = (d->flags & W4A16_PACK_MXFP4) ? 1 : 0;   // DECODE profile only (checked at prepack)
    g.a8 = a8 ? 1 : 0;
    g.A_scales = a->A_scales;
    const bool split = r->split > 1;
    r->silu_separate = a->epilogue == W4A16_EPI_SILU_MUL && !interleaved;
    const int64_t gx = (g.NC + 3) / 4;
    // split-K arrival counters (one per tile and group of four chunks) or the
    // PREFILL kernel's work-queue counters (nine ints); then the fused
    // combine's arrival counters (one per token and 256 columns)
    const uint64_t ctr = split ? round256(static_cast<uint64_t>(r->tiles_bound) * gx * 4)
                         : r->kernel == 2 ? 256 : 0;
    const int comb_groups = (d->N + 255) / 256;
    const uint64_t comb =
        a->comb_out ? round256(static_cast<uint64_t>(a->comb_T) * comb_groups * 4) : 0;
    r->ws_counters = ctr + comb;
    r->ws_partial = split ? round256(static_cast<uint64_t>(r->split) * r->rows_cap * d->N * 4) : 0;
    r->ws_y13 = r->silu_separate ? round256(static_cast<uint64_t>(r->rows_cap) * d->N * 2) : 0;
    g.ws_stride = r->rows_cap * d->N;
    char* ws = static_cast<char*>(a->workspace);
    g.counters = ctr && ws ? reinterpret_cast<int32_t*>(ws) : nullptr;
    if (a->comb_out) {
        g.comb_out = a->comb_out;
        g.comb_row_of = a->comb_row_of;
        g.comb_w = a->comb_weights;
        g.comb_T = a->comb_T;
        g.comb_groups = comb_groups;
        g.comb_counters = ws ? reinterpret_cast<int32_t*>(ws + ctr) : nullptr;
    }
    g.partials = split && ws ? reinterpret_cast<float*>(ws + r->ws_counters) : nullptr;
    if (a->epilogue == W4A16_EPI_SILU_MUL && interleaved) {
        g.out_kind = OUT_SILU;
        g.out = a->out;
    } else if (r->silu_separate) {
        g.out_kind = OUT_BF16;
        g.out = ws ? ws + r->ws_counters + r->ws_partial : nullptr;
    } else {
        g.out_kind = f32_out ? OUT_F32 : OUT_BF16;
        g.out = a->out;
    }
    return W4A16_OK;
}

// Launches of one resolved GEMM call; the workspace pointers inside r.g are
// already set.
static w4a16_status run_resolved(const w4a16_gemm_args* args, const Resolved& r, hipStream_t s) {
    if (r.kernel == 2)
        launch_gemm_large(r.g, s);
    else if (r.g.a8)
        launch_gemm_mx(r.g, r.mt, s);
    else
        launch_gemm_small(r.g, r.mt, r.wide, s);
    w4a16_status st = check_launch("w4a16 gemm");
    if (st != W4A16_OK) return st;
    if (r.silu_separate) {
        // the GEMM staged Y13 in the workspace at the rows it would have
        // written (positions, or slots with OROW_SLOT); the activation visits
        // the same rows and skips padding, so it writes only rows the caller's
        // output holds
        const bool masked = args->layout == W4A16_LAYOUT_MASKED;
        const bool contig = args->layout == W4A16_LAYOUT_CONTIGUOUS;
        if (contig)   // rows whose index names an expert
            launch_silu_mul(static_cast<const uint16_t*>(r.g.out), r.rows_cap, nullptr,
                            args->desc->N / 2, nullptr, 1, args->m_indices, args->desc->E, false,
                            static_cast<uint16_t*>(args->out), s);
        else
            launch_silu_mul(static_cast<const uint16_t*>(r.g.out), r.rows_cap,
                            masked ? nullptr : args->num_tokens_padded, args->desc->N / 2,
                            masked ? args->masked_m : nullptr, args->max_m,
                            masked ? nullptr : args->sorted_ids, args->num_slots,
                            !masked && args->orow == W4A16_OROW_SLOT,
                            static_cast<uint16_t*>(args->out), s);
        st = check_launch("silu_mul");
    }
    return st;
}

// ---- static device scratch of the allocation-free GEMM entry point ----------
//
// One array per GPU, held from module load until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed to
// kernels.
constexpr uint64_t kScratchBytes = 32ull << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static w4a16_status scratch_for_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error("no current HIP device below %d for the static scratch", kMaxDevices);
        return W4A16_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error("hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                      hipGetErrorString(e));
            return W4A16_ERR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return W4A16_OK;
}

}  // namespace w4a16

using namespace w4a16;

extern "C" {

const char* w4a16_last_error(void) { return g_err; }

int32_t w4a16_version(void) { return 100; }

w4a16_status w4a16_plan_gemm(const w4a16_desc* desc, int32_t layout, int32_t rows_hint,
                             int32_t expected_m, int32_t tile_m, w4a16_plan* plan) {
    clear_error();
    W4A16_CHECK_ARG(plan, "null plan pointer");
    w4a16_status st = check_desc(desc);
    if (st != W4A16_OK) return st;
    W4A16_CHECK_ARG(layout == W4A16_LAYOUT_INDEXED || layout == W4A16_LAYOUT_MASKED ||
                        layout == W4A16_LAYOUT_CONTIGUOUS,
                    "unknown layout %d", layout);
    W4A16_CHECK_ARG(tile_m == 0 || (tile_m >= 16 && tile_m % 16 == 0 && tile_m <= max_tile(desc)),
                    "tile_m must be 0 or a multiple of 16 up to %d for this profile", max_tile(desc));
    return plan_impl(desc, layout, rows_hint, expected_m, tile_m, 0, plan);
}

w4a16_status w4a16_moe_align_capacity(int32_t T, int32_t top_k, int32_t E_local, int32_t block_m,
                                      int32_t tile_m, int32_t* sorted_cap, int32_t* blocks_cap,
                                      int32_t* tiles_cap) {
    clear_error();
    W4A16_CHECK_ARG(sorted_cap && blocks_cap && tiles_cap, "null output pointer");
    W4A16_CHECK_ARG(T >= 0 && top_k >= 1 && E_local >= 1 && E_local <= 1024, "bad T/top_k/E_local");
    W4A16_CHECK_ARG(block_m >= 1 && block_m <= 256, "block_m must be in [1, 256]");
    W4A16_CHECK_ARG(tile_m == 0 || (tile_m >= 16 && tile_m <= 256 && tile_m % 16 == 0),
                    "tile_m must be 0 or a multiple of 16 up to 256");
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    int64_t sc = round_up(slots + static_cast<int64_t>(E_local) * (block_m - 1), block_m);
    sc = std::max<int64_t>(sc, block_m);
    W4A16_CHECK_ARG(sc < (1LL << 31), "routing too large");
    *sorted_cap = static_cast<int32_t>(sc);
    *blocks_cap = static_cast<int32_t>(sc / block_m);
    *tiles_cap = tile_m > 0 ? static_cast<int32_t>(ceil_div(slots, tile_m) + E_local) : 0;
    return W4A16_OK;
}

// The align entry points: routing ids from topk_ids, or (logits != NULL)
// from the router top-k of the logits, written to ids_out / w_out first.
static w4a16_status align_entry(const int32_t* topk_ids, int32_t T, int32_t top_k,
                                int32_t E_global, const int32_t* expert_map, int32_t E_local,
                                int32_t block_m, const w4a16_routing* routing, uint32_t flags,
                                void* stream, const float* logits, int32_t* ids_out,
                                float* w_out) {
    W4A16_CHECK_ARG(routing, "null routing buffers");
    W4A16_CHECK_ARG(T >= 0 && top_k >= 1, "bad T=%d top_k=%d", T, top_k);
    W4A16_CHECK_ARG(T == 0 || topk_ids || logits, "null topk_ids");
    W4A16_CHECK_ARG(E_global >= 1, "E_global must be positive");
    W4A16_CHECK_ARG(E_local >= 1 && E_local <= 1024, "E_local must be in [1, 1024]");
    W4A16_CHECK_ARG(block_m >= 1 && block_m <= 256, "block_m must be in [1, 256]");
    W4A16_CHECK_ARG((flags & ~W4A16_ALIGN_VALIDATE) == 0, "unknown align flags 0x%x", flags);
    const w4a16_routing& r = *routing;
    W4A16_CHECK_ARG(r.sorted_ids && r.expert_ids && r.num_tokens_padded, "routing needs sorted_ids, expert_ids, num_tokens_padded");
    int32_t sc, bc, tc;
    w4a16_status st = w4a16_moe_align_capacity(T, top_k, E_local, block_m,
                                               r.tiles ? r.tile_m : 0, &sc, &bc, &tc);
    if (st != W4A16_OK) return st;
    if (r.sorted_cap < sc || r.blocks_cap < bc) {
        set_error("routing capacity too small: sorted_cap %d < %d or blocks_cap %d < %d",
                  r.sorted_cap, sc, r.blocks_cap, bc);
        return W4A16_ERR_CAPACITY;
    }
    if (r.tiles) {
        W4A16_CHECK_ARG(r.tile_count && aligned(r.tiles, 16), "tile table needs tile_count and 16-byte alignment");
        if (r.tiles_cap < tc) {
            set_error("tiles_cap %d < %d", r.tiles_cap, tc);
            return W4A16_ERR_CAPACITY;
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    AlignArgs a{};
    a.topk_ids = topk_ids;
    a.T = T;
    a.top_k = top_k;
    a.E_global = E_global;
    a.E_local = E_local;
    a.block_m = block_m;
    a.expert_map = expert_map;
    a.r = r;
    a.logits = logits;
    a.ids_out = ids_out;
    a.weights_out = w_out;
    int32_t* flag = nullptr;
    if (flags & W4A16_ALIGN_VALIDATE) {
        if (hipGetSymbolAddress(reinterpret_cast<void**>(&flag), HIP_SYMBOL(g_routing_errors)) != hipSuccess) {
            set_error("cannot locate the routing error counter");
            return W4A16_ERR_HIP;
        }
        int32_t zero = 0;
        if (hipMemcpyAsync(flag, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess) {
            set_error("cannot reset the routing error counter");
            return W4A16_ERR_HIP;
        }
    }
    a.err_flag = flag;
    launch_align(a, s);
    st = check_launch("moe_align");
    if (st != W4A16_OK) return st;
    if (flag) {
        int32_t nbad = 0;
        if (hipMemcpyAsync(&nbad, flag, sizeof(nbad), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess) {
            set_error("routing validation read-back failed");
            return W4A16_ERR_HIP;
        }
        if (nbad) {
            set_error("%d routed slot(s) name an expert id out of range", nbad);
            return W4A16_ERR_ROUTING;
        }
    }
    return W4A16_OK;
}

w4a16_status w4a16_moe_align(const int32_t* topk_ids, int32_t T, int32_t top_k, int32_t E_global,
                             const int32_t* expert_map, int32_t E_local, int32_t block_m,
                             const w4a16_routing* routing, uint32_t flags, void* stream) {
    clear_error();
    return align_entry(topk_ids, T, top_k, E_global, expert_map, E_local, block_m, routing, flags,
                       stream, nullptr, nullptr, nullptr);
}

static w4a16_status check_router(const float* logits, int32_t T, int32_t E_global, int32_t top_k,
                                 const int32_t* topk_ids, const float* topk_weights) {
    W4A16_CHECK_ARG(T >= 0, "bad T=%d", T);
    W4A16_CHECK_ARG(E_global >= 1 && E_global <= kRouterMaxExperts,
                    "router: E_global must be in [1, %d]", kRouterMaxExperts);
    W4A16_CHECK_ARG(top_k >= 1 && top_k <= kRouterMaxTopK && top_k <= E_global,
                    "router: top_k must be in [1, min(%d, E_global)]", kRouterMaxTopK);
    W4A16_CHECK_ARG(T == 0 || (logits && topk_ids && topk_weights), "router: null buffer");
    return W4A16_OK;
}

w4a16_status w4a16_moe_router_topk(const float* logits, int32_t T, int32_t E_global, int32_t top_k,
                                   int32_t* topk_ids, float* topk_weights, void* stream) {
    clear_error();
    w4a16_status st = check_router(logits, T, E_global, top_k, topk_ids, topk_weights);
    if (st != W4A16_OK) return st;
    launch_router_topk(logits, T, E_global, top_k, topk_ids, topk_weights,
                       static_cast<hipStream_t>(stream));
    return check_launch("router_topk");
}

w4a16_status w4a16_moe_route_align(const float* logits, int32_t T, int32_t E_global,
                                   int32_t top_k, const int32_t* expert_map, int32_t E_local,
                                   int32_t block_m, const w4a16_routing* routing,
                                   int32_t* topk_ids, float* topk_weights, uint32_t flags,
                                   void* stream) {
    clear_error();
    w4a16_status st = check_router(logits, T, E_global, top_k, topk_ids, topk_weights);
    if (st != W4A16_OK) return st;
    return align_entry(topk_ids, T, top_k, E_global, expert_map, E_local, block_m, routing, flags,
                       stream, T > 0 ? logits : nullptr, topk_ids, topk_weights);
}

w4a16_status w4a16_moe_indexed_to_masked(const uint16_t* X, int64_t X_rows, int32_t H,
                                         const int32_t* topk_ids, int32_t T, int32_t top_k,
                                         int32_t E_global, const int32_t* expert_map,
                                         int32_t E_local, int32_t max_m,
                                         const w4a16_routing* scratch, uint16_t* a3,
                                         int32_t* masked_m, int32_t* row_of, int32_t* dropped,
                                         void* stream) {
    clear_error();
    W4A16_CHECK_ARG(scratch, "null routing scratch");
    W4A16_CHECK_ARG(T >= 0 && top_k >= 1 && E_local >= 1 && max_m >= 1, "bad T/top_k/E_local/max_m");
    W4A16_CHECK_ARG(H >= 8 && H % 8 == 0, "H must be a positive multiple of 8");
    W4A16_CHECK_ARG(masked_m && (T == 0 || (X && topk_ids && a3 && row_of)), "null buffer");
    W4A16_CHECK_ARG(T == 0 || (aligned(X, 16) && aligned(a3, 16)), "X and a3 must be 16-byte aligned");
    W4A16_CHECK_ARG(X_rows >= T, "X has %lld rows, needs T = %d", static_cast<long long>(X_rows), T);
    W4A16_CHECK_ARG(scratch->row_of && scratch->expert_offsets,
                    "the routing scratch needs row_of and expert_offsets");
    w4a16_routing r = *scratch;     // the sort without tiles, padding block 1
    r.tiles = nullptr;
    r.tile_count = nullptr;
    r.tiles_cap = 0;
    w4a16_status st = align_entry(topk_ids, T, top_k, E_global, expert_map, E_local, 1, &r, 0,
                                  stream, nullptr, nullptr, nullptr);
    if (st != W4A16_OK) return st;
    MaskedPlaceArgs m{};
    m.X = X;
    m.H = H;
    m.top_k = top_k;
    m.num_slots = T * top_k;
    m.sorted_ids = r.sorted_ids;
    m.expert_ids = r.expert_ids;
    m.ntp = r.num_tokens_padded;
    m.sorted_cap = r.sorted_cap;
    m.offsets = r.expert_offsets;
    m.row_of = r.row_of;
    m.E = E_local;
    m.max_m = max_m;
    m.a3 = a3;
    m.masked_m = masked_m;
    m.row_of_masked = row_of;
    m.dropped = dropped;
    launch_to_masked(m, static_cast<hipStream_t>(stream));
    return check_launch("indexed_to_masked");
}

w4a16_status w4a16_gemm_workspace_bytes(const w4a16_gemm_args* args, uint64_t* bytes) {
    clear_error();
    W4A16_CHECK_ARG(bytes, "null bytes pointer");
    Resolved r;
    w4a16_status st = resolve(args, &r);
    if (st != W4A16_OK) return st;
    *bytes = r.ws_total();
    return W4A16_OK;
}

w4a16_status w4a16_moe_w4a16_gemm(const w4a16_gemm_args* args, void* stream) {
    clear_error();
    Resolved r;
    w4a16_status st = resolve(args, &r);
    if (st != W4A16_OK) return st;
    const uint64_t need = r.ws_total();
    if (need > 0) {
        if (!args->workspace || args->workspace_bytes < need || !aligned(args->workspace, 256)) {
            set_error("workspace too small or not 256-byte aligned: %llu bytes needed",
                      static_cast<unsigned long long>(need));
            return W4A16_ERR_CAPACITY;
        }
    }
    return run_resolved(args, r, static_cast<hipStream_t>(stream));
}

w4a16_status w4a16_moe_w4a16_gemm_noalloc(const w4a16_gemm_args* args, void* stream) {
    clear_error();
    W4A16_CHECK_ARG(args, "null GEMM arguments");
    // size the call with no workspace first: a call that needs more than the
    // static scratch is refused before anything touches the device
    w4a16_gemm_args a = *args;
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    Resolved r;
    w4a16_status st = resolve(&a, &r);
    if (st != W4A16_OK) return st;
    const uint64_t need = r.ws_total();
    if (need > kScratchBytes) {
        set_error("this call needs %llu bytes of scratch; the allocation-free entry point "
                  "holds %llu (use w4a16_moe_w4a16_gemm with a workspace)",
                  static_cast<unsigned long long>(need),
                  static_cast<unsigned long long>(kScratchBytes));
        return W4A16_ERR_CAPACITY;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (need > 0) {
        void* ptr = nullptr;
        st = scratch_for_current_device(&ptr);
        if (st != W4A16_OK) return st;
        a.workspace = ptr;
        a.workspace_bytes = kScratchBytes;
        st = resolve(&a, &r);
        if (st != W4A16_OK) return st;
        // the array keeps the previous call's bytes: the counters at its
        // start must read zero when the kernels begin
        if (r.ws_counters > 0) {
            launch_zero(ptr, r.ws_counters, s);
            st = check_launch("scratch counters");
            if (st != W4A16_OK) return st;
        }
    }
    return run_resolved(&a, r, s);
}

w4a16_status w4a16_moe_silu_mul(const uint16_t* y13, int64_t rows, const int32_t* rows_dev,
                                int32_t I, uint16_t* z, void* stream) {
    clear_error();
    W4A16_CHECK_ARG(y13 && z && aligned(y13, 16) && aligned(z, 16), "null or misaligned buffers");
    W4A16_CHECK_ARG(rows >= 0 && I >= 8 && I % 8 == 0, "rows must be >= 0 and I a multiple of 8");
    launch_silu_mul(y13, rows, rows_dev, I, nullptr, 1, nullptr, 0, false, z,
                    static_cast<hipStream_t>(stream));
    return check_launch("silu_mul");
}

w4a16_status w4a16_quantize_mxfp8(const uint16_t* x, int64_t rows, const int32_t* rows_dev,
                                  int32_t K, uint8_t* codes, uint8_t* scales, void* stream) {
    clear_error();
    W4A16_CHECK_ARG(x && codes && scales && aligned(x, 16) && aligned(codes, 16),
                    "null or misaligned buffers");
    W4A16_CHECK_ARG(rows >= 0 && K >= 32 && K % 32 == 0,
                    "rows must be >= 0 and K a positive multiple of 32");
    if (rows == 0) return W4A16_OK;
    launch_quant_mxfp8(x, rows, rows_dev, K, codes, scales, static_cast<hipStream_t>(stream));
    return check_launch("quantize_mxfp8");
}

w4a16_status w4a16_moe_combine(const uint16_t* y, int64_t y_rows, int32_t H, const int32_t* row_of,
                               const float* topk_weights, int32_t T, int32_t top_k, uint16_t* out,
                               void* stream) {
    clear_error();
    W4A16_CHECK_ARG(T >= 0 && top_k >= 1 && y_rows >= 1, "bad T/top_k/y_rows");
    W4A16_CHECK_ARG(H >= 8 && H % 8 == 0, "H must be a positive multiple of 8");
    W4A16_CHECK_ARG(y && out && row_of && topk_weights, "null buffer");
    W4A16_CHECK_ARG(aligned(y, 16) && aligned(out, 16), "y and out must be 16-byte aligned");
    if (T == 0) return W4A16_OK;
    launch_combine(y, y_rows, H, row_of, topk_weights, T, top_k, out, static_cast<hipStream_t>(stream));
    return check_launch("combine");
}

}  // extern "C"
