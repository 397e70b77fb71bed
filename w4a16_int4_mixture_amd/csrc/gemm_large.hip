// Grouped W4A16 GEMM for many routed rows per expert (tiles of up to 256
// rows): an MFMA-bound kernel for CDNA4.
//
//   out[p, n] = sum_c A[row(p), c] * bf16((q[e,n,c] - 8) * s[e,n,c/32])
//
// Chord page, "H200 prefill and TP8": with many routed rows per expert the
// path is bound by the matrix units and by the dequant; the dequant (subtract,
// then scale, rounded to BF16) is amortised over the rows of a tile, the main
// loop keeps the next weights loading and dequantising while the current MMAs
// run, and block M follows the routed rows per expert.
//
// CDNA4 design.
//   * Persistent: one workgroup of four wavefronts per CU walks work items
//     (row tile, pair of 128-column chunks).  When there are more items than
//     workgroups, items come from per-XCD counters, largest tile first, each
//     row tile dealt to one XCD (workgroup w runs on XCD w % 8), so that the
//     activation rows of a tile are fetched into one L2 and reused there by
//     all its column pairs.
//   * v_mfma_f32_32x32x16_bf16.  Wavefront w works on chunk 2 * pair + w / 2
//     and, inside it, on the 32-column blocks h and h + 2 (h = w % 2), for
//     every row of the tile: with the gate/up interleave those are a gate
//     block and its up block, so SiLU * gate runs on the accumulators.  Up to
//     8 row blocks x 2 column blocks x 16 fp32 accumulators per lane (256) in
//     the accumulation registers.
//   * Activations go from HBM/L2 straight into LDS (buffer loads with the LDS
//     bit: no staging registers), whole 128-byte lines of eight rows per
//     load, one 32 KB slot per stage of two K groups (256 rows x 64 K, rows
//     contiguous, 16-byte chunks XOR-swizzled against LDS bank conflicts),
//     four slots (stages s .. s + 3); one barrier per stage.
//   * Weights: per group each lane loads 16 bytes of codes (its two blocks,
//     two K steps) into a register ring four stages ahead, and per record
//     (8 groups) 32 bytes of scales; it dequantises the next group while the
//     MFMAs of the current group run: a code byte becomes fp32
//     (v_cvt_f32_ubyte), then (q - 8) * s in one exact FMA, then bf16 (one
//     rounding).
//   * The row count of a tile picks one of eight code paths (32-row blocks);
//     all waves of a workgroup take the same path.

#include "device_common.h"
#include "internal.h"

namespace w4a16 {

namespace {

using namespace dev;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kRecWords = 4608;        // words per 8-group record (codes, then scales)
constexpr uint32_t kSlot = 32 * 1024;  // LDS bytes of one stage: 256 rows x 64 K x 2 bytes

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// The codes of one K group for one lane: (block h, step 0), (h, 1),
// (h + 2, 0), (h + 2, 1).
struct WGroup {
    u32x4 w;
};

__device__ inline uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// B operand of one (block, K step): the word's eight codes (nibble o = K
// offset o) dequantised with the scale s (c = -8 s).  With nib = 0x0F0F0F0F
// the bytes of w & nib hold offsets 0, 2, 4, 6 and those of (w >> 4) & nib
// offsets 1, 3, 5, 7; each byte converts with one v_cvt_f32_ubyte (the mask
// comes from a kernel argument so that the compiler cannot fold it into a
// per-nibble bit-field extract, which would cost one more op per code).
__device__ inline bf16x8 dequant_word(uint32_t w, uint32_t nib, float s, float c) {
    const uint32_t m0 = w & nib;
    const uint32_t m1 = (w >> 4) & nib;
    u32x4 d;
    d.x = pk_bf16(__builtin_fmaf(static_cast<float>(m0 & 0xFFu), s, c),
                  __builtin_fmaf(static_cast<float>(m1 & 0xFFu), s, c));
    d.y = pk_bf16(__builtin_fmaf(static_cast<float>((m0 >> 8) & 0xFFu), s, c),
                  __builtin_fmaf(static_cast<float>((m1 >> 8) & 0xFFu), s, c));
    d.z = pk_bf16(__builtin_fmaf(static_cast<float>((m0 >> 16) & 0xFFu), s, c),
                  __builtin_fmaf(static_cast<float>((m1 >> 16) & 0xFFu), s, c));
    d.w = pk_bf16(__builtin_fmaf(static_cast<float>(m0 >> 24), s, c),
                  __builtin_fmaf(static_cast<float>(m1 >> 24), s, c));
    return __builtin_bit_cast(bf16x8, d);
}

// Vector-memory instructions one wavefront issues per helper call; the K
// loop's waits (s_waitcnt vmcnt, completions counted in issue order) are
// written in these counts.
constexpr int kWGroupLoads = 1;   // load_wgroup: one K group of codes
constexpr int kRScaleLoads = 2;   // load_rscales: one record's scales

// Loads the codes of group ks of the chunk for this lane (code_off: the
// lane's byte offset inside a record's group).  Issues kWGroupLoads loads.
__device__ inline void load_wgroup(WGroup& g, __amdgpu_buffer_rsrc_t w, uint32_t code_off, int ks) {
    const int soff = (ks >> 3) * kRecWords * 4 + (ks & 7) * 512 * 4;
    g.w = __builtin_bit_cast(u32x4,
                             __builtin_amdgcn_raw_buffer_load_b128(w, code_off, soff, kNonTemporal));
}

// Loads this lane's scales of record rec (its 8 groups, one 32-bit word per
// group; scale_off: the lane's byte offset inside a record's scale block).
// Issues kRScaleLoads loads.
__device__ inline void load_rscales(u32x4 (&sc)[2], __amdgpu_buffer_rsrc_t w, uint32_t scale_off,
                                    int rec) {
    const int soff = rec * kRecWords * 4 + 4096 * 4;
    sc[0] = __builtin_bit_cast(u32x4,
                               __builtin_amdgcn_raw_buffer_load_b128(w, scale_off, soff, kNonTemporal));
    sc[1] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(w, scale_off + 16, soff, kNonTemporal));
}

// Scale word of group gi (0..7) of a record's scales.
__device__ inline uint32_t rscale(const u32x4 (&sc)[2], int gi) {
    const u32x4& v = sc[gi >> 2];
    return (gi & 3) == 0 ? v.x : (gi & 3) == 1 ? v.y : (gi & 3) == 2 ? v.z : v.w;
}

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt left free).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that also keeps the compiler from moving LDS accesses
// across it.  The activation slots are written by buffer-to-LDS loads whose
// completion each wave has already waited for (vmcnt), so no fence is needed
// (a fence would wait for every weight load in flight as well).
__device__ inline void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// Workgroup barrier after LDS reads or writes made with ds_ instructions: the
// compiler does not wait for them before an s_barrier it did not place, so
// this one waits for all of this wave's LDS operations first (the epilogue's
// staging writes must have landed before other waves read them).
__device__ inline void barrier_ds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct Item {
    int e, p0, nrows, pair;
};

// The four activation slots (separate LDS objects, so that the compiler can
// tell a slot being read from one being loaded); the epilogue stages 32 rows
// of fp32 results in each.
struct Slots {
    char* p[4];
};

}  // namespace

// How the store loop finds and filters output rows.
enum RowMode {
    ROWS_PLAIN = 0,   // out row = position
    ROWS_MAP = 1,     // out row from sorted_ids (padding sentinels skipped)
    ROWS_CONTIG = 2   // out row = position, stored only if m_indices names the item's expert
};

// Stores rows [r0, r1) of a work item from the fp32 staging tile in LDS
// ([128 rows][256 columns]; rows 32 k .. 32 k + 31 of the pass in slot k):
// 32 lanes per row, 8 staged values each; bf16 or fp32 rows, or SiLU(gate) *
// up of the interleaved gate/up pairs (4 outputs per lane).  KIND and ROWS
// are template parameters so that each variant is a straight loop: with the
// variants merged, the compiler could no longer tell which registers came
// from memory and waited for every store in flight before each new one.
template <int KIND, int ROWS>
__device__ __forceinline__ void store_rows_k(const GemmArgs& a, const Item& it, const Slots& sl,
                                          int r0, int r1) {
    constexpr bool silu = KIND == OUT_SILU;
    const int nout = silu ? a.N / 2 : a.N;             // output row length
    const int width = silu ? 128 : 256;                // output columns of the tile
    const int col0 = it.pair * width;
    const int cvalid = nout - col0 < width ? nout - col0 : width;
    const int q = threadIdx.x & 31;                    // 8 staged values: 8 columns or 4 pairs
    const int cc = silu ? 4 * q : 8 * q;               // first output column of this lane
    if (cc >= cvalid) return;
    // slot k (a compile-time index: the reads stay LDS reads) holds rows
    // r0 + 32 k .. r0 + 32 k + 31
#pragma unroll
    for (int k = 0; k < 4; ++k)
    for (int rr = (threadIdx.x >> 5); rr < 32; rr += 8) {
        const int r = r0 + 32 * k + rr;
        if (r >= r1) break;
        int64_t orow = it.p0 + r;
        if (ROWS == ROWS_MAP) {
            const int f = a.sorted_ids[it.p0 + r];
            if (f < 0 || f >= a.num_slots) continue;
            if (a.orow == W4A16_OROW_SLOT) orow = f;
        } else if (ROWS == ROWS_CONTIG) {
            if (a.m_indices[it.p0 + r] != it.e) continue;
        }
        const f32x4* src = reinterpret_cast<const f32x4*>(sl.p[k]) + rr * 64 + 2 * q;
        const f32x4 v0 = src[0], v1 = src[1];
        if (KIND == OUT_SILU) {
            u32x2 o;
            o.x = pk_bf16(silu_mul_bf16(v0.x, v0.y), silu_mul_bf16(v0.z, v0.w));
            o.y = pk_bf16(silu_mul_bf16(v1.x, v1.y), silu_mul_bf16(v1.z, v1.w));
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow * nout + col0 + cc) = o;
        } else if (KIND == OUT_BF16) {
            u32x4 o;
            o.x = pk_bf16(v0.x, v0.y);
            o.y = pk_bf16(v0.z, v0.w);
            o.z = pk_bf16(v1.x, v1.y);
            o.w = pk_bf16(v1.z, v1.w);
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + orow * nout + col0 + cc) = o;
        } else {
            f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow * nout + col0 + cc);
            o[0] = v0;
            o[1] = v1;
        }
    }
}

template <int ROWS>
__device__ __forceinline__ void store_rows_m(const GemmArgs& a, const Item& it, const Slots& sl,
                                          int r0, int r1) {
    if (a.out_kind == OUT_SILU) store_rows_k<OUT_SILU, ROWS>(a, it, sl, r0, r1);
    else if (a.out_kind == OUT_BF16) store_rows_k<OUT_BF16, ROWS>(a, it, sl, r0, r1);
    else store_rows_k<OUT_F32, ROWS>(a, it, sl, r0, r1);
}

__device__ __forceinline__ void store_rows(const GemmArgs& a, const Item& it, const Slots& sl,
                                        int r0, int r1) {
    const bool row_map = (a.tile_src == TILE_TABLE && a.orow == W4A16_OROW_SLOT) ||
                         a.tile_src == TILE_BLOCKS;
    if (row_map) store_rows_m<ROWS_MAP>(a, it, sl, r0, r1);
    else if (a.tile_src == TILE_CONTIG) store_rows_m<ROWS_CONTIG>(a, it, sl, r0, r1);
    else store_rows_m<ROWS_PLAIN>(a, it, sl, r0, r1);
}

// One work item with up to 32 * RB rows.
//
// The K loop runs in stages of two groups (64 K).  The activations of a stage
// sit in an LDS slot as [32 RB rows][128 bytes], row-major; the 16-byte chunk
// c of row r is stored at chunk position c ^ f(r), f(r) = (r & 7) ^ ((r >> 3)
// & 1), so that the A-operand reads (eight or sixteen consecutive rows, one
// chunk each) fall in distinct LDS banks.  Each buffer-to-LDS load brings
// eight whole rows of a stage (eight lanes per 128-byte line), which the
// vector L1 serves as eight line requests.  Four slots: while stage s is read,
// s + 1 has landed and s + 2, s + 3 are in flight.  Weights of stages s .. s +
// 3 sit in a register ring.  One barrier per stage.
template <int RB>
__device__ __forceinline__ void large_item(const GemmArgs& a, const Item& it, int wave, int lane,
                                           const Slots& sl) {
    // loads per wave and stage (one batch, `issue` below): 4 RB
    // buffer-to-LDS loads of 8 rows, dealt to the four waves, and the codes
    // of the stage's two groups
    constexpr int kDma = RB;
    constexpr int kStageOps = kDma + 2 * kWGroupLoads;
    static_assert(3 * kStageOps + 2 * kWGroupLoads + kRScaleLoads < 64,
                  "everything the prologue issues fits the 6-bit vmcnt field");

    const int chunk = it.pair * 2 + (wave >> 1);
    const int h = wave & 1;
    const bool active = chunk < a.NC;
    // rows found through sorted_ids (indexed layout); masked and contiguous
    // rows are positions
    const bool slot_rows = a.tile_src == TILE_TABLE || a.tile_src == TILE_BLOCKS;
    const int KS = a.KS;
    const int KSP = a.KSP;          // a multiple of 8; groups >= KS have zero weights
    const int SA = (KS + 1) >> 1;   // stages holding real activations

    // Activation load i of this wave covers rows 8 j .. 8 j + 7, j = wave + 4 i:
    // lane l takes row 8 j + l / 8 and global chunk (l % 8) ^ f(row).  Rows
    // past the tile reuse its first row (computed, never stored).
    const uint32_t cl = static_cast<uint32_t>((lane & 7) ^ (lane >> 3));
    uint32_t aoff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int j = wave + 4 * i;
        const int r = 8 * j + (lane >> 3);
        const int rr = r < it.nrows ? r : 0;
        int64_t row = it.p0 + rr;
        if (slot_rows && a.arow != W4A16_AROW_POSITION) {
            int f = a.sorted_ids[it.p0 + rr];
            if (f < 0 || f >= a.num_slots) f = a.sorted_ids[it.p0];
            if (f < 0 || f >= a.num_slots) f = 0;
            row = (a.arow == W4A16_AROW_TOKEN) ? f / a.top_k : f;
        }
        row = row < a.A_rows ? row : a.A_rows - 1;
        // A_rows * K * 2 < 2^32 is checked on the host
        aoff[i] = static_cast<uint32_t>(row * a.K * 2) + 16 * (cl ^ static_cast<uint32_t>(j & 1));
    }
    // In the last stage of an odd group count, the chunks of the missing
    // second group (chunk >= 4) repeat the first group's (a row's K range is
    // never left; those products meet zero weights).
    const uint32_t dpart = (cl & 4) ? 64u : 0u;
    const __amdgpu_buffer_rsrc_t x = make_rsrc(a.A, static_cast<uint64_t>(a.A_rows) * a.K * 2);

    const int64_t cbase = static_cast<int64_t>(it.e) * a.NC + (active ? chunk : a.NC - 1);
    const __amdgpu_buffer_rsrc_t w =
        make_rsrc(a.packed + cbase * a.chunk_words, static_cast<uint64_t>(a.chunk_words) * 4);
    const uint32_t code_off = static_cast<uint32_t>((h * 64 + lane) * 16);
    const uint32_t scale_off = static_cast<uint32_t>((h * 32 + (lane & 31)) * 32);
    const uint32_t nib = a.nib_mask;
    const int NREC = KSP >> 3;

    // One batch of loads: the activations of stage sa into LDS slot `slot`
    // and the codes of stage sw into ring entry r (the waits count whole
    // batches, so their order inside a batch is free).  Stages past the
    // activations repeat the last one; weight groups past KSP repeat the last
    // (never used).
    auto issue = [&](int sa, int slot, int sw, WGroup (&r)[2]) {
        const bool part = (KS & 1) && sa >= SA - 1;
        sa = sa < SA ? sa : SA - 1;
#pragma unroll
        for (int i = 0; i < kDma; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(x, LDS_PTR(sl.p[slot] + (wave + 4 * i) * 1024), 16,
                                                     part ? aoff[i] - dpart : aoff[i], sa * 128, 0, 0);
        const int g0 = 2 * sw < KSP ? 2 * sw : KSP - 1;
        const int g1 = 2 * sw + 1 < KSP ? 2 * sw + 1 : KSP - 1;
        load_wgroup(r[0], w, code_off, g0);
        load_wgroup(r[1], w, code_off, g1);
    };

    f32x16 acc[RB][2];
#pragma unroll
    for (int t = 0; t < RB; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[t][j] = f32x16{};

    // A operand of (row block t, group half hh, K step st): lane l reads row
    // 32 t + l % 32, chunk 4 hh + 2 st + l / 32, at its swizzled position
    const uint32_t fl = static_cast<uint32_t>((lane & 7) ^ ((lane >> 3) & 1));
    uint32_t aread[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int st = 0; st < 2; ++st)
            aread[hh][st] = static_cast<uint32_t>((lane & 31) * 128) +
                            16 * ((static_cast<uint32_t>(4 * hh + 2 * st + (lane >> 5))) ^ fl);

    // A operands of one K step of 16 (all row blocks), double-buffered by K
    // step; B operands of a group (both K steps), double-buffered by group
    bf16x8 av[2][RB];
    bf16x8 b[2][2][2];
    auto read_a = [&](int slot, int hh, int st, bf16x8 (&dst)[RB]) {
#pragma unroll
        for (int t = 0; t < RB; ++t)
            dst[t] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(sl.p[slot] + t * 4096 + aread[hh][st]));
    };
    // the B operands of K step st of a group: blocks h and h + 2
    auto dequant_step = [&](const WGroup& g, uint32_t sw, int st, bf16x8 (&bb)[2][2]) {
        const float s0 = __uint_as_float(sw << 16), s1 = __uint_as_float(sw & 0xFFFF0000u);
        bb[0][st] = dequant_word(st == 0 ? g.w.x : g.w.y, nib, s0, -8.0f * s0);
        bb[1][st] = dequant_word(st == 0 ? g.w.z : g.w.w, nib, s1, -8.0f * s1);
    };
    // The 2 RB MFMAs of K step st (row block outer: an accumulator's next MFMA
    // is a whole K step later).  Spread over them: one LDS read of the next
    // step's A after every other MFMA, about 48 / (2 RB) VALU ops of a half
    // group's dequant after each, and nvm buffer loads after odd MFMAs, so
    // that no burst holds up the wave's issue.
    auto mfma_step = [&](const bf16x8 (&av_)[RB], const bf16x8 (&b_)[2][2], int st, int nvm) {
#pragma unroll
        for (int t = 0; t < RB; ++t)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                acc[t][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av_[t], b_[jj][st], acc[t][jj],
                                                                     0, 0, 0);
        constexpr int kV = (48 + 2 * RB - 1) / (2 * RB);
#pragma unroll
        for (int i = 0; i < 2 * RB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (i % 2 == 1 && i / 2 < nvm) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        }
    };

    // Prologue: codes of stage 0 and the scales of record 0, then
    // (activations of s, codes of s + 1) for s = 0, 1, 2: the same order as
    // the loop's batches.  Scales: one record (four stages) per pair of loads,
    // the next record's loaded with the first batch of a trip.
    WGroup ring[4][2];
    u32x4 sc_cur[2], sc_nxt[2];
    {
        load_wgroup(ring[0][0], w, code_off, 0);
        load_wgroup(ring[0][1], w, code_off, 1);
        load_rscales(sc_cur, w, scale_off, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            issue(s, s, s + 1, ring[s + 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // issued: codes of stage 0 and the scales of record 0, then three
    // batches; the batches of stages 1 and 2 may stay in flight, so the
    // activations of stage 0 have landed
    wait_vmcnt<2 * kStageOps>();
    barrier_lds();
    read_a(0, 0, 0, av[0]);
    dequant_step(ring[0][0], rscale(sc_cur, 0), 0, b[0]);
    dequant_step(ring[0][0], rscale(sc_cur, 0), 1, b[0]);

    // Four stages per trip (slot and ring indices static; KSP / 2 is even),
    // four K steps per stage: (group 2 s, step 0), (2 s, 1), (2 s + 1, 0),
    // (2 s + 1, 1).  While the MFMAs of one K step run, the A operands of the
    // next step are read from LDS and half a group's B operands dequantised
    // (group 2 s + 1 during the first two steps, group 2 s + 2 during the
    // last two: each into the buffer half its own group no longer reads).
    // Before the last step: wait for this wave's batch of stage s - 2
    // (activations of s + 1; the batch of s - 1 may stay in flight) and
    // barrier (they all landed; every wave is done with the slot of stage
    // s - 1); then, spread over the MFMAs of the last step, load the
    // activations of stage s + 3 into that slot and the weights of stage
    // s + 4 into ring entry s % 4, and read the first A operands of stage
    // s + 1.
    const int NST = KSP >> 1;
    for (int s0 = 0; s0 < NST; s0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + u;
            const uint32_t sw1 = rscale(sc_cur, 2 * u + 1);
            __builtin_amdgcn_sched_barrier(0);
            read_a(u, 0, 1, av[1]);
            dequant_step(ring[u][1], sw1, 0, b[1]);
            mfma_step(av[0], b[0], 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            read_a(u, 1, 0, av[0]);
            dequant_step(ring[u][1], sw1, 1, b[1]);
            mfma_step(av[1], b[0], 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            // (group 2 s + 2's codes sit in ring[(u + 1) & 3][0], three
            // stages old; its scales in sc_cur, or at u == 3 in sc_nxt,
            // loaded at u == 0)
            const uint32_t sw2 = u < 3 ? rscale(sc_cur, 2 * u + 2) : rscale(sc_nxt, 0);
            read_a(u, 1, 1, av[1]);
            dequant_step(ring[(u + 1) & 3][0], sw2, 0, b[0]);
            mfma_step(av[0], b[1], 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // issued since the batch that holds the activations of stage s + 1:
            // the batch of the previous step (kStageOps), which may stay in
            // flight, followed at u == 0 by the next record's scales
            if (u == 1)
                wait_vmcnt<kStageOps + kRScaleLoads>();
            else
                wait_vmcnt<kStageOps>();
            barrier_lds();
            __builtin_amdgcn_sched_barrier(0);
            // (the batch's codes go to ring[u], both of whose groups are
            // dequantised)
            issue(s + 3, (u + 3) & 3, s + 4, ring[u]);
            if (u == 0) {
                const int rn = (s0 >> 2) + 1;
                load_rscales(sc_nxt, w, scale_off, rn < NREC ? rn : NREC - 1);
            }
            read_a((u + 1) & 3, 0, 0, av[0]);
            dequant_step(ring[(u + 1) & 3][0], sw2, 1, b[0]);
            mfma_step(av[1], b[1], 1, u == 0 ? kStageOps + kRScaleLoads : kStageOps);
        }
        sc_cur[0] = sc_nxt[0];
        sc_cur[1] = sc_nxt[1];
    }
    // drain the loads past the end before the slots are reused
    wait_vmcnt<0>();
    barrier_ds();

    // Epilogue, in passes of 128 rows: the fp32 accumulators of the pass go
    // to LDS as a [128 rows][256 columns] tile of the workgroup (the two
    // chunks side by side; for SiLU * gate, gate and up interleaved per
    // output column), then all threads store whole row segments.
    // acc[t][jj][i] holds row 32 t + 8 (i / 4) + 4 (lane / 32) + i % 4 of
    // column 32 (h + 2 jj) + lane % 32 of the chunk.
    const bool silu = a.out_kind == OUT_SILU;
    const int zc = (wave >> 1) * 64 + 32 * h + (lane & 31);          // SiLU output column
    const int c0 = (wave >> 1) * 128 + 32 * h + (lane & 31);         // plain output column
    const int s0 = silu ? 2 * zc : c0, s1 = silu ? 2 * zc + 1 : c0 + 64;
#pragma unroll
    for (int p = 0; p < (RB + 3) / 4; ++p) {
#pragma unroll
        for (int t = 4 * p; t < RB && t < 4 * p + 4; ++t) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                float* stg = reinterpret_cast<float*>(sl.p[t - 4 * p]);
                stg[r * 256 + s0] = acc[t][0][i];
                stg[r * 256 + s1] = acc[t][1][i];
            }
        }
        barrier_ds();
        store_rows(a, it, sl, 128 * p, it.nrows < 128 * p + 128 ? it.nrows : 128 * p + 128);
        barrier_ds();    // the staging bytes are reused (next pass, next item's loads)
    }
}

// Tile ty of the launch: expert, first position and rows (nrows <= 0: empty).
__device__ inline Item tile_of(const GemmArgs& a, int ty) {
    Item it{-1, 0, 0, 0};
    if (a.tile_src == TILE_TABLE) {
        const int4 t = reinterpret_cast<const int4*>(a.tiles)[ty];
        it.e = t.x;
        it.p0 = t.y;
        it.nrows = t.z;
    } else if (a.tile_src == TILE_BLOCKS) {
        it.p0 = ty * a.block_m;
        it.e = a.expert_ids[ty];
        it.nrows = a.sorted_cap - it.p0 < a.block_m ? a.sorted_cap - it.p0 : a.block_m;
    } else if (a.tile_src == TILE_MASKED) {
        // masked_m is the valid count of each expert; a count above max_m is
        // cut to max_m, so no tile reaches past the expert's rows
        const int g = ty / a.chunks_per_expert;
        const int r0 = (ty % a.chunks_per_expert) * a.tile_m;
        const int mg = a.masked_m[g];
        const int cnt = mg < a.max_m ? mg : a.max_m;
        it.e = g;
        it.p0 = g * a.max_m + r0;
        it.nrows = cnt - r0 < a.tile_m ? cnt - r0 : a.tile_m;
    } else {
        // contiguous: block ty of tile_m rows; its expert is its first row's
        // (every expert's segment starts on a 128-row boundary), a block that
        // starts with padding holds no rows; rows of other experts inside the
        // block are computed but not stored
        it.p0 = ty * a.tile_m;
        const int64_t left = a.A_rows - it.p0;
        it.e = left > 0 ? a.m_indices[it.p0] : -1;
        it.nrows = left < a.tile_m ? static_cast<int>(left) : a.tile_m;
    }
    if (it.e < 0 || it.e >= a.E) it.nrows = 0;
    it.nrows = it.nrows < 256 ? it.nrows : 256;
    return it;
}

// Tiles the work queue can order (more run in the static order).
constexpr int kMaxOrder = 256;

// Dynamic schedule for launches with more items than workgroups.  Every
// workgroup ranks the tiles by 32-row block count, largest first (ties by
// index, so the order is the same everywhere), and deals them to the eight
// XCDs in snake order (ranks x, 15-x, 16+x, 31-x, ... go to XCD x), which
// evens out the row blocks per XCD.  The items of XCD x (its tiles in that
// order, each tile's column pairs in turn) are handed out by counter q[x]:
// the column pairs of one tile run close together in time on the XCD whose
// L2 holds that tile's activation rows, and the largest items go first so
// that the last round is made of the smallest.  A workgroup whose XCD has no
// items left takes them from the other XCDs' counters.  q[8] counts the
// workgroups that found every counter spent; the last of them clears all
// nine, so the next launch finds them at zero.
__device__ inline void rank_tiles(const GemmArgs& a, int n_tiles, int* s_cost, int* s_order) {
    const int t = threadIdx.x;
    int cost = 0;
    if (t < n_tiles) {
        const Item it = tile_of(a, t);
        cost = it.nrows > 0 ? (it.nrows + 31) >> 5 : 0;
    }
    s_cost[t] = cost;
    __syncthreads();
    if (t < n_tiles) {
        int rank = 0;
        for (int u = 0; u < n_tiles; ++u) {
            const int c = s_cost[u];
            rank += c > cost || (c == cost && u < t);
        }
        s_order[rank] = t;
    }
    __syncthreads();
}

// Thread 0: the next item (tile * CP + pair) from the XCD's counter, then
// from the others'; -1 once all are spent.  `spent` marks counters found past
// their last item (they never come back).
__device__ inline int pull_item(int* q, int xcd, int n_tiles, int CP, const int* s_cost,
                                const int* s_order, unsigned& spent) {
    for (int k = 0; k < 8; ++k) {
        const int x = (xcd + k) & 7;
        if (spent & (1u << x)) continue;
        const int j = atomicAdd(q + x, 1);
        const int i = j / CP;
        const int r = 16 * (i >> 1) + ((i & 1) ? 15 - x : x);
        if (r < n_tiles && s_cost[s_order[r]] > 0) return s_order[r] * CP + j % CP;
        spent |= 1u << x;
    }
    return -1;
}

__global__ void __launch_bounds__(256) k_gemm_large(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char slot0[kSlot];
    __shared__ __attribute__((aligned(1024))) char slot1[kSlot];
    __shared__ __attribute__((aligned(1024))) char slot2[kSlot];
    __shared__ __attribute__((aligned(1024))) char slot3[kSlot];
    __shared__ int s_cost[kMaxOrder];
    __shared__ int s_order[kMaxOrder];
    __shared__ int s_pick;
    Slots sl;
    sl.p[0] = slot0;
    sl.p[1] = slot1;
    sl.p[2] = slot2;
    sl.p[3] = slot3;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    int n_tiles;
    if (a.tile_src == TILE_TABLE) {
        n_tiles = a.tile_count[0];
        n_tiles = n_tiles < a.tiles_cap ? n_tiles : a.tiles_cap;
    } else if (a.tile_src == TILE_BLOCKS) {
        n_tiles = a.ntp[0] / a.block_m;
        n_tiles = n_tiles < a.tiles_cap ? n_tiles : a.tiles_cap;
    } else {
        n_tiles = a.grid_tiles_total;   // masked and contiguous: host-known
    }
    const int CP = (a.NC + 1) / 2;
    const int nwg = gridDim.x;
    const int xcd = blockIdx.x & 7;
    const bool many = static_cast<int64_t>(n_tiles) * CP > nwg;
    const bool queued = many && a.counters && n_tiles <= kMaxOrder;
    // static order: with a whole number of workgroups per XCD, tile ty runs on
    // XCD ty % 8; otherwise items are dealt out in order
    const bool by_xcd = many && (nwg & 7) == 0;
    const int per_xcd = nwg >> 3;
    if (queued) rank_tiles(a, n_tiles, s_cost, s_order);
    unsigned spent = 0;
    for (int j = by_xcd ? (blockIdx.x >> 3) : blockIdx.x;; j += by_xcd ? per_xcd : nwg) {
        int ty, pair;
        if (queued) {
            if (threadIdx.x == 0) s_pick = pull_item(a.counters, xcd, n_tiles, CP, s_cost, s_order, spent);
            __syncthreads();
            // every wave reads s_pick before the item's first barrier, so the
            // next write cannot overtake a read
            const int pick = __builtin_amdgcn_readfirstlane(s_pick);
            if (pick < 0) break;
            ty = pick / CP;
            pair = pick % CP;
        } else if (by_xcd) {
            ty = 8 * (j / CP) + xcd;
            pair = j % CP;
            if (j / CP * 8 >= n_tiles) break;
            if (ty >= n_tiles) continue;
        } else {
            ty = j / CP;
            pair = j % CP;
            if (ty >= n_tiles) break;
        }
        Item it = tile_of(a, ty);
        if (it.nrows <= 0) continue;
        it.pair = pair;
        switch ((it.nrows + 31) >> 5) {
            case 1: large_item<1>(a, it, wave, lane, sl); break;
            case 2: large_item<2>(a, it, wave, lane, sl); break;
            case 3: large_item<3>(a, it, wave, lane, sl); break;
            case 4: large_item<4>(a, it, wave, lane, sl); break;
            case 5: large_item<5>(a, it, wave, lane, sl); break;
            case 6: large_item<6>(a, it, wave, lane, sl); break;
            case 7: large_item<7>(a, it, wave, lane, sl); break;
            default: large_item<8>(a, it, wave, lane, sl); break;
        }
    }
    if (queued && threadIdx.x == 0) {
        __threadfence();
        if (atomicAdd(a.counters + 8, 1) == nwg - 1)
            for (int x = 0; x < 9; ++x) atomicExch(a.counters + x, 0);
    }
}

static int g_num_cus = 0;

void launch_gemm_large(const GemmArgs& a, hipStream_t st) {
    if (g_num_cus <= 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    const int64_t items = static_cast<int64_t>(a.grid_tiles) * ((a.NC + 1) / 2);
    const int grid = static_cast<int>(items < g_num_cus ? items : g_num_cus);
    k_gemm_large<<<dim3(grid), dim3(256), 0, st>>>(a);
}

}  // namespace w4a16
