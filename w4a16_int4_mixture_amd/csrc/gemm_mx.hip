// Grouped A8W4 GEMM: MXFP8 activations on MXFP4 weights, streamed through
// CDNA4's block-scaled matrix instruction.
//
//   out[p, n] = sum_c e4m3(A[row(p), c]) 2^(sa[row(p), c/32] - 127)
//                     * e2m1(q[e, n, c]) 2^(sw[e, n, c/32] - 127)
//
// news.ainew.jp, "vLLM publishes Kimi K3 production support", MXFP4 MoE: the
// expert weights are MXFP4, and the AMD path has A8W4 fused operators (8-bit
// activations on the 4-bit weights).  With few routed rows per expert the
// GEMM is bound by weight traffic (Chord page, "H200 and Blackwell indexed
// decode"), as in the W4A16 streaming kernel, whose item schedule this
// kernel keeps.
//
// CDNA4 design.  v_mfma_scale_f32_16x16x128_f8f6f4 takes E4M3 A and E2M1 B
// with one E8M0 scale per 32 K of each row and column and applies the scales
// itself: no dequantisation and no scale arithmetic in the kernel.  Operand
// layout (lane l, g = l/16):
//   A: row l%16; its 32 bytes hold K = 16g + (0..15), then 64 + 16g + (0..15)
//   B: column l%16; its 32 nibbles hold K = 32g + (0..31), low nibble first
//   scales: the byte for row (column) l%16 and K block g; op_sel picks the
//   byte of the 32-bit operand (the weights' four 16-column blocks share one
//   word, one byte each)
//   D: column l%16, rows 4g + (0..3)
// A workgroup is four wavefronts on four neighbouring 64-column chunks of a
// row tile of up to 16*MT rows, over the whole K range in records of 256 K
// (two instructions per 16x16 block).
//   * Weights: each lane streams its 16-byte code slices and one scale word
//     per 128 K with non-temporal loads into a one-record register ring,
//     refilled as consumed (8 KB in flight per wavefront).
//   * Activations: the record's A fragments go from HBM/L2 into LDS with
//     buffer loads carrying the LDS bit (double-buffered, one barrier per
//     record), wavefront w loading the (step, half) = (w/2, w%2) fragments
//     of every row block; each lane's activation scale bytes come with the
//     register ring.

#include "device_common.h"
#include "internal.h"
#include "tile_store.h"

namespace w4a16 {

namespace {

using namespace dev;

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWPL = 4;                       // 16-column blocks per 64-column chunk
constexpr int kCodeWords = 512 * kWPL;        // code words of a record
constexpr int kRecWords = 544 * kWPL;         // then 32 WPL words of E8M0 bytes

// Vector-memory instructions one wavefront issues per helper call (the K
// loop's vmcnt waits are written in these counts).
constexpr int kStepLoads = kWPL + 1;          // load_step: code slices + scale word

// One 128-K step of this lane's B operands (four 16-column blocks) and their
// E8M0 scale word.
struct Step {
    u32x4 b[kWPL];
    uint32_t sc;
};

// Loads step st of the chunk (record st/2, half st%2).  Issues kStepLoads.
__device__ inline void load_step(Step& d, __amdgpu_buffer_rsrc_t w, int lane, int st) {
    const int soff = (st >> 1) * kRecWords * 4;
    const int s = st & 1;
#pragma unroll
    for (int j = 0; j < kWPL; ++j)
        d.b[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(w, (((s * kWPL + j) * 64 + lane) * 4) * 4,
                                                         soff, kNonTemporal));
    d.sc = __builtin_amdgcn_raw_buffer_load_b32(w, (kCodeWords + s * 64 + lane) * 4, soff,
                                               kNonTemporal);
}

template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier after this wavefront's LDS accesses have completed (the
// staging buffers are written by buffer-to-LDS loads whose completion each
// wavefront waits for with vmcnt first).
__device__ inline void barrier_ds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Where one wavefront reads: its chunk, the activation codes and scales, and
// each row block's activation row for this lane (rows past the tile reuse
// its first row: computed, never stored).
template <int MT>
struct MxSrc {
    __amdgpu_buffer_rsrc_t w, x, xs;
    int64_t row[MT];
};

template <int MT>
__device__ __forceinline__ MxSrc<MT> mx_src(const GemmArgs& a, int e, int p0, int nrows, int chunk,
                                            int lane) {
    MxSrc<MT> src;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int r = 16 * t + (lane & 15);
        const int rr = r < nrows ? r : 0;
        int64_t row = p0 + rr;
        if (a.arow != W4A16_AROW_POSITION) {
            int f = a.sorted_ids[p0 + rr];
            if (f < 0 || f >= a.num_slots) f = a.sorted_ids[p0];
            if (f < 0 || f >= a.num_slots) f = 0;
            row = (a.arow == W4A16_AROW_TOKEN) ? f / a.top_k : f;
        }
        src.row[t] = row < a.A_rows ? row : a.A_rows - 1;
    }
    // A_rows * K < 2^32 is checked on the host
    src.x = make_rsrc(a.A, static_cast<uint64_t>(a.A_rows) * a.K);
    src.xs = make_rsrc(a.A_scales, static_cast<uint64_t>(a.A_rows) * (a.K / 32));
    const int64_t cbase = static_cast<int64_t>(e) * a.NC + (chunk < a.NC ? chunk : a.NC - 1);
    src.w = make_rsrc(a.packed + cbase * a.chunk_words, static_cast<uint64_t>(a.chunk_words) * 4);
    return src;
}

// LDS of one record: A fragments [step s][half h][row block t][lane] x 16 B.
template <int MT>
struct MxLds {
    static constexpr int frags = 4 * MT * 64;   // u32x4 per buffer
};

// The activation fragments of record r into LDS buffer buf: this wavefront's
// (s, h) = (wave/2, wave%2) fragment of every row block, lane l reading row
// 16t + l%16 at K = 256r + 128s + 64h + 16(l/16) (a slice past K re-reads the
// row's last 16 bytes: its weights are zero).  Issues MT loads.
template <int MT>
__device__ inline void dma_record(const GemmArgs& a, const MxSrc<MT>& src, u32x4* buf, int r,
                                  int wave, int lane) {
    const int s = wave >> 1, h = wave & 1;
    int koff = 256 * r + 128 * s + 64 * h + 16 * (lane >> 4);
    koff = koff + 16 <= a.K ? koff : a.K - 16;
#pragma unroll
    for (int t = 0; t < MT; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            src.x, LDS_PTR(buf + ((s * 2 + h) * MT + t) * 64),
            16, static_cast<uint32_t>(src.row[t] * a.K + koff), 0, 0, 0);
}

// This lane's activation scale bytes of record r: block 8r + 4s + l/16 of
// row 16t + l%16 (a block past K re-reads the row's last one).  Issues 2 MT
// loads.
template <int MT>
__device__ inline void load_ascales(const GemmArgs& a, const MxSrc<MT>& src, uint32_t (&sc)[MT][2],
                                    int r, int lane) {
    const int KS = a.K / 32;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        int blk = 8 * r + 4 * s + (lane >> 4);
        blk = blk < KS ? blk : KS - 1;
#pragma unroll
        for (int t = 0; t < MT; ++t)
            sc[t][s] = __builtin_amdgcn_raw_buffer_load_b8(
                src.xs, static_cast<uint32_t>(src.row[t] * KS + blk), 0, 0);
    }
}

// One block-scaled instruction on column block J (A: E4M3, cbsz 0; B: E2M1,
// blgp 4; A scale byte 0, B scale byte J of the step's scale word).
template <int J>
__device__ __forceinline__ f32x4 mx_mfma(const i32x8& av, const u32x4& b, int sa, uint32_t sc,
                                         const f32x4& c) {
    const i32x8 bv = {static_cast<int32_t>(b.x), static_cast<int32_t>(b.y),
                      static_cast<int32_t>(b.z), static_cast<int32_t>(b.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 4, 0, sa, J,
                                                            static_cast<int>(sc));
}

// The instructions of one 128-K step for every row block and column block.
template <int MT, int S>
__device__ __forceinline__ void mx_step(const u32x4* abuf, const Step& st, const uint32_t (&asc)[MT][2],
                                        f32x4 (&acc)[MT][kWPL], int lane) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const u32x4 lo = abuf[((S * 2 + 0) * MT + t) * 64 + lane];
        const u32x4 hi = abuf[((S * 2 + 1) * MT + t) * 64 + lane];
        const i32x8 av = {static_cast<int32_t>(lo.x), static_cast<int32_t>(lo.y),
                          static_cast<int32_t>(lo.z), static_cast<int32_t>(lo.w),
                          static_cast<int32_t>(hi.x), static_cast<int32_t>(hi.y),
                          static_cast<int32_t>(hi.z), static_cast<int32_t>(hi.w)};
        const int sa = static_cast<int>(asc[t][S]);
        static_assert(kWPL == 4, "four column blocks per chunk");
        acc[t][0] = mx_mfma<0>(av, st.b[0], sa, st.sc, acc[t][0]);
        acc[t][1] = mx_mfma<1>(av, st.b[1], sa, st.sc, acc[t][1]);
        acc[t][2] = mx_mfma<2>(av, st.b[2], sa, st.sc, acc[t][2]);
        acc[t][3] = mx_mfma<3>(av, st.b[3], sa, st.sc, acc[t][3]);
    }
}

// One record on LDS buffer abuf: the two steps, each followed by the refill of
// its ring slot with the same step of record rn, then the activation scales
// of record rn.  Issues 2 kStepLoads + 2 MT loads.
template <int MT>
__device__ __forceinline__ void mx_record(const GemmArgs& a, const MxSrc<MT>& src, const u32x4* abuf,
                                          Step (&ring)[2], uint32_t (&asc)[MT][2],
                                          f32x4 (&acc)[MT][kWPL], int rn, int lane) {
    mx_step<MT, 0>(abuf, ring[0], asc, acc, lane);
    __builtin_amdgcn_sched_barrier(0);
    load_step(ring[0], src.w, lane, 2 * rn);
    __builtin_amdgcn_sched_barrier(0);
    mx_step<MT, 1>(abuf, ring[1], asc, acc, lane);
    __builtin_amdgcn_sched_barrier(0);
    load_step(ring[1], src.w, lane, 2 * rn + 1);
    load_ascales<MT>(a, src, asc, rn, lane);
    __builtin_amdgcn_sched_barrier(0);
}

// One tile item: the K loop over all records, then the stores.
template <int MT>
__device__ __forceinline__ void mx_tile(const GemmArgs& a, int e, int p0, int nrows, int chunk,
                                        int wave, int lane, u32x4* buf0, u32x4* buf1) {
    constexpr int kRefill = 2 * kStepLoads + 2 * MT;   // loads of one record's refills
    constexpr int kAct = MT;                           // dma_record
    static_assert(kRefill + kAct < 64, "waits fit the 6-bit vmcnt field");
    const MxSrc<MT> src = mx_src<MT>(a, e, p0, nrows, chunk, lane);
    const int nrec = a.KSP / 8;

    f32x4 acc[MT][kWPL];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < kWPL; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Step ring[2];
    uint32_t asc[MT][2];
    dma_record<MT>(a, src, buf0, 0, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
    load_step(ring[0], src.w, lane, 0);
    load_step(ring[1], src.w, lane, 1);
    load_ascales<MT>(a, src, asc, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (nrec > 1) {
        dma_record<MT>(a, src, buf1, 1, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kRefill + kAct>();   // issued after buffer 0: the ring, then buffer 1
    } else {
        wait_vmcnt<kRefill>();
    }
    barrier_ds();

    // records r (buffer 0) and r + 1 (buffer 1) per trip; refills take
    // record r + 1 (the last record refills itself: the ring stays in one set
    // of registers); after each record, wait for the next buffer, barrier,
    // and load record r + 2 into the buffer just read
    for (int r = 0; r < nrec; r += 2) {
        mx_record<MT>(a, src, buf0, ring, asc, acc, r + 1 < nrec ? r + 1 : r, lane);
        if (r + 1 >= nrec) break;
        wait_vmcnt<kRefill>();   // record r + 1 has landed in buffer 1
        barrier_ds();            // every wavefront is done with buffer 0
        if (r + 2 < nrec) dma_record<MT>(a, src, buf0, r + 2, wave, lane);
        mx_record<MT>(a, src, buf1, ring, asc, acc, r + 2 < nrec ? r + 2 : r + 1, lane);
        if (r + 2 >= nrec) break;
        wait_vmcnt<kRefill>();   // record r + 2 has landed in buffer 0
        barrier_ds();            // buffer 1 is free
        if (r + 3 < nrec) dma_record<MT>(a, src, buf1, r + 3, wave, lane);
    }

    if (chunk < a.NC) store_tile<MT, kWPL>(a, p0, nrows, chunk, lane, acc);
}

template <int MT>
__device__ __forceinline__ void mx_tile_part(const GemmArgs& a, int e, int p0, int nrows, int chunk,
                                             int wave, int lane, u32x4* buf0, u32x4* buf1) {
    const int mt = (nrows + 15) >> 4;
    if (MT >= 4 && mt > 3)
        mx_tile<(MT >= 4 ? 4 : 1)>(a, e, p0, nrows, chunk, wave, lane, buf0, buf1);
    else if (MT >= 3 && mt == 3)
        mx_tile<(MT >= 3 ? 3 : 1)>(a, e, p0, nrows, chunk, wave, lane, buf0, buf1);
    else if (MT >= 2 && mt == 2)
        mx_tile<(MT >= 2 ? 2 : 1)>(a, e, p0, nrows, chunk, wave, lane, buf0, buf1);
    else
        mx_tile<1>(a, e, p0, nrows, chunk, wave, lane, buf0, buf1);
}

// Workgroup w runs items w, w + G, ... (G = the grid), an item being (tile,
// group of four chunks); the item decision is uniform across the workgroup,
// so every barrier inside is reached by all four wavefronts.  The LDS
// buffers are laid out for MT row blocks; a tile with fewer blocks uses a
// prefix of them.
template <int MT>
__device__ __forceinline__ void gemm_mx_body(const GemmArgs& a) {
    __shared__ u32x4 stage0[MxLds<MT>::frags];
    __shared__ u32x4 stage1[MxLds<MT>::frags];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int n_tiles = a.tile_src == TILE_TABLE ? a.tile_count[0] : a.ntp[0] / a.block_m;
    n_tiles = n_tiles < a.tiles_cap ? n_tiles : a.tiles_cap;
    const int qs = (a.NC + 3) / 4;
    const int64_t n_items = static_cast<int64_t>(n_tiles) * qs;
    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int ty = static_cast<int>(item / qs);
        const int quad = static_cast<int>(item % qs);
        int e, p0, nrows;
        if (a.tile_src == TILE_TABLE) {
            const int4 t = reinterpret_cast<const int4*>(a.tiles)[ty];
            e = t.x;
            p0 = t.y;
            nrows = t.z;
        } else {
            p0 = ty * a.block_m;
            e = a.expert_ids[ty];
            nrows = a.sorted_cap - p0 < a.block_m ? a.sorted_cap - p0 : a.block_m;
        }
        nrows = nrows < 16 * MT ? nrows : 16 * MT;
        if (e < 0 || e >= a.E || nrows <= 0) continue;
        mx_tile_part<MT>(a, e, p0, nrows, quad * 4 + wave, wave, lane, stage0, stage1);
        // the next item reuses the staging buffers: every wavefront's LDS
        // reads have completed.  The tile's global stores need not have (a
        // release fence here would wait for all of them before the next
        // item's loads could even be issued)
        barrier_ds();
    }
}

template <int MT>
__global__ void __launch_bounds__(256) k_gemm_mx(GemmArgs a) {
    gemm_mx_body<MT>(a);
}

template <int MT>
static int mx_resident() {
    static int cached = 0;
    if (cached <= 0) {
        int dev = 0, ncu = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            ncu = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemm_mx<MT>, 256, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cached = ncu * per_cu;
    }
    return cached;
}

template <int MT>
static void launch_mx_mt(const GemmArgs& a, hipStream_t st) {
    // one workgroup per item (the host's tile estimate) up to four rounds of
    // resident workgroups, else items dealt evenly to that many
    const int64_t cap = 4 * static_cast<int64_t>(mx_resident<MT>());
    const int64_t items = static_cast<int64_t>(a.grid_tiles) * ((a.NC + 3) / 4);
    const int64_t rounds = (items + cap - 1) / cap;
    const int64_t g = rounds > 0 ? (items + rounds - 1) / rounds : 1;
    k_gemm_mx<MT><<<dim3(static_cast<unsigned>(g < 1 ? 1 : g)), dim3(256), 0, st>>>(a);
}

}  // namespace

void launch_gemm_mx(const GemmArgs& a, int mt, hipStream_t st) {
    switch (mt) {
        case 1: launch_mx_mt<1>(a, st); break;
        case 2: launch_mx_mt<2>(a, st); break;
        case 3: launch_mx_mt<3>(a, st); break;
        default: launch_mx_mt<4>(a, st); break;
    }
}

}  // namespace w4a16
