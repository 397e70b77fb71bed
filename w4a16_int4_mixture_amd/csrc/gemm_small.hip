// Grouped W4A16 GEMM for few routed rows per expert (tiles of at most 16*MT
// rows): a weight-streaming kernel for CDNA4.
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
// CDNA4 design.  A workgroup is four wavefronts on four neighbouring packed
// chunks of CW output columns of one row tile, over one K range.
//   * Codes: every lane fetches its CW/16 words of a K group with 16-byte
//     non-temporal loads; the packed layout makes each wavefront's stream
//     contiguous.  A register ring keeps D groups of codes in flight (8 or
//     16 groups: 32 or 64 VGPRs), refilled as each group is consumed.
//   * Activations and scales are staged through LDS, one stage (8 groups)
//     ahead, double-buffered, one barrier per stage: each wavefront loads a
//     quarter of the stage's activation fragments (shared by all four) and
//     its own chunk's scales for the stage (one 16-byte load per lane), with
//     buffer loads that write LDS directly; the fragments are read back in
//     MFMA A-operand order (conflict-free).
//   * A code q becomes the bf16 value 128 + q by OR-ing the exponent pattern
//     0x43 above it, two codes per v_and_or_b32; v_mfma_f32_16x16x32_bf16 (K
//     = 32 = one scale group) yields sum x (128 + q); the offset -136 sum x is
//     produced once per row block by one MFMA against a constant operand and
//     fed in as the accumulator input, so the MFMA returns the exact group
//     partial sum x (q - 8); the fp32 group scale is applied with one FMA per
//     accumulator element.  Weights are never rounded.
//   * The loop is branch-free: K ranges are aligned to the end of the ring;
//     leading slots before the range re-read its first group with zeroed
//     scales (they add exactly zero).  A range of a single stage runs alone.

#include "combine_epi.h"
#include "device_common.h"
#include "internal.h"
#include "tile_store.h"

namespace w4a16 {

namespace {

using namespace dev;

constexpr int kSG = 8;  // groups of K per LDS stage

// (x & mask) | bits: mask and bits arrive as kernel arguments (bits pinned in
// a VGPR), so the compiler emits one v_and_or_b32 per bf16 pair.
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
    return (x & mask) | bits;
}

// B operand of one 16-column block: the word's eight codes as bf16 128 + q in
// MFMA K order (the packed nibble order 0,2,4,6,1,3,5,7 puts K offsets 2p and
// 2p+1 in the two 16-bit halves of (w >> 4p) & 0x000F000F).
__device__ inline bf16x8 codes_to_b(uint32_t w, uint32_t mask, uint32_t bits) {
    u32x4 d;
    d.x = and_or(w, mask, bits);
    d.y = and_or(w >> 4, mask, bits);
    d.z = and_or(w >> 8, mask, bits);
    d.w = and_or(w >> 12, mask, bits);
    return __builtin_bit_cast(bf16x8, d);
}

// B operand of one 16-column block from MXFP4 codes: byte b of the word holds
// the E2M1 codes of K offsets 2b (low nibble) and 2b + 1, which the hardware
// conversion turns into two exact bf16 values (scale operand 1).
__device__ inline bf16x8 codes_to_b_fp4(uint32_t w) {
    u32x4 d;
    d.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    d.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    d.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    d.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return __builtin_bit_cast(bf16x8, d);
}

// Codes of one K group for one lane.
template <int WPL>
struct Codes {
    u32x4 w[WPL / 4];
};

// Where one wavefront reads: its packed chunk, the activations, and this
// lane's byte offsets into them.
template <int MT>
struct Src {
    __amdgpu_buffer_rsrc_t w;  // the packed chunk (records of codes + scales)
    __amdgpu_buffer_rsrc_t x;  // activations [A_rows, K] bf16
    uint32_t code_off;         // lane * WPL words
    uint32_t a_off[MT];        // row of MFMA A row block t, K offset 8 * (lane / 16)
};

// Vector-memory instructions one wavefront issues per helper call.  The K
// loop's waits (s_waitcnt vmcnt) are written in these counts: completions of
// loads are counted in issue order, so "at most N outstanding" names exactly
// which batches have landed.
template <int WPL>
constexpr int kCodeLoads = WPL / 4;                       // load_codes: one K group
template <int MT, int WPL>
constexpr int kStageActLoads = (kSG / 4) * MT;            // dma_stage: activation fragments
template <int WPL>
constexpr int kStageScaleLoads = WPL / 4;                 // dma_stage: this wavefront's scales
template <int MT, int WPL>
constexpr int kStageLoads = kStageActLoads<MT, WPL> + kStageScaleLoads<WPL>;

// Codes of group ks (record ks / 8, slot ks % 8) for this lane; lane_off =
// lane * WPL words, in bytes; POL: the loads' cache policy.  Issues
// kCodeLoads<WPL> loads.
template <int WPL, int POL>
__device__ inline void load_codes(Codes<WPL>& c, __amdgpu_buffer_rsrc_t w, uint32_t lane_off,
                                  int ks) {
    const int soff = ((ks >> 3) * (576 * WPL) + (ks & 7) * (64 * WPL)) * 4;
    static_assert(sizeof(c.w) / sizeof(c.w[0]) == kCodeLoads<WPL>, "one load per 16 bytes");
#pragma unroll
    for (int i = 0; i < kCodeLoads<WPL>; ++i)
        c.w[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(w, lane_off + 16 * i, soff, POL));
}

// One K group is processed in three phases so that consecutive groups overlap:
//   prep : read the A fragments and scales from LDS, unpack the codes
//   mfma : offset MFMA, then one MFMA per 16-column block (C = offset)
//   fma  : acc += scale * partial
// The loop issues mfma(g), then prep(g + 1) while those MFMAs run, then fma(g).
template <int MT, int WPL>
struct Prep {
    bf16x8 b[WPL];
    float sc[WPL];
    u32x4 av[MT];
};

template <int MT, int WPL, bool FP4>
__device__ inline void prep_group(Prep<MT, WPL>& p, const Codes<WPL>& c, const u32x4* a_lds,
                                  const uint16_t* s_lds, uint32_t mask, uint32_t bits) {
#pragma unroll
    for (int t = 0; t < MT; ++t) p.av[t] = a_lds[t * 64];
    uint32_t sw[WPL / 2];
    if constexpr (WPL == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(s_lds);
        sw[0] = v.x;
        sw[1] = v.y;
    } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(s_lds);
        sw[0] = v.x;
        sw[1] = v.y;
        sw[2] = v.z;
        sw[3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < WPL / 4; ++i) {
        if constexpr (FP4) {
            p.b[4 * i + 0] = codes_to_b_fp4(c.w[i].x);
            p.b[4 * i + 1] = codes_to_b_fp4(c.w[i].y);
            p.b[4 * i + 2] = codes_to_b_fp4(c.w[i].z);
            p.b[4 * i + 3] = codes_to_b_fp4(c.w[i].w);
        } else {
            p.b[4 * i + 0] = codes_to_b(c.w[i].x, mask, bits);
            p.b[4 * i + 1] = codes_to_b(c.w[i].y, mask, bits);
            p.b[4 * i + 2] = codes_to_b(c.w[i].z, mask, bits);
            p.b[4 * i + 3] = codes_to_b(c.w[i].w, mask, bits);
        }
    }
#pragma unroll
    for (int i = 0; i < WPL / 2; ++i) {
        p.sc[2 * i] = __uint_as_float(sw[i] << 16);
        p.sc[2 * i + 1] = __uint_as_float(sw[i] & 0xFFFF0000u);
    }
}

// Orders the unpack of a ring slot before the load that refills it (the
// scheduler may otherwise sink the unpack below the load, after which old and
// new codes need separate registers and the loop ends in copies that wait for
// the newest loads).  Emits nothing.
template <int MT, int WPL>
__device__ inline void unpacked(const Prep<MT, WPL>& p) {
#pragma unroll
    for (int j = 0; j < WPL; ++j) asm volatile("" ::"v"(p.b[j]));
}

// FP4 (MXFP4 weights): the operand already holds the weight values, so the
// MFMA starts from zero instead of the -136 sum x offset.
template <int MT, int WPL, bool FP4>
__device__ inline void mfma_group(const Prep<MT, WPL>& p, f32x4 (&d)[MT][WPL]) {
    const bf16x8 c136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u,
                                                         0xC308C308u, 0xC308C308u});  // -136
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, p.av[t]);
        const f32x4 off =
            FP4 ? zero : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, c136, zero, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < WPL; ++j)
            d[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p.b[j], off, 0, 0, 0);
    }
}

template <int MT, int WPL>
__device__ inline void fma_group(const Prep<MT, WPL>& p, const f32x4 (&d)[MT][WPL],
                                 f32x4 (&acc)[MT][WPL]) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < WPL; ++j) acc[t][j] += p.sc[j] * d[t][j];
}

// The kSG groups of one LDS stage, software-pipelined.  `refill` = false in
// the ring's last turn.  ring[r0 + g] holds group g of the stage; after its
// unpack it is refilled with group `next + g`.
template <int MT, int WPL, int D, bool FP4, int POL>
__device__ inline void stage_groups(Codes<WPL> (&ring)[D], int r0, const u32x4* acur,
                                    const uint16_t* scur, const Src<MT>& src, int next,
                                    bool refill, f32x4 (&acc)[MT][WPL], uint32_t mask,
                                    uint32_t bits, int lane) {
    Prep<MT, WPL> pc, pn;
    prep_group<MT, WPL, FP4>(pc, ring[r0], acur + lane, scur, mask, bits);
    unpacked<MT, WPL>(pc);
    __builtin_amdgcn_sched_barrier(0);
    if (refill) load_codes<WPL, POL>(ring[r0], src.w, src.code_off, next);
#pragma unroll
    for (int g = 0; g < kSG; ++g) {
        f32x4 d[MT][WPL];
        mfma_group<MT, WPL, FP4>(pc, d);
        __builtin_amdgcn_sched_barrier(0);
        if (g + 1 < kSG) {
            prep_group<MT, WPL, FP4>(pn, ring[r0 + g + 1], acur + (g + 1) * MT * 64 + lane,
                                scur + (g + 1) * 16 * WPL, mask, bits);
            unpacked<MT, WPL>(pn);
            __builtin_amdgcn_sched_barrier(0);
            if (refill) load_codes<WPL, POL>(ring[r0 + g + 1], src.w, src.code_off, next + g + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        fma_group<MT, WPL>(pc, d, acc);
        __builtin_amdgcn_sched_barrier(0);
        if (g + 1 < kSG) pc = pn;
    }
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt left free).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier after this wavefront's LDS accesses have completed.  No
// fence: the staging buffers are written by buffer-to-LDS loads, whose
// completion each wavefront has waited for (vmcnt) before the barrier, and a
// fence would also wait for every code load in flight.
__device__ inline void barrier_ds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The stage starting at group `base` (a multiple of 8) goes straight into LDS
// buffer `buf` (activations, then the four wavefronts' scales) with buffer
// loads carrying the LDS bit; lane l of each load writes 16 bytes at l * 16.
// This wavefront loads the activation fragments of groups 4 i + wave and its
// own scales: kStageLoads<MT, WPL> loads.  A virtual stage (base < ks_min,
// ahead of the K range; only the first stage of a range can be one) reads the
// activations of group ks_min and writes zero scales instead of loading them
// (one LDS store per 16 bytes, so it issues kStageScaleLoads fewer loads; a
// wait written for the full count then waits at least as long); activation
// columns past K (padding groups, whose scales are zero) are clamped to the
// last real group.
// (D and POL, the caller's ring depth and code-load policy, only keep the
// instantiations of the kernel variants apart: the host compilation pass
// rejects one instantiation reached from several.)
template <int MT, int WPL, int MTMAX, int D, bool FP4, int POL, bool MAYBE_VIRTUAL = false>
__device__ inline void dma_stage(const Src<MT>& src, u32x4* buf, int base, int ks_min, int ks_real,
                                 int wave, int lane) {
    constexpr int kAStage = kSG * MTMAX * 64;   // u32x4 of activations per buffer
    static_assert((kSG / 4) * MT == kStageActLoads<MT, WPL>, "activation loads per stage");
#pragma unroll
    for (int i = 0; i < kSG / 4; ++i) {
        int g = base + 4 * i + wave;
        if (MAYBE_VIRTUAL) g = g < ks_min ? ks_min : g;
        g = g < ks_real ? g : ks_real - 1;
#pragma unroll
        for (int t = 0; t < MT; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src.x, LDS_PTR(buf + ((4 * i + wave) * MT + t) * 64),
                                                     16, src.a_off[t], g * 64, 0, 0);
    }
    // the record's scale block (8 groups x 16 x WPL bf16) follows its codes;
    // lane l takes 16-byte pieces l, 64 + l, ...
    u32x4* sb = buf + kAStage + wave * (WPL / 4 * 64);
    if (MAYBE_VIRTUAL && base < ks_min) {
#pragma unroll
        for (int v = 0; v < WPL / 4; ++v) sb[64 * v + lane] = u32x4{0u, 0u, 0u, 0u};
    } else {
        const int soff = ((base >> 3) * (576 * WPL) + 512 * WPL) * 4;
#pragma unroll
        for (int v = 0; v < kStageScaleLoads<WPL>; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src.w, LDS_PTR(sb + 64 * v), 16,
                                                     (64 * v + lane) * 16, soff, 0, 0);
    }
}

}  // namespace

// LDS per workgroup: two staging buffers, each the activation fragments of a
// stage [kSG][MT][64] x 16 B, then the scales [4 wavefronts][WPL/4 x 64] x
// 16 B.  The buffers are separate LDS objects, so that the compiler tells
// reads of one from buffer-to-LDS loads into the other.
template <int MT, int WPL>
struct Lds {
    static constexpr int a_stage = kSG * MT * 64;   // u32x4 per activation stage
    static constexpr int s_wave = WPL / 4 * 64;     // u32x4 per wavefront scale stage
    static constexpr int s_stage = 4 * s_wave;
    static constexpr int buf = a_stage + s_stage;   // u32x4 per buffer
};

struct Stg {
    u32x4* b[2];
};

// The K loop of one workgroup tile with MT active 16-row blocks (MTMAX sizes
// the LDS layout).
//
// Codes: a ring of D groups in registers, refilled as consumed: one stage (D
// = 8, the "wide" variants: the one- and two-block kernels then fit three
// workgroups on a CU, and a decode-sized grid runs in one round) or two
// stages (D = 16, the "deep" variants: more bytes in flight per wavefront,
// for grids that do not fill the machine with resident workgroups).
// Activation fragments and scales: two LDS buffers filled by buffer-to-LDS
// loads one stage ahead.  A stage ends with a wait for this wavefront's loads
// into the other buffer (vector-memory completions are counted in order, so
// the count is the stage's ring refills, which may stay in flight) and one
// barrier, after which the buffer just read is free for the stage after next.
//
// Iterations cover two stages (16 groups); the K range is padded at its start
// by one virtual record (zero scales) when it holds an odd number of records.
// Ring slot r0 + g of a stage holds its group g: r0 = 0 for the even stage,
// and for the odd one kSG (D = 16) or 0 (D = 8).
template <int MT, int WPL, int MTMAX, int D, bool FP4, int POL>
__device__ __forceinline__ void stream_loop(const Src<MT>& src, int ks0, int ks1, int ks_real,
                                            int wave, int lane, const Stg& stg,
                                            f32x4 (&acc)[MT][WPL], uint32_t mask,
                                            uint32_t bits) {
    static_assert(D == kSG || D == 2 * kSG, "a ring of one or two stages");
    constexpr int IT = 2 * kSG;                    // groups per iteration
    constexpr int RO = D == IT ? kSG : 0;          // ring slot of the odd stage's first group
    constexpr int kRefill = kSG * kCodeLoads<WPL>;  // code loads of one stage's refills
    constexpr int kStage = kStageLoads<MT, WPL>;     // staging loads per stage and wavefront
    constexpr int kRing = D * kCodeLoads<WPL>;       // code loads that fill the ring
    static_assert(kStage + kRing < 64 && kRefill < 64, "waits fit the 6-bit vmcnt field");
    using L = Lds<MTMAX, WPL>;
    if (ks1 <= ks0) return;
    const u32x4* abuf0 = stg.b[0];
    const u32x4* abuf1 = stg.b[1];
    // this lane's scales of group g in a stage: bf16 (16 g + lane % 16) * WPL
    const uint16_t* srd0 = reinterpret_cast<const uint16_t*>(stg.b[0] + L::a_stage + wave * L::s_wave) +
                           (lane & 15) * WPL;
    const uint16_t* srd1 = reinterpret_cast<const uint16_t*>(stg.b[1] + L::a_stage + wave * L::s_wave) +
                           (lane & 15) * WPL;

    // a K range of one stage (K = 256, or a split of one record) runs alone,
    // without the virtual stage that pads other odd stage counts
    if (ks1 - ks0 == kSG) {
        Codes<WPL> one[kSG];
        dma_stage<MT, WPL, MTMAX, D, FP4, POL>(src, stg.b[0], ks0, ks0, ks_real, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kSG; ++i) load_codes<WPL, POL>(one[i], src.w, src.code_off, ks0 + i);
        __builtin_amdgcn_sched_barrier(0);
        // issued: the stage's buffer, then kSG groups of codes (= kRefill
        // loads) that may stay in flight
        wait_vmcnt<kRefill>();                   // the stage's buffer has landed
        barrier_ds();
        stage_groups<MT, WPL, kSG, FP4, POL>(one, 0, abuf0, srd0, src, 0, false, acc, mask, bits, lane);
        return;
    }

    // ks0 and ks1 are multiples of 8: the ring starts pad (0 or 8) groups early
    // on a virtual record that adds zero
    const int pad = (IT - (ks1 - ks0) % IT) % IT;
    const int kb = ks0 - pad;
    const int nit = (ks1 - kb) / IT;            // iterations of two stages

    // buffer 1's loads after the ring's, as in the loop (where a stage's loads
    // follow the refills), so that the waits for ring slots match on both paths
    Codes<WPL> ring[D];
    dma_stage<MT, WPL, MTMAX, D, FP4, POL, true>(src, stg.b[0], kb, ks0, ks_real, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < D; ++i) load_codes<WPL, POL>(ring[i], src.w, src.code_off, kb + i < ks0 ? ks0 : kb + i);
    __builtin_amdgcn_sched_barrier(0);
    dma_stage<MT, WPL, MTMAX, D, FP4, POL>(src, stg.b[1], kb + kSG, ks0, ks_real, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
    // issued: buffer 0, the ring (kRing), buffer 1 (kStage); the last two may
    // stay in flight
    wait_vmcnt<kStage + kRing>();                // buffer 0 has landed
    barrier_ds();

    for (int it = 0; it < nit - 1; ++it) {
        const int base = kb + it * IT;
        // even stage: buffer 0; its ring slots take groups D ahead
        stage_groups<MT, WPL, D, FP4, POL>(ring, 0, abuf0, srd0, src, base + D, true, acc, mask, bits, lane);
        // issued since buffer 1's loads: this stage's ring refills (kRefill)
        wait_vmcnt<kRefill>();                   // buffer 1 has landed
        barrier_ds();                            // (for every wavefront); buffer 0 is free
        dma_stage<MT, WPL, MTMAX, D, FP4, POL>(src, stg.b[0], base + IT, ks0, ks_real, wave, lane);
        // odd stage: buffer 1
        stage_groups<MT, WPL, D, FP4, POL>(ring, RO, abuf1, srd1, src, base + D + kSG, true, acc, mask, bits,
                                 lane);
        // issued since buffer 0's loads: this stage's ring refills (kRefill)
        wait_vmcnt<kRefill>();                   // buffer 0 has landed
        barrier_ds();                            // buffer 1 is free
        dma_stage<MT, WPL, MTMAX, D, FP4, POL>(src, stg.b[1], base + IT + kSG, ks0, ks_real, wave, lane);
    }
    // last iteration: with a one-stage ring the even stage still refills it
    // with the odd stage's groups
    const int last = kb + (nit - 1) * IT;
    stage_groups<MT, WPL, D, FP4, POL>(ring, 0, abuf0, srd0, src, last + kSG, D < IT, acc, mask, bits, lane);
    // issued since buffer 1's loads: the refills of this stage, if any
    wait_vmcnt<(D < IT ? kRefill : 0)>();        // buffer 1 has landed
    barrier_ds();
    stage_groups<MT, WPL, D, FP4, POL>(ring, RO, abuf1, srd1, src, 0, false, acc, mask, bits, lane);
}

// Split-K fix-up.  Every split writes its fp32 partial of the tile part, then
// one thread counts the arrival; the split that arrives last re-reads the
// others' partials and adds all of them in split order (its own from
// registers), so the sum does not depend on which split came last.  The last
// one also resets the counter to zero for the next call.  Returns true in the
// last split's workgroup, with acc holding the full sum.  No workgroup waits
// for another one.
//
// Partials are stored and loaded with device-scope coherent accesses (the
// splits of a tile may run on different XCDs, whose L2 caches are separate),
// and each wavefront waits for its stores to complete before the arrival is
// counted.  Device-scope fences are avoided on purpose: they write back and
// invalidate the whole L2 of the XCD, which costs far more than the GEMM.
template <int MT, int WPL>
__device__ __forceinline__ bool splitk_fixup(const GemmArgs& a, int p0, int nrows, int chunk,
                                             int s, bool active, int lane, int32_t* counter,
                                             f32x4 (&acc)[MT][WPL]) {
    __shared__ int last_flag;
    // byte offsets inside one split's partial [rows, N]: a per-lane part and
    // a uniform part per (t, i, j); a split's partial is below 4 GiB (host check)
    const uint32_t voff =
        static_cast<uint32_t>((static_cast<int64_t>(p0 + 4 * (lane >> 4)) * a.N + chunk * a.CW +
                               (lane & 15)) * 4);
    const uint64_t split_bytes = static_cast<uint64_t>(a.ws_stride) * 4;
    if (active) {
        const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.partials + s * a.ws_stride, split_bytes);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (16 * t + 4 * (lane >> 4) + i >= nrows) continue;
#pragma unroll
                for (int j = 0; j < WPL; ++j)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[t][j][i]), ws, voff,
                                                          ((16 * t + i) * a.N + 16 * j) * 4,
                                                          kDeviceScope);
            }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's partial has reached memory
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = atomicAdd(counter, 1);
        const bool last = prev == a.split_k - 1;
        if (last) atomicExch(counter, 0);
        last_flag = last;
    }
    __syncthreads();
    const bool last = last_flag != 0;
    if (!last) return false;
    if (!active) return true;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (16 * t + 4 * (lane >> 4) + i >= nrows) continue;
#pragma unroll
            for (int j = 0; j < WPL; ++j) {
                const int soff = ((16 * t + i) * a.N + 16 * j) * 4;
                float v = 0.0f;
                for (int q = 0; q < a.split_k; ++q) {
                    float pq = acc[t][j][i];
                    if (q != s)
                        pq = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                            make_rsrc(a.partials + q * a.ws_stride, split_bytes), voff, soff,
                            kDeviceScope));
                    v = q == 0 ? pq : v + pq;
                }
                acc[t][j][i] = v;
            }
        }
    return true;
}

// Where the wavefront on `chunk` of a tile reads: the activation row of each
// of this lane's MFMA A rows (rows past the tile reuse its first row: MFMA
// rows are independent and are not stored) and the expert's packed chunk.  A
// wavefront past the last chunk re-streams the last chunk (cache hits, only
// when N / CW is not a multiple of 4) and stores nothing: the loop stays free
// of wavefront-dependent branches.
template <int MT, int WPL>
__device__ __forceinline__ Src<MT> make_src(const GemmArgs& a, int e, int p0, int nrows,
                                             int chunk, int lane) {
    const bool slot_rows = a.tile_src != TILE_MASKED;
    Src<MT> src;
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
        // A_rows * K * 2 < 2^32 is checked on the host
        src.a_off[t] = static_cast<uint32_t>(row * a.K * 2 + 16 * (lane >> 4));
    }
    src.x = make_rsrc(a.A, static_cast<uint64_t>(a.A_rows) * a.K * 2);
    const int64_t cbase = static_cast<int64_t>(e) * a.NC + (chunk < a.NC ? chunk : a.NC - 1);
    src.w = make_rsrc(a.packed + cbase * a.chunk_words, static_cast<uint64_t>(a.chunk_words) * 4);
    src.code_off = static_cast<uint32_t>(lane * WPL * 4);
    return src;
}

// One (row tile, 4 column chunks, K split) with MT active row blocks.
// `counter`: this tile's split-K arrival counter (split_k > 1).  Returns
// whether this workgroup stored the tile's outputs (false in a K split that
// did not arrive last); the value is the same in every thread.
template <int MT, int WPL, int MTMAX, int D, bool FP4, int POL>
__device__ __forceinline__ bool gemm_tile_mt(const GemmArgs& a, int e, int p0, int nrows,
                                             int chunk, int s, int wave, int lane, const Stg& stg,
                                             int32_t* counter) {
    const bool active = chunk < a.NC;
    const Src<MT> src = make_src<MT, WPL>(a, e, p0, nrows, chunk, lane);

    // K split s covers whole records [ks0, ks1)
    const int nrec = a.KSP / 8;
    const int ks0 = 8 * static_cast<int>(static_cast<int64_t>(s) * nrec / a.split_k);
    const int ks1 = 8 * static_cast<int>(static_cast<int64_t>(s + 1) * nrec / a.split_k);

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
    stream_loop<MT, WPL, MTMAX, D, FP4, POL>(src, ks0, ks1, a.KS, wave, lane, stg, acc, a.unpack_mask, vbits);

    if (a.split_k > 1 && !splitk_fixup<MT, WPL>(a, p0, nrows, chunk, s, active, lane, counter, acc))
        return false;
    if (active) store_tile<MT, WPL>(a, p0, nrows, chunk, lane, acc);
    return true;
}

template <int MT, int WPL, int D, bool FP4, int POL>
__device__ __forceinline__ bool gemm_tile_part(const GemmArgs& a, int e, int p0, int nrows,
                                               int chunk, int s, int wave, int lane, const Stg& stg,
                                               int32_t* counter) {
    const int mt_active = (nrows + 15) >> 4;
    if (mt_active <= 1)
        return gemm_tile_mt<1, WPL, MT, D, FP4, POL>(a, e, p0, nrows, chunk, s, wave, lane, stg, counter);
    else if (MT >= 2 && mt_active == 2)
        return gemm_tile_mt<(MT >= 2 ? 2 : 1), WPL, MT, D, FP4, POL>(a, e, p0, nrows, chunk, s, wave, lane, stg,
                                                        counter);
    else if (MT >= 3 && mt_active == 3)
        return gemm_tile_mt<(MT >= 3 ? 3 : 1), WPL, MT, D, FP4, POL>(a, e, p0, nrows, chunk, s, wave, lane, stg,
                                                        counter);
    else
        return gemm_tile_mt<(MT >= 4 ? 4 : 1), WPL, MT, D, FP4, POL>(a, e, p0, nrows, chunk, s, wave, lane, stg,
                                                        counter);
}

// One tile of at most 16 * MT rows: `quad` is its group of four chunks (256
// columns), `s` its K split; the split-K arrival counter is the (tile, quad)
// one.  With the fused combine, the workgroup that stored the tile's rows
// then counts their tokens' arrivals (s_tok, s_n: LDS scratch).
template <int MT, int WPL, int D, bool FP4, int POL>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int ty, int e, int p0, int nrows,
                                          int quad, int s, int wave, int lane, const Stg& stg,
                                          int* s_tok, int* s_n) {
    const int nquads = (a.NC + 3) / 4;
    int32_t* counter = a.counters + static_cast<int64_t>(ty) * nquads + quad;
    const bool stored =
        gemm_tile_part<MT, WPL, D, FP4, POL>(a, e, p0, nrows, quad * 4 + wave, s, wave, lane, stg, counter);
    static_assert(4 * 64 == 256, "a quad of chunks is one 256-column combine group");
    if (a.comb_out && stored) comb_arrive(a, p0, nrows, quad, s_tok, s_n);
}

// Masked layout: the tiles that hold rows, in expert order.  Expert g holds
// ceil(c / tile_m) of them, c = min(masked_m[g], max_m) (a negative count is
// none).  Every wavefront scans the counts itself, 64 experts per step, so
// the results are uniform without a barrier.  Work items walk the non-empty
// tiles only: a launch's items past them are all at its end, and no empty
// (expert, chunk) slot delays the start of a real one.
__device__ inline int masked_rows_of(const GemmArgs& a, const int32_t* mm, int g) {
    if (g >= a.E) return 0;
    const int m = mm[g];
    return m < 0 ? 0 : (m < a.max_m ? m : a.max_m);
}

__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

__device__ inline int masked_tile_count(const GemmArgs& a, int lane) {
    int total = 0;
    for (int g0 = 0; g0 < a.E; g0 += 64) {
        const int t = (masked_rows_of(a, a.masked_m, g0 + lane) + a.tile_m - 1) / a.tile_m;
        total += __builtin_amdgcn_readlane(wave_incl_scan(t, lane), 63);
    }
    return total;
}

// Expert and rows of non-empty tile ty; e = -1 past the last one.  The
// counts are read again for every tile (the empty asm hides that they do not
// change), so that no per-lane scan value is kept live across the K loop.
__device__ inline void masked_tile_at(const GemmArgs& a, int ty, int lane, int& e, int& p0,
                                      int& nrows) {
    const int32_t* mm = a.masked_m;
    asm volatile("" : "+s"(mm));
    int base = 0;
    for (int g0 = 0; g0 < a.E; g0 += 64) {
        const int c = masked_rows_of(a, mm, g0 + lane);
        const int t = (c + a.tile_m - 1) / a.tile_m;
        const int incl = wave_incl_scan(t, lane);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (ty < base + total) {
            const int L = static_cast<int>(__builtin_ctzll(__ballot(base + incl > ty)));
            const int first = base + __builtin_amdgcn_readlane(incl - t, L);
            const int cnt = __builtin_amdgcn_readlane(c, L);
            const int r0 = (ty - first) * a.tile_m;
            e = g0 + L;
            p0 = e * a.max_m + r0;
            nrows = cnt - r0 < a.tile_m ? cnt - r0 : a.tile_m;
            return;
        }
        base += total;
    }
    e = -1;
    p0 = 0;
    nrows = 0;
}

// Cache policy of the code loads.  Non-temporal in general: one tile per
// expert streams the weights once.  The masked layout cuts an expert above
// the tile height into several tiles; their items (same column group and K
// split, a multiple of 8 apart in the grid) run on one XCD at the same time,
// so its code lines are kept in that XCD's L2 for the other tiles.
template <bool MK>
constexpr int kCodePolicy = MK ? 0 : kNonTemporal;

// Workgroup w runs work items w, w + G, ... (G = the grid), an item being
// (tile, group of four chunks, K split), splits of one chunk group adjacent;
// the loop covers any device-side tile count whatever the grid.  The item
// decision is uniform across the workgroup, so every barrier inside is
// reached by all four wavefronts.  D: groups of the code ring (8 or 16).  MK:
// the masked layout (its own instantiation, so that the tile scan's registers
// do not weigh on the other layouts' kernels).
template <int MT, int WPL, int D, bool FP4, bool MK>
__device__ __forceinline__ void gemm_small_body(const GemmArgs& a) {
    __shared__ u32x4 stage0[Lds<MT, WPL>::buf];
    __shared__ u32x4 stage1[Lds<MT, WPL>::buf];
    __shared__ int s_tok[16 * MT];
    __shared__ int s_n;
    Stg stg;
    stg.b[0] = stage0;
    stg.b[1] = stage1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (a.comb_out) comb_zero_unrouted(a);
    int n_tiles;
    if constexpr (MK) {
        n_tiles = masked_tile_count(a, lane);
    } else if (a.tile_src == TILE_TABLE) {
        n_tiles = a.tile_count[0];
    } else {
        n_tiles = a.ntp[0] / a.block_m;
    }
    n_tiles = n_tiles < a.tiles_cap ? n_tiles : a.tiles_cap;
    const int qs = ((a.NC + 3) / 4) * a.split_k;   // items per tile
    const int64_t n_items = static_cast<int64_t>(n_tiles) * qs;
    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int ty = static_cast<int>(item / qs);
        const int rem = static_cast<int>(item % qs);
        const int quad = rem / a.split_k, s = rem % a.split_k;
        int e, p0, nrows;
        if constexpr (MK) {
            // masked_m is the valid count of each expert; a count above max_m
            // is cut to max_m, so no tile reaches past the expert's rows
            masked_tile_at(a, ty, lane, e, p0, nrows);
        } else if (a.tile_src == TILE_TABLE) {
            const int4 t = reinterpret_cast<const int4*>(a.tiles)[ty];
            e = t.x;
            p0 = t.y;
            nrows = t.z;
        } else {
            p0 = ty * a.block_m;
            e = a.expert_ids[ty];
            nrows = a.sorted_cap - p0 < a.block_m ? a.sorted_cap - p0 : a.block_m;
        }
        // a tile-table entry taller than the launch's tile height (a table
        // written for another tile_m) is cut to it: its rows past 16 * MT are
        // not computed, and nothing is stored outside the tile
        nrows = nrows < 16 * MT ? nrows : 16 * MT;
        if (e < 0 || e >= a.E || nrows <= 0) continue;
        gemm_tile<MT, WPL, D, FP4, kCodePolicy<MK>>(a, ty, e, p0, nrows, quad, s, wave, lane, stg, s_tok,
                                                    &s_n);
        // the next item reuses the staging buffers: every wavefront's LDS
        // reads have completed.  The tile's global stores need not have (a
        // release fence here would wait for all of them before the next
        // item's loads could even be issued)
        barrier_ds();
    }
}

template <int MT, int WPL, int D, bool FP4, bool MK>
__global__ void __launch_bounds__(256) k_gemm_small(GemmArgs a) {
    gemm_small_body<MT, WPL, D, FP4, MK>(a);
}

// The two-block kernel with the one-stage ring, held to three workgroups per
// CU (168 VGPRs: four registers are kept in scratch across the K loop, none
// inside it).
template <int MT, int WPL, int D, bool FP4, bool MK>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8)))
    k_gemm_small_w3(GemmArgs a) {
    gemm_small_body<MT, WPL, D, FP4, MK>(a);
}

template <int MT, int D, bool FP4, bool MK>
static void (*small_kernel())(GemmArgs) {
    if constexpr (MT == 2 && D == 8)
        return k_gemm_small_w3<MT, 4, D, FP4, MK>;
    else
        return k_gemm_small<MT, 4, D, FP4, MK>;
}

// Workgroups of one kernel variant resident on the device at once (from the
// runtime's occupancy calculation: registers and LDS), cached per variant.
static int g_resident[5][2][2][2] = {};

static int resident_of(void (*kern)(GemmArgs), int& cached) {
    if (cached <= 0) {
        int dev = 0, ncu = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            ncu = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cached = ncu * per_cu;
    }
    return cached;
}

template <int MT, int D, bool FP4, bool MK>
static int resident_wgs() {
    return resident_of(small_kernel<MT, D, FP4, MK>(),
                       g_resident[MT][D == 8 ? 0 : 1][FP4 ? 1 : 0][MK ? 1 : 0]);
}

template <int MT, int D, bool FP4, bool MK>
static void launch_mt(const GemmArgs& a, hipStream_t st) {
    const int64_t items = static_cast<int64_t>(a.grid_tiles) * ((a.NC + 3) / 4) * a.split_k;
    // One workgroup per item (from the host's tile estimate) while they fit
    // in four rounds of resident workgroups: the hardware then hands items to
    // CUs as they free up, which balances items of unequal cost.  Beyond
    // that, items are dealt evenly to that many workgroups, which saves the
    // start-up of very short items (short K).  The masked layout's count is
    // the worst case (every expert at max_m) and its items walk the non-empty
    // tiles only, so one round of resident workgroups is launched: the items
    // past the filled tiles then cost no dispatch after the real ones.
    const int64_t resident = resident_wgs<MT, D, FP4, MK>();
    const int64_t cap = MK ? resident : 4 * resident;
    const int64_t rounds = (items + cap - 1) / cap;
    const int64_t g = rounds > 0 ? (items + rounds - 1) / rounds : 1;
    small_kernel<MT, D, FP4, MK>()<<<dim3(static_cast<unsigned>(g < 1 ? 1 : g)), dim3(256), 0, st>>>(
        a);
}

template <bool FP4, bool MK>
static void launch_variant(const GemmArgs& a, int mt, bool wide, hipStream_t st) {
    switch (mt) {
        case 1: launch_mt<1, 8, FP4, MK>(a, st); break;
        case 2:
            if (wide)
                launch_mt<2, 8, FP4, MK>(a, st);
            else
                launch_mt<2, 16, FP4, MK>(a, st);
            break;
        case 3: launch_mt<3, 16, FP4, MK>(a, st); break;
        default: launch_mt<4, 16, FP4, MK>(a, st); break;
    }
}

void launch_gemm_small(const GemmArgs& a, int mt, bool wide, hipStream_t st) {
    const bool mk = a.tile_src == TILE_MASKED;
    if (a.fp4)
        mk ? launch_variant<true, true>(a, mt, wide, st) : launch_variant<true, false>(a, mt, wide, st);
    else
        mk ? launch_variant<false, true>(a, mt, wide, st)
           : launch_variant<false, false>(a, mt, wide, st);
}

}  // namespace w4a16
