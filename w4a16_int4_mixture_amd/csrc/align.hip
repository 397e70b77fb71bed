// Routing metadata for the indexed layout: a stable counting sort of routed
// slots by local expert, padded per expert to a multiple of block_m.
//
// Chord page, "Two kernel families": the indexed family consumes vLLM's
// sorted_ids / expert_ids / num_tokens_padded; "vLLM integration": these
// buffers are over-allocated and consumed without a host read-back, so the
// path stays graph-capturable; Figure 3: activations are not padded, the
// routing indices carry the padding sentinels.
//
// B workgroups of W wavefronts; workgroup b owns a contiguous range of
// 64-slot chunks (flat slot f = t*k + j, ascending), wavefront w a contiguous
// piece of it.
//   pass 0: every workgroup counts the local slots of each expert over all
//           slots, and separately those before its own range (LDS atomics:
//           counts do not depend on order); so every workgroup derives the
//           same padded offsets, and its own bases, without exchanging
//           anything with the others
//   pass 1: per (wave, expert) counts over the workgroup's range
//   pass 2: padded offsets (wave prefix scan), per-wave bases; workgroup 0
//           writes expert_ids, padding sentinels, the GEMM tile table and
//           the counts, all workgroups the tails
//   pass 3: scatter each local slot to base + rank, record row_of
// In passes 1 and 3, for one chunk, lane l holds slot f = 64*c + l and sets
// bit l of mask[w][e] (64-bit LDS OR) for its local expert e.  Then
// popcount(mask[w][e]) counts the chunk's slots of expert e and
// popcount(mask[w][e] & lanes_below_l) is the rank of lane l's slot among
// them: both are independent of the order in which the ORs land, so the sort
// is stable and bit-reproducible without ordered atomics.

#include "internal.h"

namespace w4a16 {

namespace {

__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Chunks of 64 slots whose routing ids one wavefront loads at once.
constexpr int kBatch = 16;
// Largest expert map kept in LDS.
constexpr int kMapLds = 4096;

// Routing ids of slots c0*64 + lane .. for kBatch chunks (0 past the end),
// all loads issued at once.
__device__ inline void load_ids(const AlignArgs& a, int64_t c0, int64_t c_end, int64_t S, int lane,
                                int (&g)[kBatch]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const int64_t f = (c0 + j) * 64 + lane;
        g[j] = (c0 + j < c_end && f < S) ? a.topk_ids[f] : 0;
    }
}

// An expert map as the lookup sees it: one contiguous range (local e = g -
// base for g in [base, base + E_local), -1 elsewhere; the usual
// expert-parallel share, or the identity) is looked up by arithmetic;
// otherwise lmap is the map cached in LDS, or null (then read from global
// memory).
struct MapView {
    const int* lmap;
    int base;
    bool range;
};

// Local experts of those slots (-1: none or past the end).
__device__ inline void map_ids(const AlignArgs& a, const MapView& m, int64_t c0, int64_t c_end,
                               int64_t S, int lane, const int (&g)[kBatch], int (&eb)[kBatch],
                               int* bad) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const int64_t f = (c0 + j) * 64 + lane;
        int e = -1;
        if (c0 + j < c_end && f < S) {
            if (g[j] < 0 || g[j] >= a.E_global) {
                *bad = 1;
            } else if (m.range) {
                e = (g[j] >= m.base && g[j] - m.base < a.E_local) ? g[j] - m.base : -1;
            } else {
                e = m.lmap ? m.lmap[g[j]] : a.expert_map ? a.expert_map[g[j]] : g[j];
                if (e < -1 || e >= a.E_local) *bad = 1;
                if (e < 0 || e >= a.E_local) e = -1;
            }
        }
        eb[j] = e;
    }
}

__device__ inline void load_batch(const AlignArgs& a, const MapView& m, int64_t c0, int64_t c_end,
                                  int64_t S, int lane, int (&eb)[kBatch], int* bad) {
    int g[kBatch];
    load_ids(a, c0, c_end, S, lane, g);
    map_ids(a, m, c0, c_end, S, lane, g, eb, bad);
}

// In-place exclusive prefix sums of v[0..n) and u[0..n) by one wavefront,
// totals in tv and tu.  Lane l first sums its own run of ceil(n / 64)
// entries, so that one 64-lane scan serves any n.
__device__ void wave_exclusive_scan2(int* v, int* u, int n, int lane, int& tv, int& tu) {
    const int per = (n + 63) / 64;
    const int lo = lane * per < n ? lane * per : n;
    const int hi = lo + per < n ? lo + per : n;
    int sv = 0, su = 0;
    for (int i = lo; i < hi; ++i) {
        sv += v[i];
        su += u[i];
    }
    int iv = sv, iu = su;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int yv = __shfl_up(iv, d, 64);
        const int yu = __shfl_up(iu, d, 64);
        if (lane >= d) {
            iv += yv;
            iu += yu;
        }
    }
    int ev = iv - sv, eu = iu - su;
    for (int i = lo; i < hi; ++i) {
        const int x = v[i], y = u[i];
        v[i] = ev;
        u[i] = eu;
        ev += x;
        eu += y;
    }
    tv = __shfl(iv, 63, 64);
    tu = __shfl(iu, 63, 64);
}

// Workgroup barrier for LDS data: this wavefront's LDS accesses have
// completed; its global stores may still be in flight (nothing in this
// kernel reads back what another wavefront stored to global memory, except
// after the fused router, which uses a full barrier).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Most wavefronts of a workgroup: k_align's launch bound is 64 * kMaxWaves
// threads, and align_waves never asks for more.
constexpr int kMaxWaves = 16;

// ---- router top-k ------------------------------------------------------------
//
// One wavefront per token: lane l holds the logits of experts l, l + 64, ...
// (at most kRouterPerLane).  k rounds: each lane offers its best remaining
// expert (largest logit, lower id on equal logits), the wavefront reduces the
// 64 offers with the same order, and the owner of the winner marks it taken.
// Then weight j = e^(l_j - l_0) / sum_i e^(l_i - l_0) over the k winners, in
// fp32, summed in j order.
constexpr int kRouterPerLane = 16;   // E_global <= 1024
static_assert(64 * kRouterPerLane == kRouterMaxExperts, "16 logits per lane");

__device__ inline bool router_better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__device__ inline void router_token(const float* logits, int E, int k, int t, int lane,
                                    int32_t* ids_out, float* w_out) {
    float v[kRouterPerLane];
    const float* l = logits + static_cast<int64_t>(t) * E;
#pragma unroll
    for (int i = 0; i < kRouterPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? l[e] : -__builtin_inff();
    }
    uint32_t taken = 0;   // bit i: expert lane + 64 i already selected (or absent)
#pragma unroll
    for (int i = 0; i < kRouterPerLane; ++i)
        if (lane + 64 * i >= E) taken |= 1u << i;
    float top = 0.f, den = 0.f, my_val = 0.f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < kRouterPerLane; ++i) {
            if (taken & (1u << i)) continue;
            if (router_better(v[i], lane + 64 * i, bv, bi)) {
                bv = v[i];
                bi = lane + 64 * i;
            }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const float ov = __shfl_xor(bv, d, 64);
            const int oi = __shfl_xor(bi, d, 64);
            if (router_better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        // every lane now holds the winner (bv, bi)
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (j == 0) top = bv;
        const float ex = expf(bv - top);
        den = j == 0 ? ex : den + ex;
        if (lane == j) {
            my_val = ex;
            my_id = bi;
        }
    }
    if (lane < k) {
        ids_out[static_cast<int64_t>(t) * k + lane] = my_id;
        w_out[static_cast<int64_t>(t) * k + lane] = my_val / den;
    }
}

}  // namespace

// Router top-k alone: one wavefront per token, four per workgroup.
__global__ void __launch_bounds__(256) k_router_topk(const float* __restrict__ logits, int T, int E,
                                                     int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < T) router_token(logits, E, k, t, lane, ids, w);
}

void launch_router_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
    if (T > 0) k_router_topk<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(logits, T, E, k, ids, w);
}

__global__ void __launch_bounds__(64 * kMaxWaves) k_align(AlignArgs a) {
    extern __shared__ unsigned char smem[];
    const int E = a.E_local;
    const int W = blockDim.x / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    uint64_t* masks = reinterpret_cast<uint64_t*>(smem);          // [W][E]
    int* cnt = reinterpret_cast<int*>(masks + W * E);             // [W][E] counts, then bases
    int* pad = cnt + W * E;                                       // [E] padded counts -> offsets
    int* ntile = pad + E;                                         // [E] tiles -> tile offsets
    int* tot = ntile + E;                                         // [E] slot counts
    int* pre = tot + E;                                           // [E] counts before this range
    int* red = pre + E;                                           // [4] totals
    uint64_t* my_mask = masks + w * E;
    int* my_cnt = cnt + w * E;

    const int64_t S = static_cast<int64_t>(a.T) * a.top_k;
    const int32_t sentinel = static_cast<int32_t>(S);
    const int64_t chunks = (S + 63) / 64;
    // this workgroup's chunks, then this wave's part of them
    const int64_t cpb = (chunks + gridDim.x - 1) / gridDim.x;
    const int64_t b_begin = blockIdx.x * cpb < chunks ? blockIdx.x * cpb : chunks;
    const int64_t b_end = b_begin + cpb < chunks ? b_begin + cpb : chunks;
    const int64_t cpw = (b_end - b_begin + W - 1) / W;
    const int64_t c_begin = b_begin + w * cpw < b_end ? b_begin + w * cpw : b_end;
    const int64_t c_end = c_begin + cpw < b_end ? c_begin + cpw : b_end;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int bad = 0;

    // ---- fused router (one-workgroup launches only): wavefront w takes the
    // top-k of tokens w, w + W, ...; the ids it writes are read back below
    // by every wavefront of this workgroup
    if (a.logits) {
        for (int t = w; t < a.T; t += W)
            router_token(a.logits, a.E_global, a.top_k, t, lane, a.ids_out, a.weights_out);
        __threadfence_block();
        __syncthreads();
    }

    // ---- pass 0: per-expert counts of the slots before the range (pre)
    // and of the others (tot; pass 2 adds pre to it).  The expert map is
    // cached in LDS (when it fits); the routing ids are read 16 bytes at a
    // time, all of a thread's loads issued first, then all its map lookups,
    // then one LDS atomic per local slot.
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        tot[e] = 0;
        pre[e] = 0;
    }
    int* lmap = red + 4;                                          // [E_global] if cached
    const bool map_lds = a.E_global <= kMapLds;
    if (threadIdx.x == 0) {
        red[2] = a.E_global;
        red[3] = 1;
    }
    if (map_lds)
        for (int i = threadIdx.x; i < a.E_global; i += blockDim.x)
            lmap[i] = a.expert_map ? a.expert_map[i] : i;
    lds_barrier();
    // Is the cached map one contiguous range?  base = the global id of local
    // expert 0; then every entry is checked against g - base or -1, so the
    // arithmetic lookup gives exactly the map's values for every valid id.
    // (Only where every workgroup counts all slots: a one-workgroup sort
    // looks up too few ids to pay for the check's two barriers.)
    const bool multi = gridDim.x > 1;
    if (map_lds && multi) {
        for (int i = threadIdx.x; i < a.E_global; i += blockDim.x)
            if (lmap[i] == 0) atomicMin(&red[2], i);
        lds_barrier();
        const int base = red[2];
        for (int i = threadIdx.x; i < a.E_global; i += blockDim.x) {
            const int want = (i >= base && i - base < E) ? i - base : -1;
            if (lmap[i] != want) red[3] = 0;                  // (all writers store 0)
        }
        lds_barrier();
    }
    MapView mv;
    mv.base = __builtin_amdgcn_readfirstlane(red[2]);
    mv.range = map_lds && multi && mv.base < a.E_global &&
               __builtin_amdgcn_readfirstlane(red[3]) != 0;
    mv.lmap = map_lds ? lmap : nullptr;
    auto local_of = [&](int g) {
        if (g < 0 || g >= a.E_global) {
            bad = 1;
            return -1;
        }
        if (mv.range) return (g >= mv.base && g - mv.base < E) ? g - mv.base : -1;
        int e = map_lds ? lmap[g] : (a.expert_map ? a.expert_map[g] : g);
        if (e < -1 || e >= E) bad = 1;
        return (e >= 0 && e < E) ? e : -1;
    };
    const int64_t pre_end = b_begin * 64;                         // slots before the range
    const bool vec = (reinterpret_cast<uintptr_t>(a.topk_ids) & 15) == 0;
    // (a single workgroup takes its totals from pass 1 instead)
    const int64_t n4 = multi && vec ? S / 4 : 0;                  // 4-id groups read as int4
    for (int64_t i0 = threadIdx.x; i0 < n4; i0 += static_cast<int64_t>(blockDim.x) * kBatch) {
        int4 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + static_cast<int64_t>(j) * blockDim.x;
            v[j] = i < n4 ? reinterpret_cast<const int4*>(a.topk_ids)[i] : int4{-1, -1, -1, -1};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + static_cast<int64_t>(j) * blockDim.x;
            if (i < n4) {
                v[j].x = local_of(v[j].x);
                v[j].y = local_of(v[j].y);
                v[j].z = local_of(v[j].z);
                v[j].w = local_of(v[j].w);
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + static_cast<int64_t>(j) * blockDim.x;
            if (i >= n4) break;
            const int es[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = es[q];
                if (e < 0) continue;
                atomicAdd(4 * i + q < pre_end ? &pre[e] : &tot[e], 1);
            }
        }
    }
    for (int64_t f = 4 * n4 + threadIdx.x; multi && f < S; f += blockDim.x) {
        const int e = local_of(a.topk_ids[f]);
        if (e < 0) continue;
        atomicAdd(f < pre_end ? &pre[e] : &tot[e], 1);
    }
    // one workgroup reports out-of-range ids
    if (multi && bad && a.err_flag && blockIdx.x == 0) atomicAdd(a.err_flag, 1);
    bad = 0;
    lds_barrier();

    // ---- pass 1: counts per (wave, expert).  The routing ids of kBatch
    // chunks are loaded together, so that one memory latency covers them;
    // when one batch covers all of this wave's chunks, pass 3 reuses it.
    const bool one_batch = c_end - c_begin <= kBatch;
    int kept[kBatch];
    for (int e = lane; e < E; e += 64) my_cnt[e] = 0;
    for (int64_t c0 = c_begin; c0 < c_end; c0 += kBatch) {
        int eb[kBatch];
        load_batch(a, mv, c0, c_end, S, lane, eb, &bad);
        if (one_batch) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) kept[j] = eb[j];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (c0 + j >= c_end) break;
            for (int e = lane; e < E; e += 64) my_mask[e] = 0;
            wave_sync();
            if (eb[j] >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&my_mask[eb[j]]), 1ull << lane);
            wave_sync();
            for (int ee = lane; ee < E; ee += 64) my_cnt[ee] += __popcll(my_mask[ee]);
            wave_sync();
        }
    }
    if (!multi && bad && a.err_flag) atomicAdd(a.err_flag, 1);
    lds_barrier();

    // ---- pass 2: offsets, metadata
    const int bm = a.block_m;
    const int tm = a.r.tile_m > 0 ? a.r.tile_m : 1;
    // (the W per-wave counts of an expert are read at once, then written)
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c;
        if (!multi) {
            int cw[kMaxWaves];
#pragma unroll
            for (int ww = 0; ww < kMaxWaves; ++ww) cw[ww] = ww < W ? cnt[ww * E + e] : 0;
            c = 0;
#pragma unroll
            for (int ww = 0; ww < kMaxWaves; ++ww) c += cw[ww];
        } else {
            c = tot[e] + pre[e];
        }
        tot[e] = c;
        pad[e] = (c + bm - 1) / bm * bm;
        ntile[e] = (c + tm - 1) / tm;
    }
    lds_barrier();
    if (w == 0) {
        int total, ntiles;
        wave_exclusive_scan2(pad, ntile, E, lane, total, ntiles);
        if (lane == 0) {
            red[0] = total;
            red[1] = ntiles;
        }
    }
    lds_barrier();
    const int total = red[0];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int off = pad[e];
        int run = off + pre[e];
        int cw[kMaxWaves];
#pragma unroll
        for (int ww = 0; ww < kMaxWaves; ++ww) cw[ww] = ww < W ? cnt[ww * E + e] : 0;
#pragma unroll
        for (int ww = 0; ww < kMaxWaves; ++ww) {
            if (ww < W) cnt[ww * E + e] = run;
            run += cw[ww];
        }
        if (blockIdx.x != 0) continue;
        const int c = tot[e];
        const int p = (c + bm - 1) / bm * bm;
        for (int j = c; j < p; ++j) a.r.sorted_ids[off + j] = sentinel;
        for (int b = 0; b < p / bm; ++b) a.r.expert_ids[off / bm + b] = e;
        if (a.r.tiles) {
            const int t0 = ntile[e];
            for (int i = 0; i * tm < c; ++i) {
                int4 v;
                v.x = e;
                v.y = off + i * tm;
                v.z = (c - i * tm) < tm ? (c - i * tm) : tm;
                v.w = 0;
                reinterpret_cast<int4*>(a.r.tiles)[t0 + i] = v;
            }
        }
    }
    if (blockIdx.x == 0 && a.r.expert_offsets)
        for (int e = threadIdx.x; e <= E; e += blockDim.x)
            a.r.expert_offsets[e] = e < E ? pad[e] : total;
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        a.r.num_tokens_padded[0] = total;
        if (a.r.tiles) a.r.tile_count[0] = red[1];
    }
    const int64_t gtid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t gsize = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = total + gtid; i < a.r.sorted_cap; i += gsize) a.r.sorted_ids[i] = sentinel;
    for (int64_t b = total / bm + gtid; b < a.r.blocks_cap; b += gsize) a.r.expert_ids[b] = -1;
    // (pass 3 stores only to positions that pass 2 does not write)
    lds_barrier();

    // ---- pass 3: scatter
    for (int64_t c0 = c_begin; c0 < c_end; c0 += kBatch) {
        int eb[kBatch];
        if (one_batch) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) eb[j] = kept[j];
        } else {
            load_batch(a, mv, c0, c_end, S, lane, eb, &bad);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (c0 + j >= c_end) break;
            for (int e = lane; e < E; e += 64) my_mask[e] = 0;
            wave_sync();
            const int e = eb[j];
            const int64_t f = (c0 + j) * 64 + lane;
            if (e >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&my_mask[e]), 1ull << lane);
            wave_sync();
            if (f < S) {
                int pos = -1;
                if (e >= 0) {
                    pos = my_cnt[e] + __popcll(my_mask[e] & below);
                    a.r.sorted_ids[pos] = static_cast<int32_t>(f);
                }
                if (a.r.row_of) a.r.row_of[f] = pos;
            }
            wave_sync();
            for (int ee = lane; ee < E; ee += 64) my_cnt[ee] += __popcll(my_mask[ee]);
            wave_sync();
        }
    }
}

int align_waves(int E_local) {
    // keep the LDS footprint (12 bytes per wave and expert) under 60 KiB
    int w = kMaxWaves;
    // (plus 16 per expert and the cached expert map, at most 16 KiB)
    while (w > 1 && static_cast<int64_t>(w) * E_local * 12 + E_local * 16 + 64 + 4 * kMapLds >
                        60 * 1024)
        w >>= 1;
    return w;
}

size_t align_lds_bytes(int W, int E_local, int E_global) {
    return static_cast<size_t>(W) * E_local * 12 + static_cast<size_t>(E_local) * 16 + 16 +
           (E_global <= kMapLds ? static_cast<size_t>(E_global) * 4 : 0);
}

void launch_align(const AlignArgs& a_in, hipStream_t s) {
    AlignArgs a = a_in;
    int W = align_waves(a.E_local);
    // about one chunk of 64 slots per wavefront in each workgroup's range;
    // every workgroup also counts all slots once (pass 0)
    const int64_t chunks = (static_cast<int64_t>(a.T) * a.top_k + 63) / 64;
    int64_t nb = chunks / W;
    nb = nb < 1 ? 1 : (nb > 64 ? 64 : nb);
    if (a.logits) {
        a.topk_ids = a.ids_out;
        if (nb > 1) {
            // every workgroup counts all slots: the router runs first, alone
            launch_router_topk(a.logits, a.T, a.E_global, a.top_k, a.ids_out, a.weights_out, s);
            a.logits = nullptr;
        }
    }
    k_align<<<dim3(static_cast<unsigned>(nb)), dim3(64 * W),
              align_lds_bytes(W, a.E_local, a.E_global), s>>>(a);
}

}  // namespace w4a16
