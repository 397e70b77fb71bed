// Top-k weighted combine fused into the down GEMM's epilogue (the streaming
// kernel's; not part of the C ABI).
//
//   comb_out[t, n] = bf16( sum_{j<k, row_of[t*k+j] local} w[t, j] * Y2[row_of[t*k+j], n] )
//
// in fp32, j ascending, each product and sum rounded separately: the same
// arithmetic as the separate combine kernel, on the same bf16 rows.
//
// A token's k rows belong to different experts, so different workgroups
// store them.  After a workgroup has stored its item's rows (positions p0 ..
// p0 + nrows, one group of 256 columns), each row's token is counted once in
// a per-(token, column group) arrival counter; the workgroup whose arrival
// completes the token's count of local slots sums that token's rows for the
// group.  Nothing waits, and the sum runs in j order whichever workgroup
// arrives last.  The rows are stored and re-read with device-scope accesses
// (the storing and the summing workgroups may sit on different XCDs, whose
// L2 caches are not coherent with each other), and each thread's stores have
// completed before its workgroup counts an arrival.  The last arrival also
// resets the counter, so the counters are zero again after every call.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace w4a16 {
namespace dev {

// Loads of a token's routing entries are issued in batches of kCombBatch, so
// that one memory latency covers a batch rather than each entry.
constexpr int kCombBatch = 8;

// Local slots of token t: entries of row_of inside the position space.
__device__ inline int comb_local_slots(const GemmArgs& a, int t) {
    int n = 0;
    const int32_t* ro = a.comb_row_of + static_cast<int64_t>(t) * a.top_k;
    for (int j0 = 0; j0 < a.top_k; j0 += kCombBatch) {
        int r[kCombBatch];
#pragma unroll
        for (int q = 0; q < kCombBatch; ++q) r[q] = j0 + q < a.top_k ? ro[j0 + q] : -1;
#pragma unroll
        for (int q = 0; q < kCombBatch; ++q) n += (r[q] >= 0 && r[q] < a.sorted_cap) ? 1 : 0;
    }
    return n;
}

// Tokens with no local slot get +0 (no row of theirs ever arrives):
// workgroup b writes tokens b, b + G, ... (G = the grid).
__device__ inline void comb_zero_unrouted(const GemmArgs& a) {
    for (int t = blockIdx.x; t < a.comb_T; t += gridDim.x) {
        if (comb_local_slots(a, t) != 0) continue;
        uint16_t* o = a.comb_out + static_cast<int64_t>(t) * a.N;
        for (int c = threadIdx.x * 8; c < a.N; c += blockDim.x * 8)
            *reinterpret_cast<u32x4*>(o + c) = u32x4{0u, 0u, 0u, 0u};
    }
}

// Called by every thread of the workgroup after it stored rows [p0, p0 +
// nrows) of column group g.  s_tok: LDS, at least nrows ints; s_n: one LDS int.
__device__ inline void comb_arrive(const GemmArgs& a, int p0, int nrows, int g, int* s_tok,
                                   int* s_n) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's row stores have completed
    if (threadIdx.x == 0) *s_n = 0;
    __syncthreads();
    for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
        const int f = a.sorted_ids[p0 + r];
        if (f < 0 || f >= a.num_slots) continue;
        const int t = f / a.top_k;
        int32_t* c = a.comb_counters + static_cast<int64_t>(t) * a.comb_groups + g;
        if (atomicAdd(c, 1) == comb_local_slots(a, t) - 1) {
            atomicExch(c, 0);
            s_tok[atomicAdd(s_n, 1)] = t;
        }
    }
    __syncthreads();
    const int n = *s_n;
    // 32 threads per completed token, 8 columns (16 bytes) each
    const __amdgpu_buffer_rsrc_t y =
        make_rsrc(a.out, static_cast<uint64_t>(a.sorted_cap) * a.N * 2);
    const int c = 256 * g + 8 * (threadIdx.x & 31);
    for (int i = threadIdx.x >> 5; i < n; i += blockDim.x >> 5) {
        if (c >= a.N) continue;
        const int t = s_tok[i];
        const int32_t* ro = a.comb_row_of + static_cast<int64_t>(t) * a.top_k;
        const float* wr = a.comb_w + static_cast<int64_t>(t) * a.top_k;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < a.top_k; j0 += kCombBatch) {
            int r[kCombBatch];
            float wt[kCombBatch];
#pragma unroll
            for (int q = 0; q < kCombBatch; ++q) {
                const bool in = j0 + q < a.top_k;
                r[q] = in ? ro[j0 + q] : -1;
                wt[q] = in ? wr[j0 + q] : 0.f;
            }
            // all loads of the batch at once; an entry outside the position
            // space reads row 0 instead and its sum is not taken
            u32x4 v[kCombBatch];
#pragma unroll
            for (int q = 0; q < kCombBatch; ++q) {
                const bool ok = r[q] >= 0 && r[q] < a.sorted_cap;
                // the host keeps sorted_cap * N * 2 below 4 GiB
                const uint32_t off = static_cast<uint32_t>(
                    ((ok ? static_cast<int64_t>(r[q]) : 0) * a.N + c) * 2);
                v[q] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(y, off, 0, kDeviceScope));
            }
#pragma unroll
            for (int q = 0; q < kCombBatch; ++q) {
                if (!(r[q] >= 0 && r[q] < a.sorted_cap)) continue;
                const uint32_t w4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    acc[2 * h] =
                        __fadd_rn(acc[2 * h], __fmul_rn(wt[q], __uint_as_float(w4[h] << 16)));
                    acc[2 * h + 1] = __fadd_rn(
                        acc[2 * h + 1], __fmul_rn(wt[q], __uint_as_float(w4[h] & 0xFFFF0000u)));
                }
            }
        }
        u32x4 o;
        o.x = f32_to_bf16_rne(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[1])) << 16);
        o.y = f32_to_bf16_rne(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[3])) << 16);
        o.z = f32_to_bf16_rne(acc[4]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[5])) << 16);
        o.w = f32_to_bf16_rne(acc[6]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[7])) << 16);
        *reinterpret_cast<u32x4*>(a.comb_out + static_cast<int64_t>(t) * a.N + c) = o;
    }
    __syncthreads();   // s_tok and s_n are reused by the workgroup's next item
}

}  // namespace dev
}  // namespace w4a16
