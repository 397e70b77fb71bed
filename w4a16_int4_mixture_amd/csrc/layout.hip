// Indexed routing -> grouped masked layout on the device.
//
// Chord page, "Grouped SM90 kernels": the masked dispatch takes activations
// already placed per expert, [G, max_m, K], with each expert's valid count in
// masked_m; "vLLM integration": routing stays on the device (no host
// read-back of counts).  This is the placement, from the routing sort: with
// block_m = 1 the sort leaves no padding, so the local slot at position p of
// expert e's segment has rank p - offset[e] among that expert's slots in
// ascending slot order.  Rank i < max_m goes to row e * max_m + i; larger
// ranks are dropped (counted).
//
// One wavefront per sorted position copies the slot's activation row (16
// bytes per lane per step); the first wavefronts also write masked_m and the
// drop count, and every thread marks the non-local slots of its stride.

#include "device_common.h"
#include "internal.h"

namespace w4a16 {

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
}

__global__ void __launch_bounds__(256) k_to_masked(MaskedPlaceArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    const int64_t gtid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t gsize = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int n = a.ntp[0] < a.sorted_cap ? a.ntp[0] : a.sorted_cap;

    // counts per expert, the drop count (one thread), non-local slots
    for (int64_t e = gtid; e < a.E; e += gsize) {
        const int c = a.offsets[e + 1] - a.offsets[e];
        a.masked_m[e] = c < a.max_m ? c : a.max_m;
    }
    if (gtid == 0 && a.dropped) {
        int d = 0;
        for (int e = 0; e < a.E; ++e) {
            const int c = a.offsets[e + 1] - a.offsets[e];
            d += c > a.max_m ? c - a.max_m : 0;
        }
        a.dropped[0] = d;
    }
    for (int64_t f = gtid; f < a.num_slots; f += gsize)
        if (a.row_of[f] < 0) a.row_of_masked[f] = -1;

    // rows: wavefront per sorted position
    const int per_row = a.H / 8;   // 16-byte pieces
    for (int64_t p = wave; p < n; p += nwaves) {
        const int f = a.sorted_ids[p];
        const int e = a.expert_ids[p];
        if (f < 0 || f >= a.num_slots || e < 0 || e >= a.E) continue;
        const int64_t i = p - a.offsets[e];
        if (i >= a.max_m) {
            if (lane == 0) a.row_of_masked[f] = -1;
            continue;
        }
        const int64_t row = static_cast<int64_t>(e) * a.max_m + i;
        if (lane == 0) a.row_of_masked[f] = static_cast<int32_t>(row);
        const u32x4* src = reinterpret_cast<const u32x4*>(a.X + static_cast<int64_t>(f / a.top_k) * a.H);
        u32x4* dst = reinterpret_cast<u32x4*>(a.a3 + row * a.H);
        for (int c = lane; c < per_row; c += 64) dst[c] = src[c];
    }
}

void launch_to_masked(const MaskedPlaceArgs& a, hipStream_t s) {
    // four positions per workgroup, enough workgroups to cover the slots
    int64_t blocks = (static_cast<int64_t>(a.sorted_cap) + 3) / 4;
    blocks = blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks);
    k_to_masked<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(a);
}

}  // namespace w4a16
