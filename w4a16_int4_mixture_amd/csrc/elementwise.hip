// Bandwidth-bound steps around the GEMMs: SiLU(gate) * up (for weights
// packed without gate/up interleave) and the top-k weighted combine.  Each
// thread moves 16 bytes per access.
//
// Chord page, "Measurements": routing and activation sit outside the timed
// gate/up + down unit; the computation between and after the GEMMs is the
// plain SiLU(gate) * up of the MoE FFN and the top-k weighted sum of the
// expert outputs.

#include "device_common.h"
#include "internal.h"

namespace w4a16 {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float lo_f(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float hi_f(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ inline uint32_t bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}
__device__ inline uint32_t pack2(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }

// silu(g) * u in fp32 from bf16-valued inputs: the GEMM epilogues' own
// function, so the fused and the separate activation agree bit for bit
__device__ inline float silu_mul(float g, float u) { return dev::silu_mul_bf16(g, u); }

}  // namespace

// Z[r, j..j+7] from Y13[r, j..j+7] (gate) and Y13[r, I+j..] (up), over the
// positions p < min(*rows_dev, rows) (or p < rows):
//   masked_m != nullptr: p = g * max_m + i is skipped when i >= masked_m[g]
//                        (a count above max_m covers the expert's max_m rows);
//   sorted_ids != nullptr: p is skipped when f = sorted_ids[p] is not a slot
//                        (padding sentinel); the row is f if slot_rows, else p.
__global__ void k_silu_mul(const uint16_t* __restrict__ y13, int64_t rows,
                           const int32_t* __restrict__ rows_dev, int I,
                           const int32_t* __restrict__ masked_m, int max_m,
                           const int32_t* __restrict__ sorted_ids, int num_slots, int slot_rows,
                           uint16_t* __restrict__ z) {
    int64_t nrows = rows;
    if (rows_dev) {
        const int64_t d = rows_dev[0];
        nrows = d < rows ? (d > 0 ? d : 0) : rows;
    }
    const int per_row = I / 8;
    const int64_t total = nrows * per_row;
    for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
         idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t p = idx / per_row;
        const int j = static_cast<int>(idx % per_row) * 8;
        if (masked_m) {
            const int mg = masked_m[p / max_m];
            if ((p % max_m) >= (mg < max_m ? mg : max_m)) continue;
        }
        int64_t r = p;
        if (sorted_ids) {
            const int f = sorted_ids[p];
            if (f < 0 || f >= num_slots) continue;
            if (slot_rows) r = f;
        }
        const u32x4 g = *reinterpret_cast<const u32x4*>(y13 + r * 2 * I + j);
        const u32x4 u = *reinterpret_cast<const u32x4*>(y13 + r * 2 * I + I + j);
        u32x4 o;
        o.x = pack2(silu_mul(lo_f(g.x), lo_f(u.x)), silu_mul(hi_f(g.x), hi_f(u.x)));
        o.y = pack2(silu_mul(lo_f(g.y), lo_f(u.y)), silu_mul(hi_f(g.y), hi_f(u.y)));
        o.z = pack2(silu_mul(lo_f(g.z), lo_f(u.z)), silu_mul(hi_f(g.z), hi_f(u.z)));
        o.w = pack2(silu_mul(lo_f(g.w), lo_f(u.w)), silu_mul(hi_f(g.w), hi_f(u.w)));
        *reinterpret_cast<u32x4*>(z + r * I + j) = o;
    }
}

// grid (T, ceil(H / 512)), one wavefront per block; each lane accumulates 8
// consecutive columns of one token.  The token's routing entries are loaded in
// batches of kBatch, then the rows of a batch's local slots all at once (the
// entries are the same for every lane, so the skips are uniform branches), so
// that one memory latency covers a batch; the sum still runs in j order.
constexpr int kBatch = 8;

__global__ void __launch_bounds__(64) k_combine(const uint16_t* __restrict__ y, int64_t y_rows,
                                                int H, const int32_t* __restrict__ row_of,
                                                const float* __restrict__ w, int top_k,
                                                uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    {
        const int h = (blockIdx.y * 64 + threadIdx.x) * 8;
        if (h >= H) return;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const int32_t* ro = row_of + static_cast<int64_t>(t) * top_k;
        const float* wr = w + static_cast<int64_t>(t) * top_k;
        for (int j0 = 0; j0 < top_k; j0 += kBatch) {
            int r[kBatch];
            float wt[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const bool in = j0 + q < top_k;
                r[q] = in ? ro[j0 + q] : -1;
                wt[q] = in ? wr[j0 + q] : 0.f;
            }
            u32x4 v[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                v[q] = u32x4{0u, 0u, 0u, 0u};
                if (r[q] >= 0 && r[q] < y_rows)
                    v[q] = *reinterpret_cast<const u32x4*>(y + static_cast<int64_t>(r[q]) * H + h);
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                if (!(r[q] >= 0 && r[q] < y_rows)) continue;
                const float yv[8] = {lo_f(v[q].x), hi_f(v[q].x), lo_f(v[q].y), hi_f(v[q].y),
                                     lo_f(v[q].z), hi_f(v[q].z), lo_f(v[q].w), hi_f(v[q].w)};
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = __fadd_rn(acc[i], __fmul_rn(wt[q], yv[i]));
            }
        }
        u32x4 o;
        o.x = pack2(acc[0], acc[1]);
        o.y = pack2(acc[2], acc[3]);
        o.z = pack2(acc[4], acc[5]);
        o.w = pack2(acc[6], acc[7]);
        *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(t) * H + h) = o;
    }
}

// Zero n 16-byte words (a kernel rather than a memset, so that it can sit in
// a captured HIP graph).
__global__ void k_zero16(u32x4* __restrict__ p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

static unsigned grid_for(int64_t items, int block) {
    int64_t g = (items + block - 1) / block;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return static_cast<unsigned>(g);
}

void launch_silu_mul(const uint16_t* y13, int64_t rows, const int32_t* rows_dev, int I,
                     const int32_t* masked_m, int max_m, const int32_t* sorted_ids, int num_slots,
                     bool slot_rows, uint16_t* z, hipStream_t s) {
    k_silu_mul<<<grid_for(rows * (I / 8), 256), 256, 0, s>>>(y13, rows, rows_dev, I, masked_m,
                                                             max_m, sorted_ids, num_slots,
                                                             slot_rows ? 1 : 0, z);
}

void launch_combine(const uint16_t* y, int64_t y_rows, int H, const int32_t* row_of,
                    const float* w, int T, int top_k, uint16_t* out, hipStream_t s) {
    k_combine<<<dim3(T, (H + 511) / 512), dim3(64), 0, s>>>(y, y_rows, H, row_of, w, top_k, out);
}

void launch_zero(void* p, uint64_t bytes, hipStream_t s) {
    const int64_t n = static_cast<int64_t>(bytes / 16);
    if (n > 0) k_zero16<<<grid_for(n, 256), 256, 0, s>>>(static_cast<u32x4*>(p), n);
}

}  // namespace w4a16
