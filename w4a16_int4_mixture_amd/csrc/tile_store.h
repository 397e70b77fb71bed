// Epilogue of the streaming kernels (16x16 MFMA tiles): stores a tile's rows
// from the fp32 accumulators (not part of the C ABI).
#pragma once

#include "device_common.h"
#include "internal.h"

namespace w4a16 {
namespace dev {

// Stores the tile's rows from the accumulators: lane holds rows 16t +
// 4*(lane/16) + i of column 16j + lane%16 of the chunk.
template <int MT, int WPL>
__device__ __forceinline__ void store_tile(const GemmArgs& a, int p0, int nrows, int chunk,
                                           int lane, const f32x4 (&acc)[MT][WPL]) {
    const bool slot_rows = a.tile_src != TILE_MASKED;
    // with the fused combine, the rows are stored with device-scope stores:
    // the workgroup that sums a token may run on another XCD
    const __amdgpu_buffer_rsrc_t ydev =
        make_rsrc(a.out, a.comb_out ? static_cast<uint64_t>(a.sorted_cap) * a.N * 2 : 0);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * t + 4 * (lane >> 4) + i;
            if (r >= nrows) continue;
            int64_t orow = p0 + r;
            if (slot_rows && (a.tile_src == TILE_BLOCKS || a.orow == W4A16_OROW_SLOT)) {
                int f = a.sorted_ids[p0 + r];
                if (f < 0 || f >= a.num_slots) continue;
                if (a.orow == W4A16_OROW_SLOT) orow = f;
            }
            if (a.out_kind == OUT_SILU) {
                // gate/up interleave: columns 16j (j < WPL/2) of the chunk are
                // gate columns, 16(j + WPL/2) the matching up columns
                uint16_t* o = static_cast<uint16_t*>(a.out) + orow * (a.N / 2) +
                              chunk * (a.CW / 2) + (lane & 15);
#pragma unroll
                for (int j = 0; j < WPL / 2; ++j)
                    o[16 * j] =
                        f32_to_bf16_rne(silu_mul_bf16(acc[t][j][i], acc[t][j + WPL / 2][i]));
            } else if (a.out_kind == OUT_BF16) {
                if (a.comb_out) {
                    // sorted_cap * N * 2 < 4 GiB (host check)
                    const uint32_t off =
                        static_cast<uint32_t>((orow * a.N + chunk * a.CW + (lane & 15)) * 2);
#pragma unroll
                    for (int j = 0; j < WPL; ++j)
                        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(acc[t][j][i]), ydev,
                                                              off, 32 * j, kDeviceScope);
                } else {
                    uint16_t* o =
                        static_cast<uint16_t*>(a.out) + orow * a.N + chunk * a.CW + (lane & 15);
#pragma unroll
                    for (int j = 0; j < WPL; ++j) o[16 * j] = f32_to_bf16_rne(acc[t][j][i]);
                }
            } else {
                float* o = static_cast<float*>(a.out) + orow * a.N + chunk * a.CW + (lane & 15);
#pragma unroll
                for (int j = 0; j < WPL; ++j) o[16 * j] = acc[t][j][i];
            }
        }
    }
}

}  // namespace dev
}  // namespace w4a16
