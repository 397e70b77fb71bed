// Load-time weight prepacking: canonical INT4 codes + bf16 group scales ->
// the device layout read by the GEMM kernels.
//
// Chord page, "Indexed kernels" / Figure 2: the kernel profile and the weight
// layout are fixed when the model is loaded; "Grouped SM90 kernels": the
// packers permute the INT4 buffer bit by bit and re-lay the scales, and the
// prepared weight records its mode.  Here the permutation serves CDNA4: each
// wavefront lane fetches, with one 16-byte load per K group of 32, the codes
// of its MFMA B-operand fragments for CW/16 column blocks, and the nibble
// order lets two bf16 operands be formed per VALU op (see the codes layout in
// internal.h).  Values are never touched: the permutation is exact.

#include "internal.h"

namespace w4a16 {

int chunk_width_of(int profile) {
    switch (profile) {
        case W4A16_PROFILE_DECODE: return 64;
        case W4A16_PROFILE_PREFILL: return 128;
        default: return 0;
    }
}

static uint64_t round_up(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

w4a16_status make_geom(int profile, uint32_t flags, int E, int N, int K, int group,
                       PackGeom* g) {
    int cw = chunk_width_of(profile);
    if (cw == 0) {
        set_error("unknown profile %d", profile);
        return W4A16_ERR_UNSUPPORTED;
    }
    if (flags & ~(W4A16_PACK_GATE_UP_INTERLEAVE | W4A16_PACK_MXFP4 | W4A16_PACK_MXFP8_ACT)) {
        set_error("unknown prepack flags 0x%x", flags);
        return W4A16_ERR_UNSUPPORTED;
    }
    if ((flags & W4A16_PACK_MXFP8_ACT) && !(flags & W4A16_PACK_MXFP4)) {
        set_error("the MXFP8-activation layout is for MXFP4 weights (w4a16_prepack_mxfp4)");
        return W4A16_ERR_UNSUPPORTED;
    }
    if ((flags & W4A16_PACK_MXFP4) && profile != W4A16_PROFILE_DECODE) {
        set_error("MXFP4 weights are packed with the DECODE profile only");
        return W4A16_ERR_UNSUPPORTED;
    }
    if (E <= 0 || N <= 0 || K <= 0) {
        set_error("bad shape E=%d N=%d K=%d", E, N, K);
        return W4A16_ERR_INVALID_ARG;
    }
    if (group != 32) {
        set_error("only group size 32 is supported (got %d)", group);
        return W4A16_ERR_UNSUPPORTED;
    }
    if (K % 32 != 0) {
        set_error("K=%d is not a multiple of the group size 32", K);
        return W4A16_ERR_UNSUPPORTED;
    }
    if (N % cw != 0) {
        set_error("N=%d is not a multiple of the profile's chunk width %d", N, cw);
        return W4A16_ERR_UNSUPPORTED;
    }
    g->E = E;
    g->N = N;
    g->K = K;
    g->CW = cw;
    g->NC = N / cw;
    g->KS = K / 32;
    g->KSP = static_cast<int>(round_up(static_cast<uint64_t>(g->KS), 8));
    g->WPL = cw / 16;
    g->interleave = (flags & W4A16_PACK_GATE_UP_INTERLEAVE) != 0;
    g->mxfp4 = (flags & W4A16_PACK_MXFP4) != 0;
    g->a8 = (flags & W4A16_PACK_MXFP8_ACT) != 0;
    // 512 WPL code words, then 64 WPL words of bf16 scales or 32 WPL of E8M0
    g->stage_words = (g->a8 ? 544ull : 576ull) * g->WPL;
    g->chunk_words = g->stage_words * (g->KSP / 8);
    g->stage_bytes = g->stage_words * 4;
    g->chunk_bytes = g->chunk_words * 4;
    g->bytes = g->chunk_bytes * static_cast<uint64_t>(E) * g->NC;
    return W4A16_OK;
}

w4a16_status check_desc(const w4a16_desc* d) {
    if (!d) {
        set_error("null weight descriptor");
        return W4A16_ERR_INVALID_ARG;
    }
    if (d->magic != W4A16_DESC_MAGIC || d->version != W4A16_DESC_VERSION) {
        set_error("weight descriptor has bad magic/version (0x%x/%u): not a prepared weight",
                  d->magic, d->version);
        return W4A16_ERR_MODE_MISMATCH;
    }
    PackGeom g;
    w4a16_status st = make_geom(d->profile, d->flags, d->E, d->N, d->K, d->group, &g);
    if (st != W4A16_OK) return W4A16_ERR_MODE_MISMATCH;
    if (g.CW != d->chunk_n || g.KSP != d->k_groups || g.bytes != d->bytes ||
        g.stage_bytes != d->stage_bytes || g.chunk_bytes != d->chunk_bytes) {
        set_error("weight descriptor is inconsistent with its profile/shape");
        return W4A16_ERR_MODE_MISMATCH;
    }
    return W4A16_OK;
}

__host__ __device__ static inline uint32_t permute_word(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) out |= ((w >> (4 * nibble_k_offset(i))) & 0xFu) << (4 * i);
    return out;
}

// The bf16 scale of (row, group): the bf16 scale itself, or for MXFP4 the
// E8M0 byte b as the bf16 2^(b - 127) (exact: exponent field b, or the
// subnormal 2^-127 for b = 0; b = 255 is NaN).
__host__ __device__ static inline uint32_t scale_bits(const void* scales, const PackGeom& g,
                                                      int64_t idx) {
    if (!g.mxfp4) return static_cast<const uint16_t*>(scales)[idx];
    const uint32_t b = static_cast<const uint8_t*>(scales)[idx];
    return b == 255 ? 0x7FC0u : b == 0 ? 0x0040u : b << 7;
}

// PREFILL record word `in` (see the layout in internal.h): codes in their
// canonical nibble order, one 16-byte group per (group, half, lane).
__host__ __device__ static inline uint32_t prefill_word(const uint32_t* codes,
                                                        const void* scales, const PackGeom& g,
                                                        int64_t e, int c, int stage, int in) {
    if (in < 4096) {
        const int v = in & 3, lane = (in >> 2) & 63, h = (in >> 8) & 1;
        const int ks = stage * 8 + (in >> 9);
        if (ks >= g.KS) return 0u;
        const int j = h + 2 * (v >> 1), s = v & 1;
        const int n = canonical_column(c * 128 + 32 * j + (lane & 31), g.N, 128, g.interleave);
        return codes[(e * g.N + n) * (g.K / 8) + ks * 4 + 2 * s + (lane >> 5)];
    }
    uint32_t out = 0;
    for (int hh = 0; hh < 2; ++hh) {
        const int b = 2 * (in - 4096) + hh;   // bf16 index inside the scale block
        const int jj = b & 1, c32 = (b >> 4) & 31, h = (b >> 9) & 1;
        const int ks = stage * 8 + ((b >> 1) & 7);
        uint32_t v = 0;
        if (ks < g.KS) {
            const int n = canonical_column(c * 128 + 32 * (h + 2 * jj) + c32, g.N, 128, g.interleave);
            v = scale_bits(scales, g, (e * g.N + n) * g.KS + ks);
        }
        out |= v << (16 * hh);
    }
    return out;
}

// A8W4 record word `in` (layout in internal.h): canonical E2M1 words in the
// block-scaled MFMA's B-operand order, then E8M0 bytes four to a word.
__host__ __device__ static inline uint32_t a8_word(const uint32_t* codes, const void* scales,
                                                   const PackGeom& g, int64_t e, int c, int stage,
                                                   int in) {
    const int code_words = 512 * g.WPL;
    if (in < code_words) {
        const int w = in & 3, lane = (in >> 2) & 63, sj = in >> 8;
        const int j = sj % g.WPL, s = sj / g.WPL;
        const int kw = (stage * 256 + s * 128 + 32 * (lane >> 4)) / 8 + w;   // word along K
        if (kw * 8 >= g.K) return 0u;
        const int n = canonical_column(c * g.CW + 16 * j + (lane & 15), g.N, g.CW, g.interleave);
        return codes[(e * g.N + n) * (g.K / 8) + kw];
    }
    const int idx = in - code_words, s = idx >> 6, lane = idx & 63;
    const int ks = stage * 8 + 4 * s + (lane >> 4);
    uint32_t out = 0;
    for (int j = 0; j < g.WPL; ++j) {
        uint32_t b = 0;
        if (ks < g.KS) {
            const int n = canonical_column(c * g.CW + 16 * j + (lane & 15), g.N, g.CW, g.interleave);
            b = static_cast<const uint8_t*>(scales)[(e * g.N + n) * g.KS + ks];
        }
        out |= b << (8 * j);
    }
    return out;
}

// Word w of the packed buffer, from the canonical codes and scales.
__host__ __device__ static inline uint32_t packed_word(const uint32_t* codes, const void* scales,
                                                       const PackGeom& g, uint64_t w) {
    const uint64_t chunk_id = w / g.chunk_words;        // e * NC + c
    const int64_t e = static_cast<int64_t>(chunk_id / g.NC);
    const int c = static_cast<int>(chunk_id % g.NC);
    const uint64_t r = w % g.chunk_words;
    const int stage = static_cast<int>(r / g.stage_words);
    const int in = static_cast<int>(r % g.stage_words);
    if (g.CW == 128) return prefill_word(codes, scales, g, e, c, stage, in);
    if (g.a8) return a8_word(codes, scales, g, e, c, stage, in);
    const int code_words = 512 * g.WPL;
    if (in < code_words) {
        const int j = in % g.WPL;
        const int lane = (in / g.WPL) % 64;
        const int ks = stage * 8 + in / (64 * g.WPL);
        if (ks >= g.KS) return 0u;
        const int n = canonical_column(c * g.CW + 16 * j + (lane & 15), g.N, g.CW, g.interleave);
        // INT4: nibbles permuted for the 128 + q operand trick; MXFP4: the
        // canonical order, byte b holding K offsets 2b (low) and 2b + 1
        const uint32_t cw = codes[(e * g.N + n) * (g.K / 8) + ks * 4 + (lane >> 4)];
        return g.mxfp4 ? cw : permute_word(cw);
    }
    uint32_t out = 0;
    for (int h = 0; h < 2; ++h) {
        const int b = 2 * (in - code_words) + h;         // bf16 index inside the scale block
        const int j = b % g.WPL;
        const int c16 = (b / g.WPL) % 16;
        const int ks = stage * 8 + b / (16 * g.WPL);
        uint32_t v = 0;
        if (ks < g.KS) {
            const int n = canonical_column(c * g.CW + 16 * j + c16, g.N, g.CW, g.interleave);
            v = scale_bits(scales, g, (e * g.N + n) * g.KS + ks);
        }
        out |= v << (16 * h);
    }
    return out;
}

__global__ void k_prepack(const uint32_t* __restrict__ codes, const void* __restrict__ scales,
                          uint32_t* __restrict__ out, PackGeom g, uint64_t total) {
    const uint64_t w = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (w >= total) return;
    out[w] = packed_word(codes, scales, g, w);
}

void launch_prepack(const PackGeom& g, const uint32_t* codes, const void* scales,
                    void* packed, hipStream_t s) {
    const uint64_t total = g.bytes / 4;
    k_prepack<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
        codes, scales, static_cast<uint32_t*>(packed), g, total);
}

// Host reference of the same permutation.
static void prepack_host(const PackGeom& g, const uint32_t* codes, const void* scales,
                         void* packed) {
    uint32_t* out = static_cast<uint32_t*>(packed);
    const uint64_t total = g.bytes / 4;
    for (uint64_t w = 0; w < total; ++w) out[w] = packed_word(codes, scales, g, w);
}

static void fill_desc(const PackGeom& g, int profile, uint32_t flags, w4a16_desc* d) {
    d->magic = W4A16_DESC_MAGIC;
    d->version = W4A16_DESC_VERSION;
    d->profile = profile;
    d->flags = flags;
    d->E = g.E;
    d->N = g.N;
    d->K = g.K;
    d->group = 32;
    d->chunk_n = g.CW;
    d->k_groups = g.KSP;
    d->stage_bytes = g.stage_bytes;
    d->chunk_bytes = g.chunk_bytes;
    d->bytes = g.bytes;
}

static w4a16_status prepack_common(int32_t profile, uint32_t flags, const int32_t* codes,
                                   const void* scales, int32_t E, int32_t N, int32_t K,
                                   int32_t group, void* packed, uint64_t packed_bytes,
                                   w4a16_desc* desc, PackGeom* g, bool device) {
    w4a16_status st = make_geom(profile, flags, E, N, K, group, g);
    if (st != W4A16_OK) return st;
    W4A16_CHECK_ARG(codes && scales && packed && desc, "null pointer argument to prepack");
    W4A16_CHECK_ARG(!device || (reinterpret_cast<uintptr_t>(packed) & 255) == 0,
                    "packed buffer must be 256-byte aligned");
    W4A16_CHECK_ARG((reinterpret_cast<uintptr_t>(codes) & 3) == 0 &&
                        ((flags & W4A16_PACK_MXFP4) || (reinterpret_cast<uintptr_t>(scales) & 1) == 0),
                    "codes/scales misaligned");
    if ((flags & W4A16_PACK_GATE_UP_INTERLEAVE) && (N % 2 != 0)) {
        set_error("gate/up interleave needs an even N");
        return W4A16_ERR_UNSUPPORTED;
    }
    if (packed_bytes < g->bytes) {
        set_error("packed buffer too small: %llu < %llu bytes",
                  static_cast<unsigned long long>(packed_bytes),
                  static_cast<unsigned long long>(g->bytes));
        return W4A16_ERR_CAPACITY;
    }
    return W4A16_OK;
}

}  // namespace w4a16

using namespace w4a16;

extern "C" w4a16_status w4a16_prepack_bytes(int32_t profile, uint32_t flags, int32_t E,
                                            int32_t N, int32_t K, int32_t group,
                                            uint64_t* bytes) {
    clear_error();
    W4A16_CHECK_ARG(bytes, "null bytes pointer");
    PackGeom g;
    w4a16_status st = make_geom(profile, flags, E, N, K, group, &g);
    if (st != W4A16_OK) return st;
    *bytes = g.bytes;
    return W4A16_OK;
}

static w4a16_status prepack_device(int32_t profile, uint32_t flags, const int32_t* codes,
                                   const void* scales, int32_t E, int32_t N, int32_t K,
                                   int32_t group, void* packed, uint64_t packed_bytes,
                                   w4a16_desc* desc, void* stream) {
    PackGeom g;
    w4a16_status st = prepack_common(profile, flags, codes, scales, E, N, K, group, packed,
                                     packed_bytes, desc, &g, true);
    if (st != W4A16_OK) return st;
    launch_prepack(g, reinterpret_cast<const uint32_t*>(codes), scales, packed,
                   static_cast<hipStream_t>(stream));
    st = check_launch("prepack");
    if (st != W4A16_OK) return st;
    fill_desc(g, profile, flags, desc);
    return W4A16_OK;
}

static w4a16_status prepack_on_host(int32_t profile, uint32_t flags, const int32_t* codes,
                                    const void* scales, int32_t E, int32_t N, int32_t K,
                                    int32_t group, void* packed, uint64_t packed_bytes,
                                    w4a16_desc* desc) {
    PackGeom g;
    w4a16_status st = prepack_common(profile, flags, codes, scales, E, N, K, group, packed,
                                     packed_bytes, desc, &g, false);
    if (st != W4A16_OK) return st;
    prepack_host(g, reinterpret_cast<const uint32_t*>(codes), scales, packed);
    fill_desc(g, profile, flags, desc);
    return W4A16_OK;
}

extern "C" w4a16_status w4a16_prepack(int32_t profile, uint32_t flags, const int32_t* codes,
                                      const uint16_t* scales, int32_t E, int32_t N, int32_t K,
                                      int32_t group, void* packed, uint64_t packed_bytes,
                                      w4a16_desc* desc, void* stream) {
    clear_error();
    W4A16_CHECK_ARG(!(flags & W4A16_PACK_MXFP4), "MXFP4 weights go through w4a16_prepack_mxfp4");
    return prepack_device(profile, flags, codes, scales, E, N, K, group, packed, packed_bytes,
                          desc, stream);
}

extern "C" w4a16_status w4a16_prepack_host(int32_t profile, uint32_t flags, const int32_t* codes,
                                           const uint16_t* scales, int32_t E, int32_t N,
                                           int32_t K, int32_t group, void* packed,
                                           uint64_t packed_bytes, w4a16_desc* desc) {
    clear_error();
    W4A16_CHECK_ARG(!(flags & W4A16_PACK_MXFP4), "MXFP4 weights go through w4a16_prepack_mxfp4_host");
    return prepack_on_host(profile, flags, codes, scales, E, N, K, group, packed, packed_bytes,
                           desc);
}

extern "C" w4a16_status w4a16_prepack_mxfp4(int32_t profile, uint32_t flags, const int32_t* codes,
                                            const uint8_t* scales_e8m0, int32_t E, int32_t N,
                                            int32_t K, int32_t group, void* packed,
                                            uint64_t packed_bytes, w4a16_desc* desc,
                                            void* stream) {
    clear_error();
    return prepack_device(profile, flags | W4A16_PACK_MXFP4, codes, scales_e8m0, E, N, K, group,
                          packed, packed_bytes, desc, stream);
}

extern "C" w4a16_status w4a16_prepack_mxfp4_host(int32_t profile, uint32_t flags,
                                                 const int32_t* codes, const uint8_t* scales_e8m0,
                                                 int32_t E, int32_t N, int32_t K, int32_t group,
                                                 void* packed, uint64_t packed_bytes,
                                                 w4a16_desc* desc) {
    clear_error();
    return prepack_on_host(profile, flags | W4A16_PACK_MXFP4, codes, scales_e8m0, E, N, K, group,
                           packed, packed_bytes, desc);
}
