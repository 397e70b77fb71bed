// W4A16 INT4 MoE expert path -- plain CPU oracle.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
// call this file; only the tests, the smoke check and the benchmark's CPU
// baseline leg use it.  It shares no code, header, table or helper with the
// HIP library: it is written from the definition of the computation, slowly
// and obviously, so that it can be checked by eye against the source page.
//
// Source page (cited below as "Chord page"): "vLLM x Novita AI: Chord W4A16
// INT4 MoE kernels for Kimi K2.x" (novita.ai blog).  Section names are given
// in English translation.
//
// What is computed (the dense MoE expert FFN on dequantised INT4 weights):
//   weights  : unsigned 4-bit codes q[e][n][c] with one bf16 scale per group
//              of 32 along K, s[e][n][c/32]  (Chord page, "Grouped SM90
//              kernels", operator entry-point listing: weight [G,N,K] uint4,
//              scale [G,N,K/32] bf16; TL;DR: BF16 activations, INT4 weights,
//              group-32 scales)
//   dequant  : w = (q - 8) * s, i.e. subtract the offset, then scale
//              (Chord page, "H200 and Blackwell indexed decode": the dequant
//              subtracts and then scales).  Exact in fp32: a 4-bit integer
//              times an 8-bit-significand bf16 needs at most 12 bits.
//   gate/up  : Y13[f,n] = bf16( sum_c X[t,c] * w13[e,n,c] ), fp32 accumulate
//   act      : Z[f,j]   = bf16( silu(Y13[f,j]) * Y13[f,I+j] )
//   down     : Y2[f,h]  = bf16( sum_c Z[f,c] * w2[e,h,c] ), fp32 accumulate
//   combine  : out[t,h] = bf16( sum_j w[t,j] * Y2[row(t,j),h] ), fp32
//   routing  : indexed sorted_ids / expert_ids / num_tokens_padded ("Two
//              kernel families", "vLLM integration") and the grouped masked
//              layout with per-expert valid counts ("Grouped SM90 kernels").
//
// Readings where the page is silent (each listed with its reason in the
// design notes): low nibble of a 32-bit word = lowest K index; code 8 is
// zero; gate = first I rows of W13, up = last I rows; fp32 accumulation in
// ascending K order (the page rules out f16 accumulation, "vLLM
// integration"); bf16 rounding is round-to-nearest-even; the combine weight
// is applied to the bf16-rounded down output.
//
// Build: g++ -O2 -std=c++17 -fopenmp -ffp-contract=off -shared -fPIC
// (-ffp-contract=off keeps every multiply and add a separate rounding step.)

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ---- bf16 <-> binary32/64 (round to nearest, ties to even) ----------------

float bf16_to_float(uint16_t b) {
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Round a double to the nearest bf16 (ties to even) with one rounding step.
// bf16 has 8 significant bits, exponent range as binary32; below 2^-126 the
// quantum is fixed at 2^-133 (subnormals).
uint16_t bf16_from_double(double d) {
    if (std::isnan(d)) return 0x7FC0;
    uint16_t sign = std::signbit(d) ? 0x8000 : 0;
    double a = std::fabs(d);
    if (std::isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    std::frexp(a, &e);                       // a = m * 2^e, m in [0.5, 1)
    int qexp = (e - 1 >= -126) ? (e - 8) : -133;   // exponent of one ulp
    double q = std::ldexp(1.0, qexp);
    double r = std::nearbyint(a / q) * q;    // default mode: ties to even
    if (r >= std::ldexp(1.0, 128)) return sign | 0x7F80;   // overflow -> inf
    float rf = static_cast<float>(r);        // exact: r has <= 8 significant bits
    uint32_t u;
    std::memcpy(&u, &rf, 4);
    return sign | static_cast<uint16_t>(u >> 16);
}

uint16_t bf16_from_float(float f) { return bf16_from_double(static_cast<double>(f)); }

// ---- weight format ---------------------------------------------------------

// Code c of a row of K codes, stored eight per 32-bit word along K.
inline uint32_t code_at(const uint32_t* row_words, int64_t c) {
    return (row_words[c / 8] >> (4 * (c % 8))) & 0xFu;
}

// Dequantised weight w[c] of one output row: (q - 8) * s, exact in fp32.
// wmode 1 rounds it to bf16 (the round-after-scale order a bf16 tensor-core
// operand requires).
inline float weight_at(const uint32_t* row_words, const uint16_t* row_scales,
                       int64_t c, int wmode) {
    float q = static_cast<float>(static_cast<int>(code_at(row_words, c)) - 8);
    float w = q * bf16_to_float(row_scales[c / 32]);
    if (wmode == 1) w = bf16_to_float(bf16_from_float(w));
    return w;
}

// MXFP4 weights (news.ainew.jp, "vLLM publishes Kimi K3 production support",
// MXFP4 MoE section: 4-bit floating-point expert weights with one shared
// power-of-two scale per block of 32, the OCP microscaling format).  A code
// is an E2M1 number: sign bit 3, exponent bits 2..1, mantissa bit 0; value
// (-1)^s * 2^(e - 1) * (1 + m / 2) for e > 0 and (-1)^s * m / 2 for e = 0.
// A block scale is an E8M0 byte: 2^(b - 127), b = 255 reading as NaN.
inline float e2m1_value(uint32_t code) {
    const uint32_t e = (code >> 1) & 3u, m = code & 1u;
    const float mag = e == 0 ? 0.5f * static_cast<float>(m)
                             : std::ldexp(1.0f + 0.5f * static_cast<float>(m), static_cast<int>(e) - 1);
    return (code & 8u) ? -mag : mag;
}

inline float e8m0_value(uint8_t b) {
    return b == 255 ? std::nanf("") : std::ldexp(1.0f, static_cast<int>(b) - 127);
}

// Dequantised MXFP4 weight w[c] of one output row: e2m1(q) * 2^(b - 127),
// exact in fp32 (a 2-bit significand times a power of two) inside fp32's range.
inline float weight_at_mx(const uint32_t* row_words, const uint8_t* row_scales, int64_t c) {
    return e2m1_value(code_at(row_words, c)) * e8m0_value(row_scales[c / 32]);
}

// Local expert of routed slot f, or -1 (non-local or out of range).
inline int local_expert(const int32_t* topk_ids, int64_t f, int E_global,
                        const int32_t* expert_map, int E_local) {
    int g = topk_ids[f];
    if (g < 0 || g >= E_global) return -1;
    int e = expert_map ? expert_map[g] : g;
    if (e < 0 || e >= E_local) return -1;
    return e;
}

// One output element: sum over c ascending of a[c] * w[c] in fp32 (acc = 0),
// or in fp64 when acc64 is set (used only to measure the fp32 error).
inline double dot_row(const uint16_t* a, const uint32_t* row_words,
                      const uint16_t* row_scales, int64_t K, int wmode, int acc64) {
    if (acc64) {
        double acc = 0.0;
        for (int64_t c = 0; c < K; ++c)
            acc += static_cast<double>(bf16_to_float(a[c])) *
                   static_cast<double>(weight_at(row_words, row_scales, c, wmode));
        return acc;
    }
    float acc = 0.0f;
    for (int64_t c = 0; c < K; ++c)
        acc += bf16_to_float(a[c]) * weight_at(row_words, row_scales, c, wmode);
    return static_cast<double>(acc);
}

// One output element on MXFP4 weights: sum over c ascending of a[c] * w[c] in
// fp32.
inline double dot_row_mx(const uint16_t* a, const uint32_t* row_words, const uint8_t* row_scales,
                         int64_t K) {
    float acc = 0.0f;
    for (int64_t c = 0; c < K; ++c) acc += bf16_to_float(a[c]) * weight_at_mx(row_words, row_scales, c);
    return static_cast<double>(acc);
}

// ---- A8W4: MXFP8 activations on MXFP4 weights ----------------------------
//
// The pages name A8W4 fused operators (8-bit activations, 4-bit weights)
// beside the A16W4 ones on AMD ("vLLM publishes Kimi K3 production support",
// MXFP4 MoE section) and give no format.  Reading: the activations take the
// same OCP microscaling form as the MXFP4 weights, with E4M3 elements: one
// E8M0 scale per block of 32 along K.
//
// E4M3 (OCP 8-bit float, no infinities): sign bit 7, exponent bits 6..3
// (bias 7), mantissa bits 2..0; value (-1)^s 2^(e-7) (1 + m/8) for e > 0 and
// (-1)^s 2^-6 m/8 for e = 0; exponent 15 with mantissa 7 is NaN, so the
// largest finite magnitude is 448 (code 0x7E).
inline double e4m3_value(uint8_t b) {
    const int e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return std::nan("");
    const double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
    return (b & 0x80) ? -mag : mag;
}

// The E4M3 code nearest to v, ties to the code with an even mantissa; a
// magnitude above 448 saturates to 448.  By search over the 127 finite
// non-negative codes (their values increase with the code).
inline uint8_t e4m3_from_double(double v) {
    const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
    const double a = std::fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    for (int c = 1; c <= 0x7E; ++c) {
        const double dc = std::fabs(e4m3_value(static_cast<uint8_t>(c)) - a);
        const double db = std::fabs(e4m3_value(static_cast<uint8_t>(best)) - a);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return sign | static_cast<uint8_t>(best);
}

// One block of 32 activations -> (E8M0 scale byte, 32 E4M3 codes), after the
// OCP microscaling conversion: X = 2^(floor(log2 amax) - 8), 8 being the
// exponent of E4M3's largest normal, kept inside E8M0's range [2^-127,
// 2^127]; each element is the E4M3 code nearest to x / X (saturating).  An
// all-zero block takes the scale byte 0 and zero codes.
inline uint8_t mx_block_quantize(const uint16_t* x, uint8_t* codes) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(static_cast<double>(bf16_to_float(x[i]))));
    if (amax == 0.0) {
        for (int i = 0; i < 32; ++i) codes[i] = 0;
        return 0;
    }
    int ex = 0;
    std::frexp(amax, &ex);              // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    int b = (ex - 1) - 8 + 127;
    b = b < 0 ? 0 : b > 254 ? 254 : b;
    for (int i = 0; i < 32; ++i)
        codes[i] = e4m3_from_double(std::ldexp(static_cast<double>(bf16_to_float(x[i])), 127 - b));
    return static_cast<uint8_t>(b);
}

// One output element of A8W4: sum over c ascending of a[c] * w[c] in fp32,
// a[c] = e4m3(code) * 2^(scale - 127) (exact in fp32 within its range).
inline double dot_row_a8w4(const uint8_t* a8, const uint8_t* a_sc, const uint32_t* row_words,
                           const uint8_t* row_scales, int64_t K) {
    float acc = 0.0f;
    for (int64_t c = 0; c < K; ++c) {
        const float a = static_cast<float>(e4m3_value(a8[c])) * e8m0_value(a_sc[c / 32]);
        acc += a * weight_at_mx(row_words, row_scales, c);
    }
    return static_cast<double>(acc);
}

}  // namespace

extern "C" {

int oracle_version(void) { return 1; }

// Threads the OpenMP loops below use (set_num_threads: n >= 1; the
// benchmark's single-thread leg).
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

// ---- element helpers exposed for the pins ---------------------------------

void oracle_bf16_from_f64(const double* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_from_double(x[i]);
}

// Unpack codes [rows, K/8] words -> [rows, K] bytes in 0..15.
void oracle_unpack_codes(const uint32_t* words, int64_t rows, int64_t K, uint8_t* q) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < K; ++c)
            q[r * K + c] = static_cast<uint8_t>(code_at(words + r * (K / 8), c));
}

// Inverse of the above: [rows, K] codes (low 4 bits used) -> [rows, K/8] words.
void oracle_pack_codes(const uint8_t* q, int64_t rows, int64_t K, uint32_t* words) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t wi = 0; wi < K / 8; ++wi) {
            uint32_t w = 0;
            for (int i = 0; i < 8; ++i)
                w |= (static_cast<uint32_t>(q[r * K + wi * 8 + i]) & 0xFu) << (4 * i);
            words[r * (K / 8) + wi] = w;
        }
}

// Dequantised matrix [rows, K] as fp32 (wmode 0 exact, 1 bf16-rounded).
void oracle_dequant(const uint32_t* words, const uint16_t* scales, int64_t rows,
                    int64_t K, int wmode, float* w) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < K; ++c)
            w[r * K + c] = weight_at(words + r * (K / 8), scales + r * (K / 32), c, wmode);
}

// ---- O3: routing metadata, indexed layout ---------------------------------
//
// Chord page, "Two kernel families" and "vLLM integration": the indexed path
// consumes vLLM's sorted_ids / expert_ids / num_tokens_padded, produced into
// over-allocated buffers; Figure 3: activations are not padded, the routing
// indices carry the padding sentinels.  The plain stable counting sort:
//   for each local expert e (ascending), the slots routed to it in ascending
//   flat order f = t*k + j, then sentinels (T*k) up to a multiple of block_m;
//   expert_ids holds e for every block_m block of that segment; experts with
//   no slot get no block; num_tokens_padded is the padded total; the buffers'
//   tails hold the sentinel and -1; row_of[f] is the position of slot f in
//   sorted_ids (or -1 when f is not local).
// Returns 0, or 1 when the capacities are too small (outputs then undefined).
int oracle_moe_align(const int32_t* topk_ids, int T, int top_k, int E_global,
                     const int32_t* expert_map, int E_local, int block_m,
                     int32_t* sorted_ids, int sorted_cap, int32_t* expert_ids,
                     int blocks_cap, int32_t* num_tokens_padded, int32_t* row_of) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    const int32_t sentinel = static_cast<int32_t>(slots);
    std::vector<std::vector<int32_t>> lists(E_local);
    for (int64_t f = 0; f < slots; ++f) {
        int e = local_expert(topk_ids, f, E_global, expert_map, E_local);
        if (e >= 0) lists[e].push_back(static_cast<int32_t>(f));
    }
    int64_t total = 0;
    for (int e = 0; e < E_local; ++e) {
        int64_t c = static_cast<int64_t>(lists[e].size());
        total += (c + block_m - 1) / block_m * block_m;
    }
    if (total > sorted_cap || total / block_m > blocks_cap) return 1;
    if (row_of)
        for (int64_t f = 0; f < slots; ++f) row_of[f] = -1;
    int64_t off = 0;
    for (int e = 0; e < E_local; ++e) {
        int64_t c = static_cast<int64_t>(lists[e].size());
        int64_t p = (c + block_m - 1) / block_m * block_m;
        for (int64_t j = 0; j < p; ++j) {
            int32_t v = j < c ? lists[e][j] : sentinel;
            sorted_ids[off + j] = v;
            if (j < c && row_of) row_of[v] = static_cast<int32_t>(off + j);
        }
        for (int64_t b = 0; b < p / block_m; ++b) expert_ids[off / block_m + b] = e;
        off += p;
    }
    for (int64_t i = off; i < sorted_cap; ++i) sorted_ids[i] = sentinel;
    for (int64_t b = off / block_m; b < blocks_cap; ++b) expert_ids[b] = -1;
    num_tokens_padded[0] = static_cast<int32_t>(off);
    return 0;
}

// GEMM row tiles over the indexed layout: each local expert's routed rows
// (its segment of sorted_ids, which starts at the padded offset off_e) cut in
// order into pieces of at most tile_m rows, {expert, first position, rows, 0},
// experts ascending.  Returns the number of tiles, or -1 when tiles_cap is too
// small.  (The page leaves the schedule of row blocks open; this is the plain
// in-order cut that keeps every piece inside one expert.)
int oracle_moe_tiles(const int32_t* topk_ids, int T, int top_k, int E_global,
                     const int32_t* expert_map, int E_local, int block_m, int tile_m,
                     int32_t* tiles, int tiles_cap) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<int64_t> count(E_local, 0);
    for (int64_t f = 0; f < slots; ++f) {
        int e = local_expert(topk_ids, f, E_global, expert_map, E_local);
        if (e >= 0) ++count[e];
    }
    int64_t off = 0;
    int n = 0;
    for (int e = 0; e < E_local; ++e) {
        for (int64_t s = 0; s < count[e]; s += tile_m) {
            if (n >= tiles_cap) return -1;
            tiles[4 * n + 0] = e;
            tiles[4 * n + 1] = static_cast<int32_t>(off + s);
            tiles[4 * n + 2] = static_cast<int32_t>(count[e] - s < tile_m ? count[e] - s : tile_m);
            tiles[4 * n + 3] = 0;
            ++n;
        }
        off += (count[e] + block_m - 1) / block_m * block_m;
    }
    return n;
}

// ---- O4 / O6: one grouped W4A16 GEMM over an explicit row list ------------
//
// out[r, n] = bf16( sum_{c<K} A[a_row[r], c] * w[expert[r], n, c] ) for every
// r with expert[r] >= 0 (other rows are left untouched).  A is bf16 [*, K];
// codes [E, N, K/8]; scales [E, N, K/32].  out_f32 != 0 writes the fp32
// accumulator instead (float [R, N]).
void oracle_grouped_gemm(const uint16_t* A, const int32_t* a_row, const int32_t* expert,
                         int64_t R, const uint32_t* codes, const uint16_t* scales,
                         int E, int N, int K, int wmode, int acc64, int out_f32,
                         void* out) {
    (void)E;
    const int64_t wpr = K / 8, spr = K / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        int e = expert[r];
        if (e < 0) continue;
        const uint16_t* a = A + static_cast<int64_t>(a_row[r]) * K;
        for (int n = 0; n < N; ++n) {
            const int64_t wr = static_cast<int64_t>(e) * N + n;
            double acc = dot_row(a, codes + wr * wpr, scales + wr * spr, K, wmode, acc64);
            if (out_f32)
                static_cast<float*>(out)[r * N + n] = static_cast<float>(acc);
            else
                static_cast<uint16_t*>(out)[r * N + n] = bf16_from_double(acc);
        }
    }
}

// gate/up for every local slot f (row f of Y13 [T*k, 2I]; token t = f / k).
void oracle_moe_gate_up(const uint16_t* X, const int32_t* topk_ids, int T, int top_k,
                        int E_global, const int32_t* expert_map, int E_local,
                        const uint32_t* codes13, const uint16_t* scales13, int H, int I,
                        int wmode, uint16_t* Y13) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<int32_t> a_row(slots), expert(slots);
    for (int64_t f = 0; f < slots; ++f) {
        a_row[f] = static_cast<int32_t>(f / top_k);
        expert[f] = local_expert(topk_ids, f, E_global, expert_map, E_local);
    }
    oracle_grouped_gemm(X, a_row.data(), expert.data(), slots, codes13, scales13,
                        E_local, 2 * I, H, wmode, 0, 0, Y13);
}

// O5: Z[r, j] = bf16( silu(g) * u ), g = Y13[r, j], u = Y13[r, I + j], in
// fp64 from the bf16 inputs with one final rounding; silu(g) = g / (1 + e^-g).
void oracle_silu_mul(const uint16_t* Y13, int64_t rows, int I, uint16_t* Z) {
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < I; ++j) {
            double g = bf16_to_float(Y13[r * 2 * I + j]);
            double u = bf16_to_float(Y13[r * 2 * I + I + j]);
            double s = g / (1.0 + std::exp(-g));
            Z[r * I + j] = bf16_from_double(s * u);
        }
}

// down for every local slot f (row f of Z [T*k, I] -> row f of Y2 [T*k, H]).
void oracle_moe_down(const uint16_t* Z, const int32_t* topk_ids, int T, int top_k,
                     int E_global, const int32_t* expert_map, int E_local,
                     const uint32_t* codes2, const uint16_t* scales2, int H, int I,
                     int wmode, uint16_t* Y2) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<int32_t> a_row(slots), expert(slots);
    for (int64_t f = 0; f < slots; ++f) {
        a_row[f] = static_cast<int32_t>(f);
        expert[f] = local_expert(topk_ids, f, E_global, expert_map, E_local);
    }
    oracle_grouped_gemm(Z, a_row.data(), expert.data(), slots, codes2, scales2, E_local,
                        H, I, wmode, 0, 0, Y2);
}

// O7: out[t, h] = bf16( sum_{j<k, row_of[t*k+j] >= 0} w[t,j] * Y[row_of[t*k+j], h] )
// in fp32, j ascending (multiply, then add, each rounded).  A token with no
// local slot yields +0.
void oracle_combine(const uint16_t* Y, const int32_t* row_of, const float* topk_w, int T,
                    int top_k, int H, uint16_t* out) {
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < top_k; ++j) {
                int32_t r = row_of[static_cast<int64_t>(t) * top_k + j];
                if (r < 0) continue;
                float y = bf16_to_float(Y[static_cast<int64_t>(r) * H + h]);
                float p = topk_w[static_cast<int64_t>(t) * top_k + j] * y;
                acc = acc + p;
            }
            out[static_cast<int64_t>(t) * H + h] = bf16_from_float(acc);
        }
}

// O8: grouped masked layout.  a3 is [G, max_m, K] (or flat [G*max_m, K]);
// masked_m[g] rows of expert g are valid; the output is flat [G*max_m, N]
// (Chord page, "Grouped SM90 kernels": masked output is flat even for a
// 3-D input, rows past each expert's valid count are to be ignored).  Rows
// past masked_m[g] are left untouched; expected_m plays no part in the result.
void oracle_masked_gemm(const uint16_t* a3, const int32_t* masked_m, int G, int max_m,
                        const uint32_t* codes, const uint16_t* scales, int N, int K,
                        int wmode, uint16_t* out) {
    const int64_t R = static_cast<int64_t>(G) * max_m;
    std::vector<int32_t> a_row(R), expert(R);
    for (int g = 0; g < G; ++g)
        for (int r = 0; r < max_m; ++r) {
            int64_t i = static_cast<int64_t>(g) * max_m + r;
            a_row[i] = static_cast<int32_t>(i);
            expert[i] = (r < masked_m[g]) ? g : -1;
        }
    oracle_grouped_gemm(a3, a_row.data(), expert.data(), R, codes, scales, G, N, K, wmode,
                        0, 0, out);
}

// Grouped contiguous layout (Chord page, "Grouped SM90 kernels": the
// contiguous prefill entry takes a2 [m, K] with rows concatenated per expert,
// each expert's rows padded to a 128-row boundary, and m_indices int32 [m]
// naming each row's expert, -1 on padding rows; the output is [m, N]; Figure
// 3 shows where that padding lives).  For every row r with
// 0 <= m_indices[r] < G: out[r, :] = bf16( A[r, :] . w[m_indices[r]]^T ) in
// fp32 ascending K; every other row is left untouched.
void oracle_contiguous_gemm(const uint16_t* a2, const int32_t* m_indices, int64_t m, int G,
                            const uint32_t* codes, const uint16_t* scales, int N, int K,
                            int wmode, uint16_t* out) {
    std::vector<int32_t> a_row(m), expert(m);
    for (int64_t r = 0; r < m; ++r) {
        a_row[r] = static_cast<int32_t>(r);
        const int32_t e = m_indices[r];
        expert[r] = (e >= 0 && e < G) ? e : -1;
    }
    oracle_grouped_gemm(a2, a_row.data(), expert.data(), m, codes, scales, G, N, K, wmode, 0, 0,
                        out);
}

// ---- MXFP4 weights ------------------------------------------------------------

// Dequantised MXFP4 weights, rows x K, from codes [rows, K/8] and E8M0 scale
// bytes [rows, K/32].
void oracle_dequant_mx(const uint32_t* words, const uint8_t* scales, int64_t rows, int64_t K,
                       float* w) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < K; ++c)
            w[r * K + c] = weight_at_mx(words + r * (K / 8), scales + r * (K / 32), c);
}

// The grouped GEMM of O4 / O6 on MXFP4 weights: out[r, n] = bf16( sum_c
// A[a_row[r], c] * w[expert[r], n, c] ) for every r with expert[r] >= 0.
void oracle_grouped_gemm_mx(const uint16_t* A, const int32_t* a_row, const int32_t* expert,
                            int64_t R, const uint32_t* codes, const uint8_t* scales, int N, int K,
                            uint16_t* out) {
    const int64_t wpr = K / 8, spr = K / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        const int e = expert[r];
        if (e < 0) continue;
        const uint16_t* a = A + static_cast<int64_t>(a_row[r]) * K;
        for (int n = 0; n < N; ++n) {
            const int64_t wr = static_cast<int64_t>(e) * N + n;
            out[r * N + n] = bf16_from_double(dot_row_mx(a, codes + wr * wpr, scales + wr * spr, K));
        }
    }
}

// ---- A8W4 ---------------------------------------------------------------------

int oracle_e4m3_from_double(double v) { return e4m3_from_double(v); }
double oracle_e4m3_value(int b) { return e4m3_value(static_cast<uint8_t>(b)); }

// MXFP8 form of rows x K bf16 activations (K a multiple of 32): E4M3 codes
// [rows, K] and E8M0 scale bytes [rows, K/32].
void oracle_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                           uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / 32; ++b)
            scales[r * (K / 32) + b] = mx_block_quantize(x + r * K + 32 * b, codes + r * K + 32 * b);
}

// The grouped GEMM of O4 / O6 in A8W4: out[r, n] = sum_c a[a_row[r], c] *
// w[expert[r], n, c] over MXFP8 activations and MXFP4 weights, fp32
// accumulation; bf16 out (out_f32 = 0) or fp32.
void oracle_grouped_gemm_a8w4(const uint8_t* A8, const uint8_t* A_sc, const int32_t* a_row,
                              const int32_t* expert, int64_t R, const uint32_t* codes,
                              const uint8_t* scales, int N, int K, int out_f32, void* out) {
    const int64_t wpr = K / 8, spr = K / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        const int e = expert[r];
        if (e < 0) continue;
        const int64_t ar = a_row[r];
        for (int n = 0; n < N; ++n) {
            const int64_t wr = static_cast<int64_t>(e) * N + n;
            const double v = dot_row_a8w4(A8 + ar * K, A_sc + ar * (K / 32), codes + wr * wpr,
                                          scales + wr * spr, K);
            if (out_f32) static_cast<float*>(out)[r * N + n] = static_cast<float>(v);
            else static_cast<uint16_t*>(out)[r * N + n] = bf16_from_double(v);
        }
    }
}

// The whole indexed path O4 -> O7 in A8W4: X is quantized to MXFP8 per token
// row before gate/up, and Z per slot row before down; the other rounding
// points are those of the W4A16 path.
void oracle_moe_forward_a8w4(const uint16_t* X, const int32_t* topk_ids, const float* topk_w,
                             int T, int top_k, int E_global, const int32_t* expert_map,
                             int E_local, const uint32_t* codes13, const uint8_t* scales13,
                             const uint32_t* codes2, const uint8_t* scales2, int H, int I,
                             uint16_t* out, uint16_t* Z_opt, uint16_t* Y2_opt) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<uint16_t> y13(slots * 2 * I, 0), zv, y2v;
    uint16_t* Z = Z_opt;
    uint16_t* Y2 = Y2_opt;
    if (!Z) { zv.resize(slots * I); Z = zv.data(); }
    if (!Y2) { y2v.resize(slots * H); Y2 = y2v.data(); }
    std::memset(Z, 0, slots * I * sizeof(uint16_t));
    std::memset(Y2, 0, slots * H * sizeof(uint16_t));
    std::vector<uint8_t> x8(static_cast<size_t>(T) * H), xs(static_cast<size_t>(T) * (H / 32));
    oracle_quantize_mxfp8(X, T, H, x8.data(), xs.data());
    std::vector<int32_t> tok_row(slots), slot_row(slots), expert(slots), row_of(slots);
    for (int64_t f = 0; f < slots; ++f) {
        tok_row[f] = static_cast<int32_t>(f / top_k);
        slot_row[f] = static_cast<int32_t>(f);
        expert[f] = local_expert(topk_ids, f, E_global, expert_map, E_local);
        row_of[f] = expert[f] >= 0 ? static_cast<int32_t>(f) : -1;
    }
    oracle_grouped_gemm_a8w4(x8.data(), xs.data(), tok_row.data(), expert.data(), slots, codes13,
                             scales13, 2 * I, H, 0, y13.data());
    oracle_silu_mul(y13.data(), slots, I, Z);
    std::vector<uint8_t> z8(slots * I), zs(slots * (I / 32));
    oracle_quantize_mxfp8(Z, slots, I, z8.data(), zs.data());
    oracle_grouped_gemm_a8w4(z8.data(), zs.data(), slot_row.data(), expert.data(), slots, codes2,
                             scales2, H, I, 0, Y2);
    oracle_combine(Y2, row_of.data(), topk_w, T, top_k, H, out);
}

// ---- the step before the expert GEMMs: routing ----------------------------
//
// Router top-k (the pages name an optimised expert routing step ahead of the
// grouped GEMMs and keep it outside their timed unit; the path's weights are
// the softmax of the selected experts' router logits).  For each token t: the
// k experts with the largest logits, largest first, equal logits taken in
// ascending expert id (a stable sort of the ids by decreasing logit); weight j
// = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected logits, in fp64,
// rounded once to fp32.  This equals a softmax over all experts followed by
// top-k and renormalisation over the k kept.  Logits are finite.
void oracle_router_topk(const float* logits, int T, int E, int k, int32_t* ids, float* weights) {
    std::vector<int> order(E);
    for (int t = 0; t < T; ++t) {
        const float* l = logits + static_cast<int64_t>(t) * E;
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [l](int a, int b) { return l[a] > l[b]; });
        const double top = l[order[0]];
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += std::exp(static_cast<double>(l[order[j]]) - top);
        for (int j = 0; j < k; ++j) {
            ids[static_cast<int64_t>(t) * k + j] = order[j];
            weights[static_cast<int64_t>(t) * k + j] =
                static_cast<float>(std::exp(static_cast<double>(l[order[j]]) - top) / den);
        }
    }
}

// Indexed routing -> grouped masked layout (the pages' masked dispatch takes
// rows already placed per expert, [G, max_m, K] with the valid count of each
// expert in masked_m; this is the placement, from topk_ids).  Slots f = t*k +
// j in ascending order; the i-th local slot of expert e goes to row e*max_m +
// i when i < max_m: a3 row = X[f / k], row_of[f] = e*max_m + i.  Non-local
// slots and slots of rank i >= max_m get row_of[f] = -1 (the latter are
// dropped); masked_m[e] = min(count_e, max_m).  Rows of a3 not written keep
// their contents.  Returns the number of dropped local slots.
int oracle_indexed_to_masked(const uint16_t* X, int H, const int32_t* topk_ids, int T, int top_k,
                             int E_global, const int32_t* expert_map, int E_local, int max_m,
                             uint16_t* a3, int32_t* masked_m, int32_t* row_of) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<int32_t> count(E_local, 0);
    int dropped = 0;
    for (int64_t f = 0; f < slots; ++f) {
        row_of[f] = -1;
        const int e = local_expert(topk_ids, f, E_global, expert_map, E_local);
        if (e < 0) continue;
        const int i = count[e]++;
        if (i >= max_m) {
            ++dropped;
            continue;
        }
        const int64_t r = static_cast<int64_t>(e) * max_m + i;
        row_of[f] = static_cast<int32_t>(r);
        std::memcpy(a3 + r * H, X + (f / top_k) * H, sizeof(uint16_t) * H);
    }
    for (int e = 0; e < E_local; ++e) masked_m[e] = count[e] < max_m ? count[e] : max_m;
    return dropped;
}

// Whole indexed path O4 -> O5 -> O6 -> O7 in the slot-indexed layout.
// Intermediates may be NULL; when given they are [T*k, 2I], [T*k, I], [T*k, H]
// (rows of non-local slots are zero).
void oracle_moe_forward(const uint16_t* X, const int32_t* topk_ids, const float* topk_w,
                        int T, int top_k, int E_global, const int32_t* expert_map,
                        int E_local, const uint32_t* codes13, const uint16_t* scales13,
                        const uint32_t* codes2, const uint16_t* scales2, int H, int I,
                        int wmode, uint16_t* out, uint16_t* Y13_opt, uint16_t* Z_opt,
                        uint16_t* Y2_opt) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<uint16_t> y13v, zv, y2v;
    uint16_t* Y13 = Y13_opt;
    uint16_t* Z = Z_opt;
    uint16_t* Y2 = Y2_opt;
    if (!Y13) { y13v.resize(slots * 2 * I); Y13 = y13v.data(); }
    if (!Z) { zv.resize(slots * I); Z = zv.data(); }
    if (!Y2) { y2v.resize(slots * H); Y2 = y2v.data(); }
    std::memset(Y13, 0, slots * 2 * I * sizeof(uint16_t));
    std::memset(Z, 0, slots * I * sizeof(uint16_t));
    std::memset(Y2, 0, slots * H * sizeof(uint16_t));
    oracle_moe_gate_up(X, topk_ids, T, top_k, E_global, expert_map, E_local, codes13,
                       scales13, H, I, wmode, Y13);
    oracle_silu_mul(Y13, slots, I, Z);
    oracle_moe_down(Z, topk_ids, T, top_k, E_global, expert_map, E_local, codes2, scales2,
                    H, I, wmode, Y2);
    std::vector<int32_t> row_of(slots);
    for (int64_t f = 0; f < slots; ++f)
        row_of[f] = local_expert(topk_ids, f, E_global, expert_map, E_local) >= 0
                        ? static_cast<int32_t>(f) : -1;
    oracle_combine(Y2, row_of.data(), topk_w, T, top_k, H, out);
}

// The whole indexed path O4 -> O7 on MXFP4 weights (codes as in the INT4
// path, E8M0 scale bytes instead of bf16 scales); same rounding points.
void oracle_moe_forward_mx(const uint16_t* X, const int32_t* topk_ids, const float* topk_w,
                           int T, int top_k, int E_global, const int32_t* expert_map,
                           int E_local, const uint32_t* codes13, const uint8_t* scales13,
                           const uint32_t* codes2, const uint8_t* scales2, int H, int I,
                           uint16_t* out, uint16_t* Y13_opt, uint16_t* Z_opt, uint16_t* Y2_opt) {
    const int64_t slots = static_cast<int64_t>(T) * top_k;
    std::vector<uint16_t> y13v, zv, y2v;
    uint16_t* Y13 = Y13_opt;
    uint16_t* Z = Z_opt;
    uint16_t* Y2 = Y2_opt;
    if (!Y13) { y13v.resize(slots * 2 * I); Y13 = y13v.data(); }
    if (!Z) { zv.resize(slots * I); Z = zv.data(); }
    if (!Y2) { y2v.resize(slots * H); Y2 = y2v.data(); }
    std::memset(Y13, 0, slots * 2 * I * sizeof(uint16_t));
    std::memset(Z, 0, slots * I * sizeof(uint16_t));
    std::memset(Y2, 0, slots * H * sizeof(uint16_t));
    std::vector<int32_t> tok_row(slots), slot_row(slots), expert(slots), row_of(slots);
    for (int64_t f = 0; f < slots; ++f) {
        tok_row[f] = static_cast<int32_t>(f / top_k);
        slot_row[f] = static_cast<int32_t>(f);
        expert[f] = local_expert(topk_ids, f, E_global, expert_map, E_local);
        row_of[f] = expert[f] >= 0 ? static_cast<int32_t>(f) : -1;
    }
    oracle_grouped_gemm_mx(X, tok_row.data(), expert.data(), slots, codes13, scales13, 2 * I, H,
                           Y13);
    oracle_silu_mul(Y13, slots, I, Z);
    oracle_grouped_gemm_mx(Z, slot_row.data(), expert.data(), slots, codes2, scales2, H, I, Y2);
    oracle_combine(Y2, row_of.data(), topk_w, T, top_k, H, out);
}

// O9: a second, direct formulation used as brute force.  Token by token and
// slot by slot, with the weights dequantised on the fly, no routing metadata
// and no intermediate buffers beyond one row; the same rounding points as the
// staged path, so the two agree bit for bit.
void oracle_direct_forward(const uint16_t* X, const int32_t* topk_ids, const float* topk_w,
                           int T, int top_k, int E_global, const int32_t* expert_map,
                           int E_local, const uint32_t* codes13, const uint16_t* scales13,
                           const uint32_t* codes2, const uint16_t* scales2, int H, int I,
                           int wmode, uint16_t* out) {
    const int64_t wpr13 = H / 8, spr13 = H / 32, wpr2 = I / 8, spr2 = I / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        std::vector<float> acc(H, 0.0f);
        std::vector<uint16_t> z(I);
        const uint16_t* x = X + static_cast<int64_t>(t) * H;
        for (int j = 0; j < top_k; ++j) {
            int g = topk_ids[static_cast<int64_t>(t) * top_k + j];
            if (g < 0 || g >= E_global) continue;
            int e = expert_map ? expert_map[g] : g;
            if (e < 0 || e >= E_local) continue;
            for (int i = 0; i < I; ++i) {
                int64_t rg = static_cast<int64_t>(e) * 2 * I + i;        // gate row
                int64_t ru = rg + I;                                      // up row
                float sg = 0.0f, su = 0.0f;
                for (int c = 0; c < H; ++c) {
                    float xv = bf16_to_float(x[c]);
                    sg += xv * weight_at(codes13 + rg * wpr13, scales13 + rg * spr13, c, wmode);
                    su += xv * weight_at(codes13 + ru * wpr13, scales13 + ru * spr13, c, wmode);
                }
                double gb = bf16_to_float(bf16_from_float(sg));
                double ub = bf16_to_float(bf16_from_float(su));
                z[i] = bf16_from_double(gb / (1.0 + std::exp(-gb)) * ub);
            }
            float wt = topk_w[static_cast<int64_t>(t) * top_k + j];
            for (int h = 0; h < H; ++h) {
                int64_t rd = static_cast<int64_t>(e) * H + h;
                float s = 0.0f;
                for (int c = 0; c < I; ++c)
                    s += bf16_to_float(z[c]) * weight_at(codes2 + rd * wpr2, scales2 + rd * spr2, c, wmode);
                float y = bf16_to_float(bf16_from_float(s));
                float p = wt * y;
                acc[h] = acc[h] + p;
            }
        }
        for (int h = 0; h < H; ++h) out[static_cast<int64_t>(t) * H + h] = bf16_from_float(acc[h]);
    }
}

}  // extern "C"
