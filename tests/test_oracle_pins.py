"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes a part of the oracle with something independent of its code:
exact rational arithmetic (bf16 rounding), closed forms (one-hot rows give a
column of the dequantised matrix), exact-integer invariants (integer
activations with power-of-two scales make every fp32 sum exact), a textbook
special case (one expert, unit scales = a plain matrix product), a
floating-point error bound (fp32 accumulation vs exact), brute force (Python
``sorted`` for the routing sort) and a second, direct formulation of the whole
path.  A plausible slip anywhere in the oracle (wrong nibble order, wrong group
index, gate/up swapped, a dropped offset, a transposed operand, an unstable
sort, an off-by-one in padding) fails at least one of them.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers ----

def f32_of_bf16(b):
    return synth.bf16_bits_to_f32(b)


def bf16_of_exact(x: float) -> int:
    """Round a real number (given exactly) to bf16, ties to even, from the
    definition: pick the nearer of the two neighbouring bf16 values."""
    fx = Fraction(x)
    if fx == 0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if fx < 0 else 0
    a = abs(fx)
    # enumerate: find exponent e with 2^e <= a < 2^(e+1)
    e = math.floor(math.log2(float(a)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp_e = max(e - 7, -133)
    ulp = Fraction(2) ** ulp_e
    lo = (a // ulp) * ulp
    hi = lo + ulp
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:
        r = lo if (lo / ulp) % 2 == 0 else hi
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = np.array([float(r)], dtype=np.float32).view(np.uint32)[0] >> 16
    return sign | int(bits)


def signed_q(codes, K):
    """(q - 8) from hand-written nibble extraction (low nibble = lowest K)."""
    w = np.asarray(codes).view(np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = (w[..., None] >> shifts) & 0xF
    return q.reshape(w.shape[:-1] + (K,)).astype(np.int64) - 8


# ------------------------------------------------------- bf16 rounding pin ----

def test_bf16_rounding_matches_exact_rational_rounding():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(300) * np.exp2(rng.integers(-140, 130, 300)))
    # exact ties between neighbouring bf16 values (must go to the even one)
    for b in [0x3F80, 0x3F81, 0x4000, 0x0001, 0x0002, 0x7F7E, 0x8081]:
        lo = float(f32_of_bf16(np.array([b], np.uint16))[0])
        hi = float(f32_of_bf16(np.array([b + 1], np.uint16))[0])
        vals += [(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0), np.nextafter((lo + hi) / 2, 1e300)]
    vals += [0.0, -0.0, 1.0, -1.0, 3.4e38, 3.5e38, 1e-45, 2.0**-133, 2.0**-134, 3 * 2.0**-135]
    got = oracle.bf16_from_f64(np.array(vals))
    want = np.array([bf16_of_exact(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_special_values():
    got = oracle.bf16_from_f64(np.array([np.inf, -np.inf, np.nan]))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    assert (got[2] & 0x7F80) == 0x7F80 and (got[2] & 0x7F) != 0


# ------------------------------------------------------------- weight format ----

def test_unpack_closed_form_word():
    # nibble i of the word is code i along K
    w = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32).view(np.int32)
    q = oracle.unpack_codes(w, 16)
    assert q.tolist() == [list(range(16))]


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(2)
    w = rng.integers(0, 2**32, size=(3, 5, 12), dtype=np.uint32).view(np.int32)
    q = oracle.unpack_codes(w, 96)
    assert q.max() <= 15
    assert np.array_equal(oracle.pack_codes(q), w)
    q2 = rng.integers(0, 16, size=(7, 64), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q2), 64), q2)


def test_dequant_values_and_offset():
    # codes 0, 8, 15 -> -8 s, 0, 7 s; scale groups of 32 along K
    K = 64
    q = np.zeros((1, K), np.uint8)
    q[0, 0], q[0, 1], q[0, 2] = 0, 8, 15
    q[0, 32], q[0, 33] = 15, 0
    w = oracle.pack_codes(q)
    s = np.array([[0x3F80, 0x4040]], np.uint16)     # 1.0 for group 0, 3.0 for group 1
    d = oracle.dequant(w, s, K)
    assert d[0, 0] == -8.0 and d[0, 1] == 0.0 and d[0, 2] == 7.0
    assert d[0, 3] == -8.0                           # code 0 again
    assert d[0, 32] == 21.0 and d[0, 33] == -24.0


def test_dequant_exact_and_bf16_mode():
    rng = np.random.default_rng(3)
    K = 128
    w = rng.integers(0, 2**32, size=(4, K // 8), dtype=np.uint32).view(np.int32)
    s = synth.random_scales(rng, 1, 4, K)[0]
    d0 = oracle.dequant(w, s, K, 0).astype(np.float64)
    sq = signed_q(w, K)
    sf = np.repeat(f32_of_bf16(s).astype(np.float64), 32, axis=1)
    exact = sq * sf
    assert np.array_equal(d0, exact)                 # exact in fp32
    d1 = oracle.dequant(w, s, K, 1)
    want = np.array([bf16_of_exact(v) for v in exact.ravel()], np.uint16)
    assert np.array_equal(d1.ravel(), f32_of_bf16(want))


# ----------------------------------------------------- one-hot closed form ----

@pytest.mark.parametrize("c", [0, 7, 8, 31, 32, 33, 63, 95])
def test_one_hot_rows_read_out_one_column(c):
    """X = e_c, k = 1, one slot per expert -> Y13[f, n] = bf16((q[e,n,c]-8) s[e,n,c/32])."""
    E, H, I = 3, 96, 32
    rng = np.random.default_rng(10 + c)
    codes = rng.integers(0, 2**32, size=(E, 2 * I, H // 8), dtype=np.uint32).view(np.int32)
    scales = synth.random_scales(rng, E, 2 * I, H)
    X = np.zeros((E, H), np.uint16)
    X[:, c] = 0x3F80
    ids = np.arange(E, dtype=np.int32)[:, None]       # token t -> expert t
    Y = oracle.moe_gate_up(X, ids, E, None, codes, scales)
    q = signed_q(codes, H)[:, :, c]
    s = f32_of_bf16(scales[:, :, c // 32]).astype(np.float64)
    want = np.array([bf16_of_exact(v) for v in (q * s).ravel()], np.uint16).reshape(E, 2 * I)
    assert np.array_equal(Y, want)


def test_gate_is_first_half_up_is_second_half():
    """Make gate = 2 and up = 3 for every j (one-hot X, unit scales): Z = silu(2)*3;
    swapping the halves would give silu(3)*2."""
    E, H, I = 1, 32, 32
    q = np.full((1, 2 * I, H), 8, np.uint8)
    q[0, :I, 0] = 10        # gate rows: weight 2 at c = 0
    q[0, I:, 0] = 11        # up rows:   weight 3 at c = 0
    codes = oracle.pack_codes(q)
    scales = np.full((1, 2 * I, 1), 0x3F80, np.uint16)
    X = np.zeros((1, H), np.uint16)
    X[0, 0] = 0x3F80
    Y13 = oracle.moe_gate_up(X, np.zeros((1, 1), np.int32), 1, None, codes, scales)
    assert np.all(f32_of_bf16(Y13[0, :I]) == 2.0) and np.all(f32_of_bf16(Y13[0, I:]) == 3.0)
    Z = oracle.silu_mul(Y13)
    want = bf16_of_exact(2.0 / (1.0 + math.exp(-2.0)) * 3.0)
    assert np.all(Z == want)
    assert want != bf16_of_exact(3.0 / (1.0 + math.exp(-3.0)) * 2.0)


# -------------------------------------------------- exactness invariant P4 ----

def _exact_problem(seed, E, H, I, T, k):
    rng = np.random.default_rng(seed)
    d = synth.random_small(seed, E, H, I, T, k)
    Xi = rng.integers(-4, 5, size=(T, H))
    d["X"] = synth.bf16_trunc(Xi.astype(np.float32))
    m13 = rng.integers(6, 9, size=(E, 2 * I, H // 32))
    m2 = rng.integers(6, 9, size=(E, H, I // 32))
    d["scales13"] = synth.bf16_trunc(np.exp2(-m13).astype(np.float32))
    d["scales2"] = synth.bf16_trunc(np.exp2(-m2).astype(np.float32))
    d["Xi"] = Xi
    return d


def _exact_gemm(Aint, codes, scales, K):
    """sum_g s_g * sum_{c in g} a_c (q_c - 8) with integers, then exact float64."""
    sq = signed_q(codes, K)                                  # [N, K]
    s = f32_of_bf16(scales).astype(np.float64)               # [N, K/32]
    prod = Aint[:, None, :].astype(np.int64) * sq[None, :, :]  # [R, N, K]
    grp = prod.reshape(prod.shape[0], prod.shape[1], K // 32, 32).sum(-1)
    return (grp * s[None]).sum(-1)                           # exact: small dyadic values


def test_exactness_invariant_gate_up_and_down():
    E, H, I, T, k = 4, 128, 64, 6, 2
    d = _exact_problem(5, E, H, I, T, k)
    Y13 = oracle.moe_gate_up(d["X"], d["topk_ids"], E, None, d["codes13"], d["scales13"])
    for f in range(T * k):
        e = d["topk_ids"].ravel()[f]
        want = _exact_gemm(d["Xi"][f // k][None], d["codes13"][e], d["scales13"][e], H)[0]
        wb = np.array([bf16_of_exact(v) for v in want], np.uint16)
        assert np.array_equal(Y13[f], wb)
    # down on integer Z, standalone
    rng = np.random.default_rng(6)
    Zi = rng.integers(-4, 5, size=(T * k, I))
    Zb = synth.bf16_trunc(Zi.astype(np.float32))
    Y2 = oracle.moe_down(Zb, d["topk_ids"], E, None, d["codes2"], d["scales2"])
    for f in range(T * k):
        e = d["topk_ids"].ravel()[f]
        want = _exact_gemm(Zi[f][None], d["codes2"][e], d["scales2"][e], I)[0]
        assert np.array_equal(Y2[f], np.array([bf16_of_exact(v) for v in want], np.uint16))


def test_exactness_fp32_accumulator_equals_exact_sum():
    E, H, I, T, k = 2, 256, 32, 4, 1
    d = _exact_problem(7, E, H, I, T, k)
    ids = d["topk_ids"]
    acc = oracle.grouped_gemm(d["X"], np.arange(T, dtype=np.int32), ids[:, 0].copy(),
                              d["codes13"], d["scales13"], 2 * I, H, out_f32=True)
    for t in range(T):
        e = ids[t, 0]
        want = _exact_gemm(d["Xi"][t][None], d["codes13"][e], d["scales13"][e], H)[0]
        assert np.array_equal(acc[t].astype(np.float64), want)


# ------------------------------------------------ textbook special case P5 ----

def test_one_expert_unit_scales_is_plain_matmul_within_fp32_bound():
    H, I, T = 512, 64, 9
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 2**32, size=(1, 2 * I, H // 8), dtype=np.uint32).view(np.int32)
    scales = np.full((1, 2 * I, H // 32), 0x3F80, np.uint16)
    X = synth.random_activations(rng, T, H)
    acc = oracle.grouped_gemm(X, np.arange(T, dtype=np.int32), np.zeros(T, np.int32),
                              codes, scales, 2 * I, H, out_f32=True).astype(np.float64)
    Xf = f32_of_bf16(X).astype(np.float64)
    Wf = signed_q(codes[0], H).astype(np.float64)
    exact = Xf @ Wf.T                                    # numpy's own product
    absdot = np.abs(Xf) @ np.abs(Wf).T
    u = 2.0**-24
    gamma = H * u / (1 - H * u)
    assert np.all(np.abs(acc - exact) <= gamma * absdot)
    # and the bf16 output is the RNE of that accumulator
    Yb = oracle.grouped_gemm(X, np.arange(T, dtype=np.int32), np.zeros(T, np.int32),
                             codes, scales, 2 * I, H)
    assert np.array_equal(Yb, oracle.bf16_from_f64(acc))


def test_fp32_accumulation_within_error_bound_of_fp64():
    H, N, T = 1024, 48, 5
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 2**32, size=(1, N, H // 8), dtype=np.uint32).view(np.int32)
    scales = synth.random_scales(rng, 1, N, H)
    X = synth.random_activations(rng, T, H)
    args = (X, np.arange(T, dtype=np.int32), np.zeros(T, np.int32), codes, scales, N, H)
    a32 = oracle.grouped_gemm(*args, out_f32=True).astype(np.float64)
    Xf = f32_of_bf16(X).astype(np.float64)
    Wf = signed_q(codes[0], H) * np.repeat(f32_of_bf16(scales[0]).astype(np.float64), 32, 1)
    exact = Xf @ Wf.T
    gamma = H * 2.0**-24 / (1 - H * 2.0**-24)
    assert np.all(np.abs(a32 - exact) <= gamma * (np.abs(Xf) @ np.abs(Wf).T))


# ----------------------------------------------------------- routing P6 ----

def _brute_align(ids, E_global, E_local, block_m, expert_map):
    T, k = ids.shape
    slots = T * k
    pairs = []
    for f in range(slots):
        g = int(ids.ravel()[f])
        if g < 0 or g >= E_global:
            continue
        e = int(expert_map[g]) if expert_map is not None else g
        if 0 <= e < E_local:
            pairs.append((e, f))
    pairs = sorted(pairs)
    sorted_ids, expert_ids = [], []
    for e in range(E_local):
        seg = [f for (ee, f) in pairs if ee == e]
        if not seg:
            continue
        pad = -len(seg) % block_m
        sorted_ids += seg + [slots] * pad
        expert_ids += [e] * ((len(seg) + pad) // block_m)
    return sorted_ids, expert_ids


@pytest.mark.parametrize("T,k,Eg,El,bm", [(16, 2, 8, 8, 16), (64, 8, 384, 48, 16),
                                           (37, 3, 10, 4, 8), (5, 2, 6, 6, 1), (1, 1, 4, 4, 64),
                                           (200, 8, 64, 64, 32)])
def test_align_matches_brute_force_sort(T, k, Eg, El, bm):
    rng = np.random.default_rng(T * 7 + k)
    ids = np.argsort(rng.random((T, Eg)), axis=1)[:, :k].astype(np.int32)
    ids.ravel()[rng.integers(0, T * k, 3)] = [-1, Eg, Eg + 5]     # out-of-range ids: skipped
    em = None
    if El != Eg:
        em = np.full(Eg, -1, np.int32)
        em[rng.permutation(Eg)[:El]] = np.arange(El, dtype=np.int32)
    r = oracle.moe_align(ids, Eg, El, bm, expert_map=em)
    want_s, want_e = _brute_align(ids, Eg, El, bm, em)
    n = r["num_tokens_padded"]
    assert n == len(want_s)
    assert r["sorted_ids"][:n].tolist() == want_s
    assert r["expert_ids"][: n // bm].tolist() == want_e
    assert np.all(r["sorted_ids"][n:] == T * k) and np.all(r["expert_ids"][n // bm:] == -1)
    # invariants
    valid = r["sorted_ids"][:n][r["sorted_ids"][:n] < T * k]
    assert len(set(valid.tolist())) == valid.size
    ro = r["row_of"]
    for f in range(T * k):
        if ro[f] >= 0:
            assert r["sorted_ids"][ro[f]] == f
    assert (ro >= 0).sum() == valid.size


def test_align_capacity_error():
    ids = np.zeros((4, 1), np.int32)
    with pytest.raises(ValueError):
        oracle.moe_align(ids, 1, 1, 16, sorted_cap=8, blocks_cap=4)


# ----------------------------------------------------------------- SiLU P7 ----

def _bf16_of_f64_vec(v):
    """Independent double -> bf16 (RNE) via integer rounding of float64 bits;
    normal bf16 range only (callers keep |v| >= 2^-126 or v == 0)."""
    v = np.asarray(v, np.float64)
    bits = v.view(np.uint64)
    drop = np.uint64(52 - 7)
    lsb = (bits >> drop) & np.uint64(1)
    r = (bits + (np.uint64(1) << (drop - np.uint64(1))) - np.uint64(1) + lsb) >> drop << drop
    f = r.view(np.float64).astype(np.float32)          # exact: 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_silu_over_all_finite_bf16_inputs():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = f32_of_bf16(b).astype(np.float64)
    ok = np.isfinite(g)
    b, g = b[ok], g[ok]
    Y13 = np.stack([b, np.full_like(b, 0x3F80)], axis=1)          # I = 1, up = 1
    Z = oracle.silu_mul(Y13)[:, 0]
    ref = np.array([x / (1.0 + math.exp(-x)) if x > -700 else 0.0 for x in g])
    normal = (np.abs(ref) >= 2.0**-126) | (ref == 0)
    assert np.array_equal(Z[normal] & 0x7FFF, _bf16_of_f64_vec(np.abs(ref[normal])))
    # closed forms
    assert Z[b == 0][0] == 0
    big = g > 20
    assert np.array_equal(Z[big], b[big])                # silu(x) = x to bf16 precision
    neg = g < -100
    assert np.all(f32_of_bf16(Z[neg]) == 0)


# -------------------------------------------------------------- combine P8 ----

def test_combine_equal_rows_and_power_of_two_weights():
    rng = np.random.default_rng(11)
    T, k, H = 3, 4, 64
    Y = synth.random_activations(rng, 5, H)
    row_of = np.array([0, 0, 0, 0, 1, -1, 1, 1, 2, 3, 4, -1], np.int32)
    w = np.array([[0.25, 0.25, 0.25, 0.25], [0.5, 0.9, 0.25, 0.25], [0.5, 0.25, 0.125, 7.0]],
                 np.float32)
    out = oracle.combine(Y, row_of, w)
    assert np.array_equal(out[0], Y[0])                  # k equal rows, weights sum to 1
    assert np.array_equal(out[1], Y[1])                  # non-local slot ignored
    yf = f32_of_bf16(Y).astype(np.float64)
    exact = 0.5 * yf[2] + 0.25 * yf[3] + 0.125 * yf[4]
    assert np.array_equal(out[2], np.array([bf16_of_exact(v) for v in exact], np.uint16))
    out0 = oracle.combine(Y, np.full(T * k, -1, np.int32), w)
    assert np.all(out0 == 0)                             # no local slot -> +0


# ---------------------------------------------- brute force P1 and masked ----

@pytest.mark.parametrize("seed,E,H,I,T,k,Eg", [(0, 4, 64, 32, 8, 3, 4), (1, 3, 32, 64, 5, 2, 7),
                                               (2, 8, 256, 128, 16, 2, 8), (3, 2, 96, 32, 6, 1, 2)])
def test_staged_path_equals_direct_formulation(seed, E, H, I, T, k, Eg):
    d = synth.random_small(seed, E, H, I, T, k, E_global=Eg)
    args = (d["X"], d["topk_ids"], d["topk_weights"], Eg, d["expert_map"], d["codes13"],
            d["scales13"], d["codes2"], d["scales2"])
    for wmode in (0, 1):
        staged = oracle.moe_forward(*args, wmode=wmode)
        direct = oracle.direct_forward(*args, wmode=wmode)
        assert np.array_equal(staged, direct)


def test_tiny_workload_staged_equals_direct():
    d = synth.make_workload("tiny", seed=0)
    wl = d["wl"]
    args = (d["X"], d["topk_ids"], d["topk_weights"], wl.E_global, d["expert_map"],
            d["codes13"], d["scales13"], d["codes2"], d["scales2"])
    assert np.array_equal(oracle.moe_forward(*args), oracle.direct_forward(*args))


def test_masked_layout_equals_row_list_gemm_and_ignores_padding():
    rng = np.random.default_rng(12)
    G, max_m, K, N = 4, 8, 64, 32
    counts = np.array([3, 0, 8, 5], np.int32)
    a3 = np.full((G, max_m, K), 0x7FC0, np.uint16)                 # NaN poison
    for g in range(G):
        a3[g, : counts[g]] = synth.random_activations(rng, counts[g], K)
    codes = rng.integers(0, 2**32, size=(G, N, K // 8), dtype=np.uint32).view(np.int32)
    scales = synth.random_scales(rng, G, N, K)
    sentinel = np.full((G * max_m, N), 0xABCD, np.uint16)
    out = oracle.masked_gemm(a3, counts, codes, scales, out=sentinel.copy())
    for g in range(G):
        rows = g * max_m + np.arange(max_m)
        valid = rows[: counts[g]]
        ref = oracle.grouped_gemm(a3.reshape(G * max_m, K), valid.astype(np.int32),
                                  np.full(valid.size, g, np.int32), codes, scales, N, K)
        assert np.array_equal(out[valid], ref)
        assert np.all(out[rows[counts[g]:]] == 0xABCD)             # untouched
    assert not np.any(np.isnan(f32_of_bf16(out[out != 0xABCD])))


@pytest.mark.parametrize("T,k,Eg,El,bm,tm", [(64, 8, 384, 48, 16, 32), (37, 3, 10, 4, 8, 16),
                                              (300, 8, 16, 16, 16, 64)])
def test_tiles_cover_each_expert_segment_in_order(T, k, Eg, El, bm, tm):
    """Brute force: the tiles of expert e are its valid rows [off_e, off_e + c_e) cut
    into consecutive pieces of at most tm rows, experts ascending."""
    rng = np.random.default_rng(T + tm)
    ids = np.argsort(rng.random((T, Eg)), axis=1)[:, :k].astype(np.int32)
    em = None
    if El != Eg:
        em = np.full(Eg, -1, np.int32)
        em[:El] = np.arange(El, dtype=np.int32)
    tiles = oracle.moe_tiles(ids, Eg, El, bm, tm, em)
    al = oracle.moe_align(ids, Eg, El, bm, em)
    s = al["sorted_ids"]
    want = []
    p = 0
    while p < al["num_tokens_padded"]:
        e = al["expert_ids"][p // bm]
        seg_end = p
        while seg_end < al["num_tokens_padded"] and al["expert_ids"][seg_end // bm] == e:
            seg_end += bm
        valid = [q for q in range(p, seg_end) if s[q] < T * k]
        for i in range(0, len(valid), tm):
            piece = valid[i:i + tm]
            assert piece == list(range(piece[0], piece[0] + len(piece)))
            want.append([e, piece[0], len(piece), 0])
        p = seg_end
    assert tiles.tolist() == want


# ------------------------------------------------ grouped contiguous layout ----

def _contiguous_layout(counts, align=128):
    """m_indices of the contiguous layout: each expert's rows concatenated,
    padded to a multiple of `align` with -1 (experts with no rows take no
    space)."""
    mi = []
    for e, c in enumerate(counts):
        if c == 0:
            continue
        p = -(-c // align) * align
        mi += [e] * c + [-1] * (p - c)
    return np.array(mi, np.int32)


def test_contiguous_exactness_invariant_and_padding_rows_untouched():
    """Integer activations and power-of-two scales make every product and sum
    exact, so each valid row is the exact integer-arithmetic product rounded
    once to bf16; padding rows (NaN-poisoned activations, index -1) keep the
    output's previous contents."""
    rng = np.random.default_rng(21)
    G, K, N = 4, 128, 32
    counts = [5, 0, 130, 17]
    mi = _contiguous_layout(counts)
    m = mi.size
    assert m == 128 + 256 + 128
    Ai = rng.integers(-4, 5, size=(m, K))
    A = synth.bf16_trunc(Ai.astype(np.float32))
    A[mi < 0] = 0x7FC0
    codes = rng.integers(0, 2**32, size=(G, N, K // 8), dtype=np.uint32).view(np.int32)
    scales = synth.bf16_trunc(np.exp2(-rng.integers(6, 9, size=(G, N, K // 32))).astype(np.float32))
    out = oracle.contiguous_gemm(A, mi, codes, scales, out=np.full((m, N), 0xABCD, np.uint16))
    for r in range(m):
        e = mi[r]
        if e < 0:
            assert np.all(out[r] == 0xABCD)
            continue
        want = _exact_gemm(Ai[r][None], codes[e], scales[e], K)[0]
        assert np.array_equal(out[r], np.array([bf16_of_exact(v) for v in want], np.uint16))


@pytest.mark.parametrize("c", [0, 9, 32, 63])
def test_contiguous_one_hot_rows_read_their_own_expert(c):
    """A row that is the unit vector e_c reads out column c of its own
    expert's dequantised matrix: (q[e, n, c] - 8) * s[e, n, c / 32], rounded
    to bf16 (rows of three experts, and of an index past the experts, which is
    treated as padding)."""
    rng = np.random.default_rng(30 + c)
    G, K, N = 3, 64, 16
    mi = np.array([2, 2, 0, 1, 1, 1, -1, 7], np.int32)
    A = np.zeros((mi.size, K), np.uint16)
    A[:, c] = 0x3F80
    codes = rng.integers(0, 2**32, size=(G, N, K // 8), dtype=np.uint32).view(np.int32)
    scales = synth.random_scales(rng, G, N, K)
    out = oracle.contiguous_gemm(A, mi, codes, scales, out=np.full((mi.size, N), 0x1111, np.uint16))
    q = signed_q(codes, K)[:, :, c]
    s = f32_of_bf16(scales[:, :, c // 32]).astype(np.float64)
    for r, e in enumerate(mi):
        if e < 0 or e >= G:
            assert np.all(out[r] == 0x1111)
        else:
            want = np.array([bf16_of_exact(v) for v in q[e] * s[e]], np.uint16)
            assert np.array_equal(out[r], want)


# ------------------------------------------------------------- routing step ----

def test_router_equal_logits_give_lowest_ids_and_equal_weights():
    """All logits equal: the k lowest expert ids, each weight exactly 1/k (k a
    power of two)."""
    ids, w = oracle.router_topk(np.full((3, 12), 0.75, np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == np.float32(0.25))


def test_router_two_experts_closed_form():
    """Two selected logits ln 3 apart: weights 3/4 and 1/4 (to fp32 rounding of
    the logits), largest first; the unselected logits play no part."""
    lg = np.array([[-5.0, np.log(3.0), 0.0, -7.0]], np.float32)
    ids, w = oracle.router_topk(lg, 2)
    assert ids.tolist() == [[1, 2]]
    assert abs(float(w[0, 0]) - 0.75) < 1e-6 and abs(float(w[0, 1]) - 0.25) < 1e-6


def test_router_matches_full_softmax_then_topk_then_renormalise():
    """Softmax over all experts, keep the k largest probabilities (stable by
    id), renormalise: the same experts in the same order and the same weights
    within fp32 rounding (numpy fp64 as the second formulation)."""
    rng = np.random.default_rng(40)
    T, E, k = 50, 384, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[0, 10] = lg[0, 20] = lg[0, 5] = 9.0                 # a tie among the largest
    ids, w = oracle.router_topk(lg, k)
    p = np.exp(lg.astype(np.float64) - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = np.stack([np.lexsort((np.arange(E), -p[t]))[:k] for t in range(T)])
    assert np.array_equal(ids, want)
    assert ids[0, :3].tolist() == [5, 10, 20]
    sel = np.take_along_axis(p, want, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=2e-7, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def _place_brute_force(X, ids, em, E, max_m):
    """Independent placement: local slots grouped by expert with a stable
    argsort, rank within the expert from the sorted order."""
    T, k = ids.shape
    g = ids.ravel()
    loc = np.where((g >= 0) & (g < len(em)), em[np.clip(g, 0, len(em) - 1)], -1)
    f_local = np.nonzero(loc >= 0)[0]
    order = f_local[np.argsort(loc[f_local], kind="stable")]
    row_of = np.full(T * k, -1, np.int64)
    a3 = np.full((E * max_m, X.shape[1]), 0xDEAD, np.uint16)
    mm = np.zeros(E, np.int64)
    dropped = 0
    for e in range(E):
        fs = order[loc[order] == e]
        mm[e] = min(fs.size, max_m)
        dropped += max(0, fs.size - max_m)
        for i, f in enumerate(fs[:max_m]):
            row_of[f] = e * max_m + i
            a3[e * max_m + i] = X[f // k]
    return a3, mm, row_of, dropped


@pytest.mark.parametrize("T,k,Eg,E,max_m", [(20, 3, 10, 4, 32), (64, 8, 40, 12, 16), (5, 2, 6, 6, 1)])
def test_indexed_to_masked_matches_brute_force(T, k, Eg, E, max_m):
    """Every local slot lands in its expert's rows in ascending slot order;
    slots past max_m are dropped and counted; non-local and out-of-range ids
    map to -1; rows never written keep their contents."""
    rng = np.random.default_rng(T + max_m)
    ids = np.argsort(rng.random((T, Eg)), axis=1)[:, :k].astype(np.int32)
    ids[0, 0] = -3
    em = np.full(Eg, -1, np.int32)
    em[rng.permutation(Eg)[:E]] = rng.permutation(E).astype(np.int32)
    X = synth.random_activations(rng, T, 64)
    a3, mm, row_of, dropped = oracle.indexed_to_masked(
        X, ids, Eg, em, E, max_m, a3=np.full((E * max_m, 64), 0xDEAD, np.uint16))
    wa3, wmm, wrow, wdrop = _place_brute_force(X, ids, em, E, max_m)
    assert np.array_equal(a3, wa3) and np.array_equal(mm, wmm)
    assert np.array_equal(row_of, wrow) and dropped == wdrop
    if max_m == 1:
        assert dropped > 0


# ----------------------------------------------------------------- MXFP4 ----

# E2M1 values of codes 0..15 as the OCP microscaling format fixes them
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_mxfp4_code_and_scale_values():
    """Every E2M1 code (low nibble = lowest K) and E8M0 scales 127 (1), 0
    (2^-127), 254 (2^127 with code 0.5), 124 (1/8); 255 reads as NaN."""
    words = oracle.pack_codes(np.arange(32, dtype=np.uint8).reshape(1, 32) % 16)
    for b, sc in [(127, 1.0), (0, 2.0 ** -127), (124, 0.125)]:
        w = oracle.dequant_mx(words, np.array([[b]], np.uint8), 32)[0]
        want = np.array(E2M1_TABLE * 2, np.float64) * sc
        assert np.array_equal(w.astype(np.float64), want)
        assert np.array_equal(np.signbit(w[8:16]), np.ones(8, bool))
    w = oracle.dequant_mx(words, np.array([[254]], np.uint8), 32)[0]
    assert w[1] == 2.0 ** 126
    assert np.all(np.isnan(oracle.dequant_mx(words, np.array([[255]], np.uint8), 32)[0]))


@pytest.mark.parametrize("c", [0, 7, 8, 31, 33, 63])
def test_mxfp4_one_hot_reads_a_column(c):
    """X = e_c reads column c of the dequantised MXFP4 matrix, each value
    E2M1(q) * 2^(b - 127) exact in bf16."""
    rng = np.random.default_rng(60 + c)
    E, N, K = 2, 16, 64
    codes = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    sc = rng.integers(118, 130, size=(E, N, K // 32)).astype(np.uint8)
    X = np.zeros((1, K), np.uint16)
    X[0, c] = 0x3F80
    q = (codes.view(np.uint32)[..., c // 8] >> (4 * (c % 8))) & 0xF
    for e in range(E):
        got = oracle.grouped_gemm_mx(X, np.zeros(1, np.int32), np.array([e], np.int32), codes,
                                     sc, N, K)[0]
        # the fp32 sum starts at +0, so a code of -0 reads as +0
        want = [bf16_of_exact(E2M1_TABLE[int(q[e, n])] * 2.0 ** (int(sc[e, n, c // 32]) - 127)
                              + 0.0) if E2M1_TABLE[int(q[e, n])] != 0 else 0
                for n in range(N)]
        assert np.array_equal(got, np.array(want, np.uint16))


def test_mxfp4_path_equals_int4_path_on_shared_values():
    """MXFP4 weights whose values all lie in {0, +-1, +-2, +-3, +-4, +-6} x 2^k are
    INT4 weights too (q = v + 8, bf16 scale 2^k): the MXFP4 path must then give
    the INT4 path's bits exactly, through gate/up, SiLU, down and combine."""
    rng = np.random.default_rng(70)
    E, H, I, T, k = 3, 128, 64, 7, 2
    d = synth.random_small(70, E, H, I, T, k)
    shared = [0, 2, 4, 5, 6, 7, 10, 12, 13, 14, 15]          # codes whose E2M1 value is an integer
    def mx_and_int4(N, K):
        qmx = rng.choice(shared, size=(E, N, K))
        b = rng.integers(119, 123, size=(E, N, K // 32)).astype(np.uint8)
        vals = np.array(E2M1_TABLE)[qmx]
        qint = (vals + 8).astype(np.uint8)
        sbf = synth.bf16_trunc(np.exp2(b.astype(np.float64) - 127).astype(np.float32))
        return (oracle.pack_codes(qmx.astype(np.uint8)), b,
                oracle.pack_codes(qint), sbf)
    c13, s13, i13, b13 = mx_and_int4(2 * I, H)
    c2, s2, i2, b2 = mx_and_int4(H, I)
    mx = oracle.moe_forward_mx(d["X"], d["topk_ids"], d["topk_weights"], E, None, c13, s13, c2, s2,
                               intermediates=True)
    ref = oracle.moe_forward(d["X"], d["topk_ids"], d["topk_weights"], E, None, i13, b13, i2, b2,
                             intermediates=True)
    for key in ("Y13", "Z", "Y2", "out"):
        assert np.array_equal(mx[key], ref[key]), key


# ------------------------------------------------------------------ A8W4 ----

def test_e4m3_values_closed_forms():
    """E4M3 bytes by the format's definition: 1.0, the largest finite 448, the
    smallest subnormal 2^-9, the smallest normal 2^-6, -3, -0 and the two NaNs."""
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0xC4) == -3.0
    v = oracle.e4m3_value(0x80)
    assert v == 0.0 and np.signbit(v)
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_rounding_matches_torch_and_saturates():
    """Nearest-even E4M3 rounding against torch's float8_e4m3fn conversion on
    every code, every midpoint between neighbouring codes (ties) and random
    values up to torch's last non-NaN input; beyond 448 + 16 the encoder
    saturates to 448."""
    import torch
    vals = [oracle.e4m3_value(b) for b in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    rng = np.random.default_rng(80)
    rand = list(rng.uniform(-463.9, 463.9, 2000)) + list(np.exp2(rng.uniform(-12, 8, 2000)))
    xs = np.array(vals + mids + [-v for v in mids] + rand, np.float32)
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_from_double(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, want)
    assert oracle.e4m3_from_double(1e6) == 0x7E and oracle.e4m3_from_double(-470.0) == 0xFE


def test_mxfp8_block_scale_and_codes():
    """Block rules of the microscaling conversion: amax = 2^k gives scale byte
    k - 8 + 127 and code 0x78 (256) for that element; amax = 3 * 2^k gives
    k + 1 - 8 + 127 and 0x7C (384), 1.5 * 2^k gives k - 8 + 127 and 0x7C; an all-zero block gives byte 0 and zero
    codes; other elements are x / 2^(b - 127) rounded as torch rounds them."""
    import torch
    rng = np.random.default_rng(81)
    for k_exp, mant, b_want, c_want in [(0, 1.0, 119, 0x78), (5, 3.0, 125, 0x7C),
                                        (-20, 1.0, 99, 0x78), (100, 1.5, 219, 0x7C)]:
        x = rng.uniform(-1, 1, 32) * mant * 2.0 ** k_exp * 0.9
        x[7] = mant * 2.0 ** k_exp
        xb = synth.bf16_trunc(x.astype(np.float32)).reshape(1, 32)
        codes, sc = oracle.quantize_mxfp8(xb)
        assert sc[0, 0] == b_want and codes[0, 7] == c_want
        xf = synth.bf16_bits_to_f32(xb[0]).astype(np.float64) / 2.0 ** (int(sc[0, 0]) - 127)
        want = torch.from_numpy(xf.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(codes[0], want.numpy())
    codes, sc = oracle.quantize_mxfp8(np.zeros((1, 64), np.uint16))
    assert np.all(codes == 0) and np.all(sc == 0)


def test_mxfp8_quantization_error_bound():
    """Every element of a block lies within half an E4M3 step of x: 2^-4 |x|
    in the normal range, 2^-10 X below it (X the block scale); elements of
    blocks whose amax/X exceeds 448 saturate at 448 X."""
    rng = np.random.default_rng(82)
    x = synth.bf16_trunc((rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1))))
                         .astype(np.float32))
    codes, sc = oracle.quantize_mxfp8(x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    X = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    deq = np.vectorize(oracle.e4m3_value)(codes) * X
    err = np.abs(deq - xf)
    sat = np.abs(xf) > 448 * X
    assert np.all(np.abs(deq[sat]) == 448 * X[sat])
    ok = ~sat
    assert np.all(err[ok] <= np.maximum(np.abs(xf[ok]) * 2.0 ** -4, X[ok] * 2.0 ** -10))


def test_a8w4_gemm_reads_dequantized_activations():
    """The A8W4 GEMM on MXFP8 activations equals the MXFP4 GEMM on the
    activations' dequantised values (exact in bf16), bit for bit; and a one-hot
    MXFP8 row reads one weight column times e4m3 * 2^(b - 127)."""
    rng = np.random.default_rng(83)
    E, N, K, R = 3, 32, 128, 20
    codes = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    ws = rng.integers(120, 134, size=(E, N, K // 32)).astype(np.uint8)
    X = synth.bf16_trunc(rng.standard_normal((R, K)).astype(np.float32))
    x8, xs = oracle.quantize_mxfp8(X)
    deq = np.vectorize(oracle.e4m3_value)(x8) * np.repeat(np.exp2(xs.astype(np.float64) - 127), 32, 1)
    Xd = synth.bf16_trunc(deq.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(Xd).astype(np.float64), deq)   # exact in bf16
    a_row = np.arange(R, dtype=np.int32)
    ex = rng.integers(-1, E, R).astype(np.int32)
    got = oracle.grouped_gemm_a8w4(x8, xs, a_row, ex, codes, ws, N, K)
    want = oracle.grouped_gemm_mx(Xd, a_row, ex, codes, ws, N, K)
    assert np.array_equal(got[ex >= 0], want[ex >= 0])
    # one-hot: code 0x44 (3) at K position 37 with scale byte 130 (x8)
    a8 = np.zeros((1, K), np.uint8); a8[0, 37] = 0x44
    asc = np.full((1, K // 32), 127, np.uint8); asc[0, 1] = 130
    w = oracle.dequant_mx(codes, ws, K)
    for e in range(E):
        got = oracle.grouped_gemm_a8w4(a8, asc, np.zeros(1, np.int32), np.array([e], np.int32),
                                       codes, ws, N, K, out_f32=True)[0]
        assert np.array_equal(got.astype(np.float64), 24.0 * w[e, :, 37].astype(np.float64) + 0.0)


def test_a8w4_forward_is_the_composition_and_close_to_mxfp4():
    """The A8W4 indexed path equals its stages run one by one (X quantized per
    token, Z per slot row), and stays close to the bf16-activation MXFP4 path
    on the same weights (the activations' 3-bit mantissas cost at most a few
    per cent)."""
    rng = np.random.default_rng(84)
    E, H, I, T, k = 4, 256, 128, 9, 2
    d = synth.random_small(84, E, H, I, T, k)
    w = synth.make_weights_mxfp4(E, H, I, seed=84)
    r = oracle.moe_forward_a8w4(d["X"], d["topk_ids"], d["topk_weights"], E, None, w["codes13"],
                                w["scales13"], w["codes2"], w["scales2"], intermediates=True)
    slots = T * k
    ex = d["topk_ids"].ravel().astype(np.int32)
    x8, xs = oracle.quantize_mxfp8(d["X"])
    y13 = oracle.grouped_gemm_a8w4(x8, xs, np.arange(slots, dtype=np.int32) // k, ex,
                                   w["codes13"], w["scales13"], 2 * I, H)
    z = oracle.silu_mul(y13)
    assert np.array_equal(z, r["Z"])
    z8, zs = oracle.quantize_mxfp8(z)
    y2 = oracle.grouped_gemm_a8w4(z8, zs, np.arange(slots, dtype=np.int32), ex, w["codes2"],
                                  w["scales2"], H, I)
    assert np.array_equal(y2, r["Y2"])
    out = oracle.combine(y2, np.arange(slots, dtype=np.int32), d["topk_weights"])
    assert np.array_equal(out, r["out"])
    ref = oracle.moe_forward_mx(d["X"], d["topk_ids"], d["topk_weights"], E, None, w["codes13"],
                                w["scales13"], w["codes2"], w["scales2"])
    a = synth.bf16_bits_to_f32(r["out"]).astype(np.float64)
    b = synth.bf16_bits_to_f32(ref).astype(np.float64)
    assert np.abs(a - b).max() <= 0.1 * np.abs(b).max()
