"""Seeded synthetic inputs for the W4A16 INT4 MoE expert path.

This module only draws random numbers and lays them out in the boundary
formats; it holds none of the path's arithmetic (no dequantisation, no routing
sort, no GEMM, no activation, no combine).  Both the CPU oracle and the HIP path
consume exactly the arrays produced here, so the two sides always see identical
bytes.

Formats produced (all numpy, little-endian):
  * activations  : uint16 bf16 bit patterns, X ~ N(0, 1) truncated to bf16
  * weight codes : int32 [E, N, K/8]; uniform random 32-bit words, i.e. eight
                   independent uniform 4-bit codes per word
  * group scales : uint16 bf16 [E, N, K/32] ~ U(0.005, 0.02) truncated to bf16
  * topk_ids     : int32 [T, k] global expert ids, distinct within a token
  * topk_weights : float32 [T, k], softmax over k N(0,1) router logits
  * expert_map   : int32 [E_global], global id -> local id or -1

Workloads (the Kimi-K2.x-like serving shapes used throughout):
  tiny     8 experts, top-2, hidden 256, intermediate 128, 16 tokens
  decode   one GPU's EP8 share: 48 of 384 experts, hidden 7168, intermediate
           2048, 64 tokens, each picking 8 distinct *local* experts
           (about 9-15 routed rows per local expert)
  prefill  same 48-expert share, 8192 tokens top-8 over 384 experts with a
           +-30% per-expert imbalance on the local experts
  tp8      all 384 experts with the intermediate dimension cut to 256,
           1024 tokens, uniform top-8
  masked   grouped-masked decode share: 12 local experts (EP32), 256 routed
           rows with Zipf(1.2) counts, 3 empty experts, padded to a multiple
           of expected_m = 32
  contiguous  grouped-contiguous prefill share: 48 local experts (EP8), 768
           tokens x top-8 over the local experts with exactly 128 rows per
           expert, dispatched into the contiguous layout (rows concatenated
           per expert, segments padded to 128 rows, m_indices)
"""
from __future__ import annotations

import dataclasses
import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens
    top_k: int
    E_global: int
    E_local: int
    H: int              # hidden (K of gate/up, N of down)
    I: int              # intermediate (gate/up each I wide; K of down)
    routing: str        # "uniform" | "local_distinct" | "gumbel_imbalance" | "masked_zipf"
    masked_rows: int = 0
    zipf_s: float = 0.0
    empty_experts: int = 0
    expected_m: int = 0
    rows_per_expert: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", T=16, top_k=2, E_global=8, E_local=8, H=256, I=128,
                     routing="uniform"),
    "decode": Workload("decode", T=64, top_k=8, E_global=384, E_local=48, H=7168,
                       I=2048, routing="local_distinct"),
    "prefill": Workload("prefill", T=8192, top_k=8, E_global=384, E_local=48,
                        H=7168, I=2048, routing="gumbel_imbalance"),
    "tp8": Workload("tp8", T=1024, top_k=8, E_global=384, E_local=384, H=7168,
                    I=256, routing="uniform"),
    "masked": Workload("masked", T=256, top_k=8, E_global=384, E_local=12, H=7168,
                       I=2048, routing="masked_zipf", masked_rows=256, zipf_s=1.2,
                       empty_experts=3, expected_m=32),
    "contiguous": Workload("contiguous", T=768, top_k=8, E_global=384, E_local=48, H=7168,
                           I=2048, routing="balanced_local", rows_per_expert=128),
}


def _streams(seed: int, n: int = 8):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def bf16_trunc(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns by dropping the low 16 bits.

    Used only to *draw* bf16 inputs; it is a sampling choice, not a rounding
    rule of the path.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_codes(rng, E: int, N: int, K: int) -> np.ndarray:
    """int32 [E, N, K/8]: every bit uniform, so every 4-bit code is uniform."""
    assert K % 8 == 0
    return rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)


def random_scales(rng, E: int, N: int, K: int, lo=0.005, hi=0.02) -> np.ndarray:
    assert K % 32 == 0
    return bf16_trunc(rng.uniform(lo, hi, size=(E, N, K // 32)).astype(np.float32))


def random_activations(rng, rows: int, K: int) -> np.ndarray:
    return bf16_trunc(rng.standard_normal((rows, K), dtype=np.float32))


def _softmax_weights(rng, T: int, k: int) -> np.ndarray:
    logits = rng.standard_normal((T, k)).astype(np.float64)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def _distinct_uniform(rng, T: int, k: int, n: int) -> np.ndarray:
    keys = rng.random((T, n))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def expert_map_for(wl: Workload) -> np.ndarray | None:
    """Global -> local expert id for this GPU's share (local = global 0..E_local-1)."""
    if wl.E_local == wl.E_global:
        return None
    m = np.full(wl.E_global, -1, dtype=np.int32)
    m[: wl.E_local] = np.arange(wl.E_local, dtype=np.int32)
    return m


def make_routing(wl: Workload, rng) -> dict:
    """topk_ids [T,k] (global ids) and topk_weights [T,k] for a workload."""
    T, k = wl.T, wl.top_k
    out = {}
    if wl.routing == "uniform":
        ids = _distinct_uniform(rng, T, k, wl.E_global)
    elif wl.routing == "local_distinct":
        # every token picks k distinct experts among this GPU's local share
        ids = _distinct_uniform(rng, T, k, wl.E_local)
    elif wl.routing == "gumbel_imbalance":
        # Gumbel-top-k over all global experts; local experts carry a weight
        # 1 + delta, delta ~ U(-0.3, 0.3): Poisson-like counts with +-30% spread
        w = np.ones(wl.E_global)
        w[: wl.E_local] += rng.uniform(-0.3, 0.3, size=wl.E_local)
        keys = np.log(w)[None, :] + rng.gumbel(size=(T, wl.E_global))
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    elif wl.routing == "balanced_local":
        # every local expert gets exactly T * k / E_local rows: token t takes
        # experts sigma((b_t + j * step) mod E) for j < k, where the offsets
        # b_t run over each residue equally often (shuffled) and sigma is a
        # random relabelling
        E = wl.E_local
        step = E // k
        assert E % k == 0 and T % E == 0 and T * k // E == wl.rows_per_expert
        b = rng.permutation(np.tile(np.arange(E), T // E))
        sigma = rng.permutation(E)
        ids = sigma[(b[:, None] + step * np.arange(k)[None, :]) % E].astype(np.int32)
    elif wl.routing == "masked_zipf":
        return _masked_routing(wl, rng)
    else:
        raise ValueError(wl.routing)
    out["topk_ids"] = np.ascontiguousarray(ids, dtype=np.int32)
    out["topk_weights"] = _softmax_weights(rng, T, k)
    return out


def _masked_routing(wl: Workload, rng) -> dict:
    """Grouped-masked decode share.

    G local experts; `empty_experts` of them (seeded choice) get no rows, the
    others share `masked_rows` rows with Zipf(s) probabilities over their
    (seeded) ranks.  Every token owns exactly one local slot (slot index
    uniform in 0..k-1); its other k-1 slots name distinct non-local experts.
    """
    G, T, k = wl.E_local, wl.T, wl.top_k
    assert T == wl.masked_rows
    perm = rng.permutation(G)
    empty = np.sort(perm[: wl.empty_experts])
    active = perm[wl.empty_experts:]            # rank order = this order
    ranks = np.arange(1, active.size + 1, dtype=np.float64)
    p = ranks ** (-wl.zipf_s)
    p /= p.sum()
    cnt = rng.multinomial(T, p)
    counts = np.zeros(G, dtype=np.int32)
    counts[active] = cnt
    max_m = int(-(-counts.max() // wl.expected_m) * wl.expected_m)
    # token -> (expert, row): tokens shuffled, then dealt out in expert order
    tok_order = rng.permutation(T)
    tok_expert = np.empty(T, dtype=np.int32)
    tok_row = np.empty(T, dtype=np.int32)
    pos = 0
    for g in range(G):
        c = int(counts[g])
        sel = tok_order[pos:pos + c]
        tok_expert[sel] = g
        tok_row[sel] = np.arange(c, dtype=np.int32)
        pos += c
    local_slot = rng.integers(0, k, size=T).astype(np.int32)
    nonlocal_ids = (G + _distinct_uniform(rng, T, k - 1, wl.E_global - G)).astype(np.int32)
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = np.insert(nonlocal_ids[t], local_slot[t], tok_expert[t])
    row_of = np.full(T * k, -1, dtype=np.int32)
    row_of[np.arange(T) * k + local_slot] = tok_expert * max_m + tok_row
    return {
        "topk_ids": ids,
        "topk_weights": _softmax_weights(rng, T, k),
        "masked_m": counts,
        "max_m": max_m,
        "empty": empty,
        "tok_expert": tok_expert,
        "tok_row": tok_row,
        "row_of": row_of,
    }


def place_masked(X: np.ndarray, routing: dict, G: int, poison: bool = True) -> np.ndarray:
    """Caller-side dispatch into the masked layout a3 [G, max_m, K].

    Rows past each expert's valid count are filled with bf16 NaN so that any
    read of them into a valid output shows up.
    """
    max_m = routing["max_m"]
    K = X.shape[1]
    a3 = np.full((G, max_m, K), BF16_NAN if poison else 0, dtype=np.uint16)
    a3[routing["tok_expert"], routing["tok_row"]] = X
    return a3


def place_contiguous(X: np.ndarray, topk_ids: np.ndarray, expert_map, E_local: int,
                     align: int = 128, poison: bool = True) -> dict:
    """Caller-side dispatch into the grouped contiguous layout.

    Local expert e's routed slots (ascending flat slot f = t*k + j) become
    consecutive rows holding X[f // k]; each expert's segment is padded to a
    multiple of `align` rows (experts with no slot take none).  Returns a2
    [m, H] (padding rows bf16 NaN when poison), m_indices [m] (expert of each
    row, -1 on padding) and row_of [T*k] (row of slot f, -1 if not local).
    """
    T, k = topk_ids.shape
    flat = topk_ids.ravel()
    ok = (flat >= 0) & (flat < (len(expert_map) if expert_map is not None else E_local))
    loc = np.full(flat.size, -1, np.int64)
    loc[ok] = flat[ok] if expert_map is None else expert_map[flat[ok]]
    loc[(loc < 0) | (loc >= E_local)] = -1
    rows, mi = [], []
    row_of = np.full(T * k, -1, np.int32)
    m = 0
    for e in range(E_local):
        slots = np.nonzero(loc == e)[0]
        if slots.size == 0:
            continue
        p = -(-slots.size // align) * align
        row_of[slots] = m + np.arange(slots.size, dtype=np.int32)
        rows.append(slots)
        mi.append(np.concatenate([np.full(slots.size, e, np.int32),
                                  np.full(p - slots.size, -1, np.int32)]))
        m += p
    m_indices = np.concatenate(mi) if mi else np.zeros(0, np.int32)
    a2 = np.full((m, X.shape[1]), BF16_NAN if poison else 0, dtype=np.uint16)
    for slots, mie in zip(rows, mi):
        start = int(row_of[slots[0]])
        a2[start:start + slots.size] = X[slots // k]
    return {"a2": a2, "m_indices": m_indices, "row_of": row_of}


def random_scales_e8m0(rng, E: int, N: int, K: int, lo: int = 119, hi: int = 121) -> np.ndarray:
    """E8M0 block-scale bytes [E, N, K/32], uniform over [lo, hi] (2^-8 .. 2^-6:
    weights of about the INT4 weights' magnitude)."""
    assert K % 32 == 0
    return rng.integers(lo, hi + 1, size=(E, N, K // 32)).astype(np.uint8)


def make_weights_mxfp4(E: int, H: int, I: int, seed: int = 0) -> dict:
    """MXFP4 W13 and W2: uniform E2M1 codes (every 4-bit code), E8M0 scales."""
    r = _streams(seed + 1000)
    return {"codes13": random_codes(r[1], E, 2 * I, H),
            "scales13": random_scales_e8m0(r[2], E, 2 * I, H),
            "codes2": random_codes(r[3], E, H, I),
            "scales2": random_scales_e8m0(r[4], E, H, I)}


def make_weights(E: int, H: int, I: int, seed: int = 0, which=("w13", "w2")) -> dict:
    """W13 codes [E, 2I, H/8] + scales [E, 2I, H/32]; W2 codes [E, H, I/8] + scales."""
    r = _streams(seed)
    out = {}
    if "w13" in which:
        out["codes13"] = random_codes(r[1], E, 2 * I, H)
        out["scales13"] = random_scales(r[2], E, 2 * I, H)
    if "w2" in which:
        out["codes2"] = random_codes(r[3], E, H, I)
        out["scales2"] = random_scales(r[4], E, H, I)
    return out


def make_workload(name: str, seed: int = 0, weights: bool = True) -> dict:
    """All inputs of one workload, seed-deterministic."""
    wl = WORKLOADS[name]
    r = _streams(seed)
    d = {"wl": wl, "seed": seed}
    d["X"] = random_activations(r[0], wl.T, wl.H)
    d.update(make_routing(wl, r[5]))
    d["expert_map"] = expert_map_for(wl)
    if weights:
        d.update(make_weights(wl.E_local, wl.H, wl.I, seed))
    if wl.routing == "masked_zipf":
        d["a3"] = place_masked(d["X"], d, wl.E_local)
    if wl.routing == "balanced_local":
        d.update(place_contiguous(d["X"], d["topk_ids"], d["expert_map"], wl.E_local))
    return d


def random_small(seed: int, E: int, H: int, I: int, T: int, k: int,
                 E_global: int | None = None) -> dict:
    """Small random MoE problem for brute-force and parity sweeps."""
    r = _streams(seed)
    Eg = E if E_global is None else E_global
    d = {"X": random_activations(r[0], T, H)}
    d["topk_ids"] = _distinct_uniform(r[5], T, k, Eg)
    d["topk_weights"] = _softmax_weights(r[6], T, k)
    if Eg != E:
        m = np.full(Eg, -1, dtype=np.int32)
        m[:E] = np.arange(E, dtype=np.int32)
        d["expert_map"] = m
    else:
        d["expert_map"] = None
    d.update(make_weights(E, H, I, seed))
    return d
