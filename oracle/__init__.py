"""CPU oracle of the W4A16 INT4 MoE expert path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.  The
numerics live in ``w4a16_oracle.cpp`` (plain C++, no HIP); this module only
builds it with g++ and marshals numpy arrays.

Parity pins: every function here is pinned in ``tests/test_oracle_pins.py``
against closed forms, brute force, exact-arithmetic invariants and
independently written numpy references.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (OpenMP, no FP contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on (n >= 1)."""
    _load().oracle_set_num_threads(ctypes.c_int(int(n)))


# ---- element helpers -------------------------------------------------------

def bf16_from_f64(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float64), np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_from_f64(_p(x), ctypes.c_int64(x.size), _p(out))
    return out


def unpack_codes(words: np.ndarray, K: int) -> np.ndarray:
    words = _c(words, np.int32)
    rows = words.size // (K // 8)
    q = np.empty(words.shape[:-1] + (K,), dtype=np.uint8)
    _load().oracle_unpack_codes(_p(words), ctypes.c_int64(rows), ctypes.c_int64(K), _p(q))
    return q


def pack_codes(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    K = q.shape[-1]
    rows = q.size // K
    w = np.empty(q.shape[:-1] + (K // 8,), dtype=np.int32)
    _load().oracle_pack_codes(_p(q), ctypes.c_int64(rows), ctypes.c_int64(K), _p(w))
    return w


def dequant(words: np.ndarray, scales: np.ndarray, K: int, wmode: int = 0) -> np.ndarray:
    words = _c(words, np.int32)
    scales = _c(scales, np.uint16)
    rows = words.size // (K // 8)
    w = np.empty(words.shape[:-1] + (K,), dtype=np.float32)
    _load().oracle_dequant(_p(words), _p(scales), ctypes.c_int64(rows), ctypes.c_int64(K),
                           ctypes.c_int(wmode), _p(w))
    return w


# ---- routing ---------------------------------------------------------------

def align_capacity(T: int, top_k: int, E_local: int, block_m: int):
    slots = T * top_k
    sorted_cap = slots + E_local * (block_m - 1)
    sorted_cap = (sorted_cap + block_m - 1) // block_m * block_m
    return sorted_cap, sorted_cap // block_m


def moe_align(topk_ids, E_global: int, E_local: int, block_m: int, expert_map=None,
              sorted_cap: int | None = None, blocks_cap: int | None = None) -> dict:
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    if sorted_cap is None or blocks_cap is None:
        sc, bc = align_capacity(T, k, E_local, block_m)
        sorted_cap = sc if sorted_cap is None else sorted_cap
        blocks_cap = bc if blocks_cap is None else blocks_cap
    em = _c(expert_map, np.int32)
    sorted_ids = np.empty(sorted_cap, dtype=np.int32)
    expert_ids = np.empty(blocks_cap, dtype=np.int32)
    ntp = np.empty(1, dtype=np.int32)
    row_of = np.empty(T * k, dtype=np.int32)
    rc = _load().oracle_moe_align(_p(ids), T, k, E_global, _p(em), E_local, block_m,
                                  _p(sorted_ids), sorted_cap, _p(expert_ids), blocks_cap,
                                  _p(ntp), _p(row_of))
    if rc != 0:
        raise ValueError("capacity too small")
    return {"sorted_ids": sorted_ids, "expert_ids": expert_ids,
            "num_tokens_padded": int(ntp[0]), "row_of": row_of}


def moe_tiles(topk_ids, E_global: int, E_local: int, block_m: int, tile_m: int,
              expert_map=None) -> np.ndarray:
    """int32 [n_tiles, 4] = {expert, first position, rows, 0}."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    cap = -(-T * k // tile_m) + E_local
    tiles = np.zeros((max(cap, 1), 4), dtype=np.int32)
    n = _load().oracle_moe_tiles(_p(ids), T, k, E_global, _p(_c(expert_map, np.int32)),
                                 E_local, block_m, tile_m, _p(tiles), cap)
    if n < 0:
        raise ValueError("tile capacity too small")
    return tiles[:n]


# ---- GEMM stages -----------------------------------------------------------

def grouped_gemm(A, a_row, expert, codes, scales, N: int, K: int, wmode: int = 0,
                 acc64: bool = False, out_f32: bool = False, out=None):
    A = _c(A, np.uint16)
    a_row = _c(a_row, np.int32)
    expert = _c(expert, np.int32)
    codes = _c(codes, np.int32)
    scales = _c(scales, np.uint16)
    R = a_row.size
    E = codes.shape[0]
    if out is None:
        out = np.zeros((R, N), dtype=np.float32 if out_f32 else np.uint16)
    _load().oracle_grouped_gemm(_p(A), _p(a_row), _p(expert), ctypes.c_int64(R), _p(codes),
                                _p(scales), E, N, K, wmode, int(acc64), int(out_f32), _p(out))
    return out


def moe_gate_up(X, topk_ids, E_global, expert_map, codes13, scales13, wmode=0):
    X = _c(X, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E_local, N13, _ = codes13.shape
    I = N13 // 2
    H = X.shape[1]
    Y13 = np.zeros((T * k, 2 * I), dtype=np.uint16)
    _load().oracle_moe_gate_up(_p(X), _p(ids), T, k, E_global, _p(_c(expert_map, np.int32)),
                               E_local, _p(_c(codes13, np.int32)), _p(_c(scales13, np.uint16)),
                               H, I, wmode, _p(Y13))
    return Y13


def silu_mul(Y13) -> np.ndarray:
    Y13 = _c(Y13, np.uint16)
    rows, two_i = Y13.shape
    Z = np.empty((rows, two_i // 2), dtype=np.uint16)
    _load().oracle_silu_mul(_p(Y13), ctypes.c_int64(rows), two_i // 2, _p(Z))
    return Z


def moe_down(Z, topk_ids, E_global, expert_map, codes2, scales2, wmode=0):
    Z = _c(Z, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E_local, H, _ = codes2.shape
    I = Z.shape[1]
    Y2 = np.zeros((T * k, H), dtype=np.uint16)
    _load().oracle_moe_down(_p(Z), _p(ids), T, k, E_global, _p(_c(expert_map, np.int32)),
                            E_local, _p(_c(codes2, np.int32)), _p(_c(scales2, np.uint16)),
                            H, I, wmode, _p(Y2))
    return Y2


def combine(Y, row_of, topk_weights) -> np.ndarray:
    Y = _c(Y, np.uint16)
    row_of = _c(row_of, np.int32)
    w = _c(topk_weights, np.float32)
    T, k = w.shape
    H = Y.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    _load().oracle_combine(_p(Y), _p(row_of), _p(w), T, k, H, _p(out))
    return out


def masked_gemm(a3, masked_m, codes, scales, wmode=0, out=None):
    a3 = _c(a3, np.uint16)
    mm = _c(masked_m, np.int32)
    G, N, _ = codes.shape
    max_m = a3.shape[-2] if a3.ndim == 3 else a3.shape[0] // G
    K = a3.shape[-1]
    if out is None:
        out = np.zeros((G * max_m, N), dtype=np.uint16)
    _load().oracle_masked_gemm(_p(a3), _p(mm), G, max_m, _p(_c(codes, np.int32)),
                               _p(_c(scales, np.uint16)), N, K, wmode, _p(out))
    return out


def contiguous_gemm(a2, m_indices, codes, scales, wmode=0, out=None):
    """Grouped contiguous layout: a2 [m, K] bf16, m_indices int32 [m] (expert
    of each row, -1 on padding) -> out [m, N]; rows whose index is not an
    expert are left as they are in `out` (zeros when out is None)."""
    a2 = _c(a2, np.uint16)
    mi = _c(m_indices, np.int32)
    G, N, _ = codes.shape
    m, K = a2.shape
    assert mi.shape == (m,)
    if out is None:
        out = np.zeros((m, N), dtype=np.uint16)
    _load().oracle_contiguous_gemm(_p(a2), _p(mi), ctypes.c_int64(m), G,
                                   _p(_c(codes, np.int32)), _p(_c(scales, np.uint16)), N, K,
                                   wmode, _p(out))
    return out


def dequant_mx(words: np.ndarray, scales_e8m0: np.ndarray, K: int) -> np.ndarray:
    """MXFP4 weights: e2m1 codes (8 per int32 along K) times 2^(b - 127) per 32."""
    words = _c(words, np.int32)
    sc = _c(scales_e8m0, np.uint8)
    rows = words.size // (K // 8)
    w = np.empty(words.shape[:-1] + (K,), dtype=np.float32)
    _load().oracle_dequant_mx(_p(words), _p(sc), ctypes.c_int64(rows), ctypes.c_int64(K), _p(w))
    return w


def grouped_gemm_mx(A, a_row, expert, codes, scales_e8m0, N: int, K: int) -> np.ndarray:
    A = _c(A, np.uint16)
    a_row = _c(a_row, np.int32)
    expert = _c(expert, np.int32)
    R = a_row.size
    out = np.zeros((R, N), dtype=np.uint16)
    _load().oracle_grouped_gemm_mx(_p(A), _p(a_row), _p(expert), ctypes.c_int64(R),
                                   _p(_c(codes, np.int32)), _p(_c(scales_e8m0, np.uint8)), N, K,
                                   _p(out))
    return out


def moe_forward_mx(X, topk_ids, topk_weights, E_global, expert_map, codes13, scales13,
                   codes2, scales2, intermediates=False):
    """The indexed path on MXFP4 weights (scales: E8M0 bytes [E, N, K/32])."""
    X = _c(X, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E_local, N13, _ = codes13.shape
    I = N13 // 2
    H = X.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    Y13 = Z = Y2 = None
    if intermediates:
        Y13 = np.empty((T * k, 2 * I), dtype=np.uint16)
        Z = np.empty((T * k, I), dtype=np.uint16)
        Y2 = np.empty((T * k, H), dtype=np.uint16)
    _load().oracle_moe_forward_mx(_p(X), _p(ids), _p(_c(topk_weights, np.float32)), T, k,
                                  E_global, _p(_c(expert_map, np.int32)), E_local,
                                  _p(_c(codes13, np.int32)), _p(_c(scales13, np.uint8)),
                                  _p(_c(codes2, np.int32)), _p(_c(scales2, np.uint8)), H, I,
                                  _p(out), _p(Y13), _p(Z), _p(Y2))
    if intermediates:
        return {"out": out, "Y13": Y13, "Z": Z, "Y2": Y2}
    return out


def e4m3_value(b: int) -> float:
    """Value of an E4M3 byte (OCP 8-bit float, NaN at 0x7F / 0xFF)."""
    f = _load().oracle_e4m3_value
    f.restype = ctypes.c_double
    return float(f(ctypes.c_int(int(b))))


def e4m3_from_double(v: float) -> int:
    """Nearest E4M3 code (ties to even mantissa; saturating at 448)."""
    f = _load().oracle_e4m3_from_double
    f.argtypes = [ctypes.c_double]
    return int(f(float(v)))


def quantize_mxfp8(x, K: int | None = None):
    """bf16 bits [rows, K] -> (E4M3 codes uint8 [rows, K], E8M0 scales uint8
    [rows, K/32]): the OCP microscaling conversion per block of 32."""
    x = _c(x, np.uint16)
    K = x.shape[-1] if K is None else K
    rows = x.size // K
    codes = np.empty(x.shape[:-1] + (K,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (K // 32,), dtype=np.uint8)
    _load().oracle_quantize_mxfp8(_p(x), ctypes.c_int64(rows), ctypes.c_int64(K), _p(codes),
                                  _p(scales))
    return codes, scales


def grouped_gemm_a8w4(A8, A_sc, a_row, expert, codes, scales_e8m0, N: int, K: int,
                      out_f32: bool = False) -> np.ndarray:
    """Grouped GEMM on MXFP8 activations (codes A8 [rows, K], scales A_sc
    [rows, K/32]) and MXFP4 weights; bf16 bits or fp32 out."""
    A8 = _c(A8, np.uint8)
    A_sc = _c(A_sc, np.uint8)
    a_row = _c(a_row, np.int32)
    expert = _c(expert, np.int32)
    R = a_row.size
    out = np.zeros((R, N), dtype=np.float32 if out_f32 else np.uint16)
    _load().oracle_grouped_gemm_a8w4(_p(A8), _p(A_sc), _p(a_row), _p(expert), ctypes.c_int64(R),
                                     _p(_c(codes, np.int32)), _p(_c(scales_e8m0, np.uint8)), N, K,
                                     int(out_f32), _p(out))
    return out


def moe_forward_a8w4(X, topk_ids, topk_weights, E_global, expert_map, codes13, scales13,
                     codes2, scales2, intermediates=False):
    """The indexed path in A8W4: MXFP8 activations (X and Z quantized per row)
    on MXFP4 weights."""
    X = _c(X, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E_local, N13, _ = codes13.shape
    I = N13 // 2
    H = X.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    Z = Y2 = None
    if intermediates:
        Z = np.empty((T * k, I), dtype=np.uint16)
        Y2 = np.empty((T * k, H), dtype=np.uint16)
    _load().oracle_moe_forward_a8w4(_p(X), _p(ids), _p(_c(topk_weights, np.float32)), T, k,
                                    E_global, _p(_c(expert_map, np.int32)), E_local,
                                    _p(_c(codes13, np.int32)), _p(_c(scales13, np.uint8)),
                                    _p(_c(codes2, np.int32)), _p(_c(scales2, np.uint8)), H, I,
                                    _p(out), _p(Z), _p(Y2))
    if intermediates:
        return {"out": out, "Z": Z, "Y2": Y2}
    return out


def router_topk(logits, k):
    """Router logits float32 [T, E] -> (topk_ids int32 [T, k], weights float32
    [T, k]): largest logits first (ties: lower id first), softmax over the k
    selected logits."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _load().oracle_router_topk(_p(lg), T, E, k, _p(ids), _p(w))
    return ids, w


def indexed_to_masked(X, topk_ids, E_global, expert_map, E_local, max_m, a3=None):
    """Place each local slot's activation row into the grouped masked layout.
    Returns (a3 [E_local * max_m, H], masked_m [E_local], row_of [T*k],
    dropped); rows of a3 not written keep their contents (zeros when a3 is
    None)."""
    X = _c(X, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    H = X.shape[1]
    if a3 is None:
        a3 = np.zeros((E_local * max_m, H), dtype=np.uint16)
    mm = np.empty(E_local, dtype=np.int32)
    row_of = np.empty(T * k, dtype=np.int32)
    dropped = _load().oracle_indexed_to_masked(_p(X), H, _p(ids), T, k, E_global,
                                               _p(_c(expert_map, np.int32)), E_local, max_m,
                                               _p(a3), _p(mm), _p(row_of))
    return a3, mm, row_of, int(dropped)


def moe_forward(X, topk_ids, topk_weights, E_global, expert_map, codes13, scales13,
                codes2, scales2, wmode=0, intermediates=False):
    X = _c(X, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E_local, N13, H8 = codes13.shape
    I = N13 // 2
    H = X.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    Y13 = Z = Y2 = None
    if intermediates:
        Y13 = np.empty((T * k, 2 * I), dtype=np.uint16)
        Z = np.empty((T * k, I), dtype=np.uint16)
        Y2 = np.empty((T * k, H), dtype=np.uint16)
    _load().oracle_moe_forward(_p(X), _p(ids), _p(_c(topk_weights, np.float32)), T, k,
                               E_global, _p(_c(expert_map, np.int32)), E_local,
                               _p(_c(codes13, np.int32)), _p(_c(scales13, np.uint16)),
                               _p(_c(codes2, np.int32)), _p(_c(scales2, np.uint16)), H, I,
                               wmode, _p(out), _p(Y13), _p(Z), _p(Y2))
    if intermediates:
        return {"out": out, "Y13": Y13, "Z": Z, "Y2": Y2}
    return out


def direct_forward(X, topk_ids, topk_weights, E_global, expert_map, codes13, scales13,
                   codes2, scales2, wmode=0):
    X = _c(X, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E_local, N13, _ = codes13.shape
    I = N13 // 2
    H = X.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    _load().oracle_direct_forward(_p(X), _p(ids), _p(_c(topk_weights, np.float32)), T, k,
                                  E_global, _p(_c(expert_map, np.int32)), E_local,
                                  _p(_c(codes13, np.int32)), _p(_c(scales13, np.uint16)),
                                  _p(_c(codes2, np.int32)), _p(_c(scales2, np.uint16)), H, I,
                                  wmode, _p(out))
    return out
