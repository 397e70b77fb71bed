"""ctypes mirror of include/w4a16moe.h (argument marshalling only).

Every function here has the name of the C entry point it forwards to.  Device
buffers are passed as torch tensors (their data pointers); PyTorch supplies
device memory and the current HIP stream, nothing else.  A missing library is
an ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads PyTorch's HIP runtime first; the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16moe.so")

# ---- constants (mirror the header) -------------------------------------------
W4A16_OK = 0
W4A16_ERR_INVALID_ARG = 1
W4A16_ERR_UNSUPPORTED = 2
W4A16_ERR_MODE_MISMATCH = 3
W4A16_ERR_CAPACITY = 4
W4A16_ERR_ROUTING = 5
W4A16_ERR_HIP = 6
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "MODE_MISMATCH",
                4: "CAPACITY", 5: "ROUTING", 6: "HIP"}

W4A16_PROFILE_DECODE = 1
W4A16_PROFILE_PREFILL = 2
W4A16_PACK_GATE_UP_INTERLEAVE = 0x1
W4A16_PACK_MXFP4 = 0x2
W4A16_PACK_MXFP8_ACT = 0x4
W4A16_DESC_MAGIC = 0x4D413457
W4A16_DESC_VERSION = 1
W4A16_ALIGN_VALIDATE = 0x1
W4A16_LAYOUT_INDEXED = 0
W4A16_LAYOUT_MASKED = 1
W4A16_LAYOUT_CONTIGUOUS = 2
W4A16_AROW_TOKEN = 0
W4A16_AROW_SLOT = 1
W4A16_AROW_POSITION = 2
W4A16_OROW_POSITION = 0
W4A16_OROW_SLOT = 1
W4A16_EPI_STORE = 0
W4A16_EPI_SILU_MUL = 1
W4A16_GEMM_F32_OUT = 0x1

_i32p = ctypes.POINTER(ctypes.c_int32)


class w4a16_desc(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("profile", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("group", ctypes.c_int32), ("chunk_n", ctypes.c_int32),
                ("k_groups", ctypes.c_int32), ("stage_bytes", ctypes.c_uint64),
                ("chunk_bytes", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


class w4a16_routing(ctypes.Structure):
    _fields_ = [("sorted_ids", ctypes.c_void_p), ("sorted_cap", ctypes.c_int32),
                ("expert_ids", ctypes.c_void_p), ("blocks_cap", ctypes.c_int32),
                ("num_tokens_padded", ctypes.c_void_p), ("row_of", ctypes.c_void_p),
                ("tiles", ctypes.c_void_p), ("tiles_cap", ctypes.c_int32),
                ("tile_count", ctypes.c_void_p), ("tile_m", ctypes.c_int32),
                ("expert_offsets", ctypes.c_void_p)]


class w4a16_gemm_args(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("split_k", ctypes.c_int32),
                ("A", ctypes.c_void_p), ("A_rows", ctypes.c_int64),
                ("arow", ctypes.c_int32), ("orow", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("sorted_ids", ctypes.c_void_p), ("sorted_cap", ctypes.c_int32),
                ("expert_ids", ctypes.c_void_p), ("blocks_cap", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("num_tokens_padded", ctypes.c_void_p),
                ("tiles", ctypes.c_void_p), ("tiles_cap", ctypes.c_int32),
                ("tile_count", ctypes.c_void_p), ("tile_m", ctypes.c_int32),
                ("rows_hint", ctypes.c_int32),
                ("masked_m", ctypes.c_void_p), ("max_m", ctypes.c_int32),
                ("expected_m", ctypes.c_int32),
                ("packed", ctypes.c_void_p), ("desc", ctypes.POINTER(w4a16_desc)),
                ("out", ctypes.c_void_p), ("out_rows", ctypes.c_int64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
                ("m_indices", ctypes.c_void_p),
                ("comb_out", ctypes.c_void_p), ("comb_row_of", ctypes.c_void_p),
                ("comb_weights", ctypes.c_void_p), ("comb_T", ctypes.c_int32),
                ("A_scales", ctypes.c_void_p)]


class w4a16_plan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("ring_groups", ctypes.c_int32)]


# name -> (restype, argtypes); the full exported surface of the header
SIGNATURES = {
    "w4a16_last_error": (ctypes.c_char_p, []),
    "w4a16_version": (ctypes.c_int32, []),
    "w4a16_prepack_bytes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_uint32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_uint64)]),
    "w4a16_prepack": (ctypes.c_int, [ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_uint64, ctypes.POINTER(w4a16_desc),
                                     ctypes.c_void_p]),
    "w4a16_prepack_host": (ctypes.c_int, [ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_uint64, ctypes.POINTER(w4a16_desc)]),
    "w4a16_prepack_mxfp4": (ctypes.c_int, [ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_uint64, ctypes.POINTER(w4a16_desc),
                                           ctypes.c_void_p]),
    "w4a16_prepack_mxfp4_host": (ctypes.c_int, [ctypes.c_int32, ctypes.c_uint32,
                                                ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64,
                                                ctypes.POINTER(w4a16_desc)]),
    "w4a16_moe_align_capacity": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, _i32p, _i32p,
                                                _i32p]),
    "w4a16_moe_align": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.POINTER(w4a16_routing),
                                       ctypes.c_uint32, ctypes.c_void_p]),
    "w4a16_gemm_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(w4a16_gemm_args),
                                                  ctypes.POINTER(ctypes.c_uint64)]),
    "w4a16_moe_w4a16_gemm": (ctypes.c_int, [ctypes.POINTER(w4a16_gemm_args), ctypes.c_void_p]),
    "w4a16_moe_w4a16_gemm_noalloc": (ctypes.c_int, [ctypes.POINTER(w4a16_gemm_args),
                                                    ctypes.c_void_p]),
    "w4a16_moe_silu_mul": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "w4a16_quantize_mxfp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]),
    "w4a16_moe_combine": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "w4a16_moe_router_topk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "w4a16_moe_route_align": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.POINTER(w4a16_routing),
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                             ctypes.c_void_p]),
    "w4a16_moe_indexed_to_masked": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64,
                                                   ctypes.c_int32, ctypes.c_void_p,
                                                   ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_void_p,
                                                   ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.POINTER(w4a16_routing),
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p]),
    "w4a16_plan_gemm": (ctypes.c_int, [ctypes.POINTER(w4a16_desc), ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(w4a16_plan)]),
}


class W4A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m w4a16_int4_mixture_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def check(status: int) -> None:
    if status != W4A16_OK:
        msg = lib().w4a16_last_error().decode(errors="replace")
        raise W4A16Error(status, msg)


# ---- the C entry points, one to one --------------------------------------------

def w4a16_version() -> int:
    return int(lib().w4a16_version())


def w4a16_last_error() -> str:
    return lib().w4a16_last_error().decode(errors="replace")


def w4a16_prepack_bytes(profile, flags, E, N, K, group=32) -> int:
    out = ctypes.c_uint64()
    check(lib().w4a16_prepack_bytes(profile, flags, E, N, K, group, ctypes.byref(out)))
    return out.value


def w4a16_prepack(profile, flags, codes, scales, E, N, K, group, packed, stream=None) -> w4a16_desc:
    desc = w4a16_desc()
    nbytes = packed.numel() * packed.element_size()
    check(lib().w4a16_prepack(profile, flags, ptr(codes), ptr(scales), E, N, K, group,
                              ptr(packed), nbytes, ctypes.byref(desc), stream_handle(stream)))
    return desc


def w4a16_prepack_host(profile, flags, codes, scales, E, N, K, group, packed) -> w4a16_desc:
    """Host reference of the permutation; numpy arrays in and out."""
    desc = w4a16_desc()
    check(lib().w4a16_prepack_host(profile, flags, codes.ctypes.data, scales.ctypes.data, E, N,
                                   K, group, packed.ctypes.data, packed.nbytes,
                                   ctypes.byref(desc)))
    return desc


def w4a16_prepack_mxfp4(profile, flags, codes, scales_e8m0, E, N, K, group, packed,
                        stream=None) -> w4a16_desc:
    desc = w4a16_desc()
    nbytes = packed.numel() * packed.element_size()
    check(lib().w4a16_prepack_mxfp4(profile, flags, ptr(codes), ptr(scales_e8m0), E, N, K, group,
                                    ptr(packed), nbytes, ctypes.byref(desc),
                                    stream_handle(stream)))
    return desc


def w4a16_prepack_mxfp4_host(profile, flags, codes, scales_e8m0, E, N, K, group,
                             packed) -> w4a16_desc:
    """Host reference of the MXFP4 permutation; numpy arrays in and out."""
    desc = w4a16_desc()
    check(lib().w4a16_prepack_mxfp4_host(profile, flags, codes.ctypes.data,
                                         scales_e8m0.ctypes.data, E, N, K, group,
                                         packed.ctypes.data, packed.nbytes, ctypes.byref(desc)))
    return desc


def w4a16_moe_align_capacity(T, top_k, E_local, block_m, tile_m=0):
    sc, bc, tc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    check(lib().w4a16_moe_align_capacity(T, top_k, E_local, block_m, tile_m, ctypes.byref(sc),
                                         ctypes.byref(bc), ctypes.byref(tc)))
    return sc.value, bc.value, tc.value


def w4a16_moe_align(topk_ids, T, top_k, E_global, expert_map, E_local, block_m, routing,
                    flags=0, stream=None) -> None:
    check(lib().w4a16_moe_align(ptr(topk_ids), T, top_k, E_global, ptr(expert_map), E_local,
                                block_m, ctypes.byref(routing), flags, stream_handle(stream)))


def w4a16_gemm_workspace_bytes(args: w4a16_gemm_args) -> int:
    out = ctypes.c_uint64()
    check(lib().w4a16_gemm_workspace_bytes(ctypes.byref(args), ctypes.byref(out)))
    return out.value


def w4a16_moe_w4a16_gemm(args: w4a16_gemm_args, stream=None) -> None:
    check(lib().w4a16_moe_w4a16_gemm(ctypes.byref(args), stream_handle(stream)))


def w4a16_moe_w4a16_gemm_noalloc(args: w4a16_gemm_args, stream=None) -> None:
    check(lib().w4a16_moe_w4a16_gemm_noalloc(ctypes.byref(args), stream_handle(stream)))


def w4a16_moe_silu_mul(y13, rows, rows_dev, I, z, stream=None) -> None:
    check(lib().w4a16_moe_silu_mul(ptr(y13), rows, ptr(rows_dev), I, ptr(z),
                                   stream_handle(stream)))


def w4a16_quantize_mxfp8(x, rows, rows_dev, K, codes, scales, stream=None) -> None:
    check(lib().w4a16_quantize_mxfp8(ptr(x), rows, ptr(rows_dev), K, ptr(codes), ptr(scales),
                                     stream_handle(stream)))


def w4a16_moe_combine(y, y_rows, H, row_of, topk_weights, T, top_k, out, stream=None) -> None:
    check(lib().w4a16_moe_combine(ptr(y), y_rows, H, ptr(row_of), ptr(topk_weights), T, top_k,
                                  ptr(out), stream_handle(stream)))


def w4a16_moe_router_topk(logits, T, E_global, top_k, topk_ids, topk_weights,
                          stream=None) -> None:
    check(lib().w4a16_moe_router_topk(ptr(logits), T, E_global, top_k, ptr(topk_ids),
                                      ptr(topk_weights), stream_handle(stream)))


def w4a16_moe_route_align(logits, T, E_global, top_k, expert_map, E_local, block_m, routing,
                          topk_ids, topk_weights, flags=0, stream=None) -> None:
    check(lib().w4a16_moe_route_align(ptr(logits), T, E_global, top_k, ptr(expert_map),
                                      E_local, block_m, ctypes.byref(routing), ptr(topk_ids),
                                      ptr(topk_weights), flags, stream_handle(stream)))


def w4a16_moe_indexed_to_masked(X, X_rows, H, topk_ids, T, top_k, E_global, expert_map,
                                E_local, max_m, scratch, a3, masked_m, row_of, dropped=None,
                                stream=None) -> None:
    check(lib().w4a16_moe_indexed_to_masked(ptr(X), X_rows, H, ptr(topk_ids), T, top_k,
                                            E_global, ptr(expert_map), E_local, max_m,
                                            ctypes.byref(scratch), ptr(a3), ptr(masked_m),
                                            ptr(row_of), ptr(dropped), stream_handle(stream)))


def w4a16_plan_gemm(desc, layout, rows_hint=0, expected_m=0, tile_m=0) -> w4a16_plan:
    p = w4a16_plan()
    check(lib().w4a16_plan_gemm(ctypes.byref(desc), layout, rows_hint, expected_m, tile_m,
                                ctypes.byref(p)))
    return p
