"""W4A16 INT4 MoE expert path for AMD MI355X (gfx950).

Python side of the C-ABI library ``libw4a16moe.so``: ``_capi`` forwards each
C entry point one to one; the helpers below only allocate device buffers with
PyTorch and chain those calls.  Every step of the path (routing sort, both
grouped GEMMs, activation, combine, prepacking) runs in the library's HIP
kernels.

Typical use (indexed layout)::

    w13 = prepare_weight(codes13, scales13, PROFILE_DECODE)
    w2 = prepare_weight(codes2, scales2, PROFILE_DECODE)
    path = IndexedPath(w13, w2, T=64, top_k=8, E_global=384, rows_hint=512)
    out = path(X, topk_ids, topk_weights, expert_map)          # bf16 [T, H]
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _capi
from ._capi import (W4A16Error, W4A16_PROFILE_DECODE as PROFILE_DECODE,  # noqa: F401
                    W4A16_PROFILE_PREFILL as PROFILE_PREFILL,
                    W4A16_PACK_GATE_UP_INTERLEAVE as PACK_GATE_UP_INTERLEAVE,
                    W4A16_PACK_MXFP8_ACT as PACK_MXFP8_ACT)

BF16 = torch.int16  # bf16 tensors travel as raw 16-bit patterns


def _dev_empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes, device):
    """GEMM workspace: 256-byte granular and zeroed (its split-K arrival
    counters must start at zero; calls leave them zero)."""
    return torch.zeros(((nbytes + 255) // 256 * 256,), dtype=torch.uint8, device=device)


@dataclass
class PreparedWeight:
    packed: torch.Tensor        # uint8 device buffer
    desc: _capi.w4a16_desc

    @property
    def E(self):
        return self.desc.E

    @property
    def N(self):
        return self.desc.N

    @property
    def K(self):
        return self.desc.K


def _check_weight_inputs(codes: torch.Tensor, scales: torch.Tensor, scale_dtypes, what: str):
    """The packer reads codes and scales through raw pointers sized from the
    codes' shape: refuse a dtype or shape that does not match it."""
    if codes.dim() != 3 or codes.dtype != torch.int32:
        raise ValueError(f"{what}: codes must be int32 [E, N, K/8] (eight 4-bit codes per word), "
                         f"got {codes.dtype} {tuple(codes.shape)}")
    E, N, K8 = codes.shape
    if scales.dtype not in scale_dtypes or tuple(scales.shape) != (E, N, K8 * 8 // 32):
        raise ValueError(f"{what}: scales must be {[str(d) for d in scale_dtypes]} "
                         f"[{E}, {N}, {K8 * 8 // 32}], got {scales.dtype} {tuple(scales.shape)}")
    if codes.device != scales.device:
        raise ValueError(f"{what}: codes and scales on different devices")
    return E, N, K8 * 8


def prepare_weight(codes: torch.Tensor, scales: torch.Tensor, profile: int, flags: int = 0,
                   stream=None) -> PreparedWeight:
    """codes int32 [E, N, K/8], scales bf16 bits [E, N, K/32] (device) -> packed weight."""
    E, N, K = _check_weight_inputs(codes, scales, (torch.int16, torch.bfloat16), "prepare_weight")
    nbytes = _capi.w4a16_prepack_bytes(profile, flags, E, N, K, 32)
    packed = _dev_empty((nbytes,), torch.uint8, codes.device)
    desc = _capi.w4a16_prepack(profile, flags, codes.contiguous(), scales.contiguous(), E, N, K,
                               32, packed, stream)
    return PreparedWeight(packed, desc)


def prepare_weight_mxfp4(codes: torch.Tensor, scales_e8m0: torch.Tensor, flags: int = 0,
                         stream=None) -> PreparedWeight:
    """MXFP4 weights: E2M1 codes int32 [E, N, K/8], E8M0 scale bytes uint8
    [E, N, K/32] (device) -> packed weight (DECODE profile).  flags may add
    PACK_MXFP8_ACT (A8W4: the GEMMs then take MXFP8 activations)."""
    E, N, K = _check_weight_inputs(codes, scales_e8m0, (torch.uint8,), "prepare_weight_mxfp4")
    nbytes = _capi.w4a16_prepack_bytes(PROFILE_DECODE, flags | _capi.W4A16_PACK_MXFP4, E, N, K, 32)
    packed = _dev_empty((nbytes,), torch.uint8, codes.device)
    desc = _capi.w4a16_prepack_mxfp4(PROFILE_DECODE, flags, codes.contiguous(),
                                     scales_e8m0.contiguous(), E, N, K, 32, packed, stream)
    return PreparedWeight(packed, desc)


class Routing:
    """Device buffers of the indexed routing metadata (over-allocated)."""

    def __init__(self, T, top_k, E_local, block_m, tile_m, device):
        sc, bc, tc = _capi.w4a16_moe_align_capacity(T, top_k, E_local, block_m, tile_m)
        self.T, self.top_k, self.E_local = T, top_k, E_local
        self.block_m, self.tile_m = block_m, tile_m
        self.sorted_cap, self.blocks_cap, self.tiles_cap = sc, bc, tc
        self.sorted_ids = _dev_empty((sc,), torch.int32, device)
        self.expert_ids = _dev_empty((bc,), torch.int32, device)
        self.num_tokens_padded = _dev_empty((1,), torch.int32, device)
        self.row_of = _dev_empty((max(1, T * top_k),), torch.int32, device)
        self.tiles = _dev_empty((max(1, tc), 4), torch.int32, device)
        self.tile_count = _dev_empty((1,), torch.int32, device)
        self.c = _capi.w4a16_routing(
            sorted_ids=self.sorted_ids.data_ptr(), sorted_cap=sc,
            expert_ids=self.expert_ids.data_ptr(), blocks_cap=bc,
            num_tokens_padded=self.num_tokens_padded.data_ptr(),
            row_of=self.row_of.data_ptr(), tiles=self.tiles.data_ptr() if tc else None,
            tiles_cap=tc, tile_count=self.tile_count.data_ptr(), tile_m=tile_m)

    def align(self, topk_ids, E_global, expert_map=None, flags=0, stream=None):
        _capi.w4a16_moe_align(topk_ids, self.T, self.top_k, E_global, expert_map, self.E_local,
                              self.block_m, self.c, flags, stream)


class MXFP8:
    """MXFP8 activations (A8W4): E4M3 codes uint8 [rows, K] and E8M0 scale
    bytes uint8 [rows, K/32] on the device."""

    def __init__(self, rows: int, K: int, device="cuda"):
        self.codes = _dev_empty((rows, K), torch.uint8, device)
        self.scales = _dev_empty((rows, K // 32), torch.uint8, device)
        self.shape = (rows, K)

    def data_ptr(self):
        return self.codes.data_ptr()


def quantize_mxfp8(x: torch.Tensor, out: MXFP8 = None, rows_dev=None, stream=None) -> MXFP8:
    """bf16 bits [rows, K] -> MXFP8 (the library's microscaling conversion),
    rows [0, min(*rows_dev, rows)) when rows_dev (device int32 [1]) is given."""
    rows, K = x.shape
    out = MXFP8(rows, K, x.device) if out is None else out
    _capi.w4a16_quantize_mxfp8(x, rows, rows_dev, K, out.codes, out.scales, stream)
    return out


def gemm_args_indexed(w: PreparedWeight, A, routing: Routing, out, arow, epilogue=0, flags=0,
                      split_k=0, rows_hint=0, workspace=None, orow=_capi.W4A16_OROW_POSITION,
                      use_tiles=True):
    """A: bf16 bits [rows, K], or MXFP8 for a weight packed with PACK_MXFP8_ACT."""
    a = _capi.w4a16_gemm_args()
    a.layout = _capi.W4A16_LAYOUT_INDEXED
    a.epilogue = epilogue
    a.flags = flags
    a.split_k = split_k
    a.A = A.data_ptr()
    a.A_rows = A.shape[0]
    if isinstance(A, MXFP8):
        a.A_scales = A.scales.data_ptr()
    a.arow = arow
    a.orow = orow
    a.top_k = routing.top_k
    a.num_slots = routing.T * routing.top_k
    a.sorted_ids = routing.sorted_ids.data_ptr()
    a.sorted_cap = routing.sorted_cap
    a.expert_ids = routing.expert_ids.data_ptr()
    a.blocks_cap = routing.blocks_cap
    a.block_m = routing.block_m
    a.num_tokens_padded = routing.num_tokens_padded.data_ptr()
    if use_tiles and routing.tiles_cap:
        a.tiles = routing.tiles.data_ptr()
        a.tiles_cap = routing.tiles_cap
        a.tile_count = routing.tile_count.data_ptr()
        a.tile_m = routing.tile_m
    a.rows_hint = rows_hint
    a.packed = w.packed.data_ptr()
    a.desc = ctypes.pointer(w.desc)
    a.out = out.data_ptr()
    a.out_rows = out.shape[0]
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    # the struct holds raw pointers: keep the tensors alive with it, so that a
    # temporary passed in is not freed (and its memory handed out again)
    # before the launch
    a._refs = (w, A, routing, out, workspace)
    return a


def gemm_args_masked(w: PreparedWeight, A, masked_m, max_m, expected_m, out, epilogue=0,
                     flags=0, workspace=None):
    a = _capi.w4a16_gemm_args()
    a.layout = _capi.W4A16_LAYOUT_MASKED
    a.epilogue = epilogue
    a.flags = flags
    a.A = A.data_ptr()
    a.A_rows = A.shape[0]
    a.masked_m = masked_m.data_ptr()
    a.max_m = max_m
    a.expected_m = expected_m
    a.packed = w.packed.data_ptr()
    a.desc = ctypes.pointer(w.desc)
    a.out = out.data_ptr()
    a.out_rows = out.shape[0]
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    # the struct holds raw pointers: keep the tensors alive with it, so that a
    # temporary passed in is not freed (and its memory handed out again)
    # before the launch
    a._refs = (w, A, out, workspace, masked_m)
    return a


def gemm_args_contiguous(w: PreparedWeight, A, m_indices, out, epilogue=0, flags=0,
                         workspace=None):
    """Grouped contiguous layout: A [m, K] rows per expert (segments padded to
    128 rows), m_indices int32 [m] (-1 on padding) -> out [m, N]."""
    a = _capi.w4a16_gemm_args()
    a.layout = _capi.W4A16_LAYOUT_CONTIGUOUS
    a.epilogue = epilogue
    a.flags = flags
    a.A = A.data_ptr()
    a.A_rows = A.shape[0]
    a.m_indices = m_indices.data_ptr()
    a.packed = w.packed.data_ptr()
    a.desc = ctypes.pointer(w.desc)
    a.out = out.data_ptr()
    a.out_rows = out.shape[0]
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a._refs = (w, A, out, workspace, m_indices)
    return a


def run_gemm(args: _capi.w4a16_gemm_args, device, keep=None, stream=None):
    """Run one GEMM stage, allocating its workspace when the call needs one."""
    need = _capi.w4a16_gemm_workspace_bytes(args)
    ws = None
    if need and not args.workspace:
        ws = _workspace(need, device)
        args.workspace = ws.data_ptr()
        args.workspace_bytes = ws.numel()
        if stream is not None:
            ws.record_stream(stream)    # not reused before the launch on `stream` ends
    _capi.w4a16_moe_w4a16_gemm(args, stream)
    if keep is not None and ws is not None:
        keep.append(ws)
    return ws


class IndexedPath:
    """The whole indexed path with every buffer allocated once:
    align -> gate/up GEMM -> SiLU*gate -> down GEMM -> top-k combine.

    With a W13 packed with gate/up interleave, SiLU*gate runs inside the
    gate/up GEMM (one launch that writes Z); with a plain W13 the gate/up GEMM
    stores Y13 and SiLU*gate is a call of its own (act).  With fuse_combine
    (DECODE-profile weights) the top-k combine runs in the down GEMM's
    epilogue; by default it is a call of its own."""

    def __init__(self, w13: PreparedWeight, w2: PreparedWeight, T: int, top_k: int,
                 E_global: int, rows_hint: int = 0, tile_m: int = 0, split_k13: int = 0,
                 split_k2: int = 0, device="cuda", fuse_combine: bool = False):
        assert w13.E == w2.E and w13.N == 2 * w2.K and w13.K == w2.N
        self.w13, self.w2 = w13, w2
        self.T, self.top_k, self.E_global, self.E = T, top_k, E_global, w13.E
        self.H, self.I = w13.K, w2.K
        self.rows_hint = rows_hint
        plan = _capi.w4a16_plan_gemm(w13.desc, _capi.W4A16_LAYOUT_INDEXED, rows_hint, 0, tile_m)
        self.plan = plan
        self.routing = Routing(T, top_k, self.E, plan.block_m, plan.tile_m, device)
        cap = self.routing.sorted_cap
        self.separate_act = not (w13.desc.flags & PACK_GATE_UP_INTERLEAVE)
        # A8W4: X and Z go to the GEMMs as MXFP8
        self.a8 = bool(w13.desc.flags & PACK_MXFP8_ACT)
        assert self.a8 == bool(w2.desc.flags & PACK_MXFP8_ACT)
        assert not (self.a8 and fuse_combine), "A8W4 keeps the combine as a call of its own"
        self.X8 = MXFP8(max(T, 1), self.H, device) if self.a8 else None
        self.Z8 = MXFP8(cap, self.I, device) if self.a8 else None
        self.Y13 = _dev_empty((cap, 2 * self.I), BF16, device) if self.separate_act else None
        self.Z = _dev_empty((cap, self.I), BF16, device)
        self.Y2 = _dev_empty((cap, self.H), BF16, device)
        self.out = _dev_empty((max(T, 1), self.H), BF16, device)
        self.split_k13, self.split_k2 = split_k13, split_k2
        self.fuse_combine = fuse_combine
        self.device = device
        self._ws = {}
        self._tw = None            # top-k weights the fused combine reads

    def _ws_for(self, key, args):
        need = _capi.w4a16_gemm_workspace_bytes(args)
        if need == 0:
            return
        buf = self._ws.get(key)
        if buf is None or buf.numel() < need:
            buf = _workspace(need, self.device)
            self._ws[key] = buf
        args.workspace = buf.data_ptr()
        args.workspace_bytes = buf.numel()

    def gate_up_args(self, X, out=None, epilogue=_capi.W4A16_EPI_SILU_MUL, flags=0):
        """X: bf16 bits [T, H], or (A8W4) its MXFP8 form (quant_x)."""
        out = self.Z if out is None else out
        if self.a8 and not isinstance(X, MXFP8):
            X = self.X8
        a = gemm_args_indexed(self.w13, X, self.routing, out, _capi.W4A16_AROW_TOKEN,
                              epilogue=epilogue, flags=flags, split_k=self.split_k13,
                              rows_hint=self.rows_hint)
        self._ws_for(("g", epilogue, flags), a)
        return a

    def down_args(self, Z=None, out=None, flags=0, topk_weights=None):
        """Down GEMM arguments; with topk_weights (and fuse_combine) the
        top-k combine into self.out runs in its epilogue."""
        Z = (self.Z8 if self.a8 else self.Z) if Z is None else Z
        out = self.Y2 if out is None else out
        a = gemm_args_indexed(self.w2, Z, self.routing, out, _capi.W4A16_AROW_POSITION,
                              flags=flags, split_k=self.split_k2, rows_hint=self.rows_hint)
        fused = self.fuse_combine and topk_weights is not None
        if fused:
            a.comb_out = self.out.data_ptr()
            a.comb_row_of = self.routing.row_of.data_ptr()
            a.comb_weights = topk_weights.data_ptr()
            a.comb_T = self.T
            a._refs = a._refs + (topk_weights, self.out)
        self._ws_for(("d", flags, fused), a)
        return a

    def stage_args(self, X, topk_weights=None):
        """Argument structs of the two GEMM stages as the path launches them
        (the down GEMM with the fused combine when topk_weights is given and
        fuse_combine is on)."""
        da = self.down_args(topk_weights=topk_weights)
        if self.separate_act:
            return self.gate_up_args(X, out=self.Y13, epilogue=_capi.W4A16_EPI_STORE), da
        return self.gate_up_args(X), da

    def quant_x(self, X, stream=None):
        """A8W4: X (bf16 bits [T, H]) -> self.X8."""
        quantize_mxfp8(X, self.X8, stream=stream)

    def quant_z(self, stream=None):
        """A8W4: the routed rows of Z -> self.Z8 (rows below num_tokens_padded)."""
        quantize_mxfp8(self.Z, self.Z8, rows_dev=self.routing.num_tokens_padded, stream=stream)

    def combine(self, topk_weights, stream=None):
        """The top-k combine as a call of its own (Y2 -> out)."""
        _capi.w4a16_moe_combine(self.Y2, self.Y2.shape[0], self.H, self.routing.row_of,
                                topk_weights, self.T, self.top_k, self.out, stream)

    def act(self, stream=None):
        """SiLU*gate on the rows of the padded routed layout (separate_act)."""
        r = self.routing
        _capi.w4a16_moe_silu_mul(self.Y13, r.sorted_cap, r.num_tokens_padded, self.I, self.Z,
                                 stream)

    def __call__(self, X, topk_ids, topk_weights, expert_map=None, stream=None):
        self.routing.align(topk_ids, self.E_global, expert_map, stream=stream)
        ga, da = self.stage_args(X, topk_weights)
        if self.a8:
            self.quant_x(X, stream)
        _capi.w4a16_moe_w4a16_gemm(ga, stream)
        if self.separate_act:
            self.act(stream)
        if self.a8:
            self.quant_z(stream)
        _capi.w4a16_moe_w4a16_gemm(da, stream)
        if not self.fuse_combine:
            self.combine(topk_weights, stream)
        return self.out


class MaskedPath:
    """Grouped masked layout: gate/up (+ SiLU*gate) -> down on [G*max_m] rows,
    then the top-k combine through the caller's row map."""

    def __init__(self, w13: PreparedWeight, w2: PreparedWeight, max_m: int, expected_m: int,
                 T: int, top_k: int, device="cuda"):
        self.w13, self.w2 = w13, w2
        self.G, self.max_m, self.expected_m = w13.E, max_m, expected_m
        self.T, self.top_k = T, top_k
        self.H, self.I = w13.K, w2.K
        rows = self.G * max_m
        self.Z = _dev_empty((rows, self.I), BF16, device)
        self.Y2 = _dev_empty((rows, self.H), BF16, device)
        self.out = _dev_empty((max(T, 1), self.H), BF16, device)
        self.device = device
        self._ws = {}

    def _ws_for(self, key, args):
        need = _capi.w4a16_gemm_workspace_bytes(args)
        if need == 0:
            return
        buf = self._ws.get(key)
        if buf is None or buf.numel() < need:
            buf = _workspace(need, self.device)
            self._ws[key] = buf
        args.workspace = buf.data_ptr()
        args.workspace_bytes = buf.numel()

    def gate_up_args(self, a3, masked_m, out=None, epilogue=_capi.W4A16_EPI_SILU_MUL, flags=0):
        out = self.Z if out is None else out
        a = gemm_args_masked(self.w13, a3, masked_m, self.max_m, self.expected_m, out,
                             epilogue=epilogue, flags=flags)
        self._ws_for(("g", epilogue, flags), a)
        return a

    def down_args(self, masked_m, Z=None, out=None, flags=0):
        Z = self.Z if Z is None else Z
        out = self.Y2 if out is None else out
        a = gemm_args_masked(self.w2, Z, masked_m, self.max_m, self.expected_m, out, flags=flags)
        self._ws_for(("d", flags), a)
        return a

    def __call__(self, a3, masked_m, row_of, topk_weights, stream=None):
        _capi.w4a16_moe_w4a16_gemm(self.gate_up_args(a3, masked_m), stream)
        _capi.w4a16_moe_w4a16_gemm(self.down_args(masked_m), stream)
        _capi.w4a16_moe_combine(self.Y2, self.Y2.shape[0], self.H, row_of, topk_weights, self.T,
                                self.top_k, self.out, stream)
        return self.out


class ContiguousPath:
    """Grouped contiguous layout (prefill): gate/up (+ SiLU*gate) -> down on
    the caller's [m] rows, then the top-k combine through the caller's row
    map (slot -> row).  Weights packed with the PREFILL profile."""

    def __init__(self, w13: PreparedWeight, w2: PreparedWeight, m: int, T: int, top_k: int,
                 device="cuda"):
        self.w13, self.w2 = w13, w2
        self.m, self.T, self.top_k = m, T, top_k
        self.H, self.I = w13.K, w2.K
        self.plan = _capi.w4a16_plan_gemm(w13.desc, _capi.W4A16_LAYOUT_CONTIGUOUS, m)
        self.Z = _dev_empty((max(m, 1), self.I), BF16, device)
        self.Y2 = _dev_empty((max(m, 1), self.H), BF16, device)
        self.out = _dev_empty((max(T, 1), self.H), BF16, device)
        self.device = device
        self._ws = {}

    def _ws_for(self, key, args):
        need = _capi.w4a16_gemm_workspace_bytes(args)
        if need == 0:
            return
        buf = self._ws.get(key)
        if buf is None or buf.numel() < need:
            buf = _workspace(need, self.device)
            self._ws[key] = buf
        args.workspace = buf.data_ptr()
        args.workspace_bytes = buf.numel()

    def gate_up_args(self, a2, m_indices, out=None, epilogue=_capi.W4A16_EPI_SILU_MUL, flags=0):
        out = self.Z if out is None else out
        a = gemm_args_contiguous(self.w13, a2, m_indices, out, epilogue=epilogue, flags=flags)
        self._ws_for(("g", epilogue, flags), a)
        return a

    def down_args(self, m_indices, Z=None, out=None, flags=0):
        Z = self.Z if Z is None else Z
        out = self.Y2 if out is None else out
        a = gemm_args_contiguous(self.w2, Z, m_indices, out, flags=flags)
        self._ws_for(("d", flags), a)
        return a

    def __call__(self, a2, m_indices, row_of, topk_weights, stream=None):
        _capi.w4a16_moe_w4a16_gemm(self.gate_up_args(a2, m_indices), stream)
        _capi.w4a16_moe_w4a16_gemm(self.down_args(m_indices), stream)
        _capi.w4a16_moe_combine(self.Y2, self.Y2.shape[0], self.H, row_of, topk_weights, self.T,
                                self.top_k, self.out, stream)
        return self.out
