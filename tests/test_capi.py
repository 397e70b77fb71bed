"""Host-side tests of the C-ABI library (no GPU needed).

* every function declared in include/w4a16moe.h is exported by libw4a16moe.so;
* the ctypes structures agree with the C layout (sizes and offsets printed by a
  program compiled from the header with gcc);
* argument checks reject bad calls before anything is launched, with the
  documented status codes;
* the host prepack writes exactly the documented device layout;
* the schedule chooser follows its stated rules.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16moe.h")

capi = pytest.importorskip("w4a16_int4_mixture_amd._capi")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    lib = capi.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", capi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert set(names) <= exported
    assert set(names) == set(capi.SIGNATURES)


def _c_layout(tmp_path):
    structs = {
        "w4a16_desc": [f[0] for f in capi.w4a16_desc._fields_],
        "w4a16_routing": [f[0] for f in capi.w4a16_routing._fields_],
        "w4a16_gemm_args": [f[0] for f in capi.w4a16_gemm_args._fields_],
        "w4a16_plan": [f[0] for f in capi.w4a16_plan._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for s, fields in structs.items():
        lines.append(f'printf("{s} sizeof %zu\\n", sizeof({s}));')
        for f in fields:
            lines.append(f'printf("{s} {f} %zu\\n", offsetof({s}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    return [l.split() for l in out.splitlines()]


def test_ctypes_structs_match_c_layout(tmp_path):
    for s, what, val in _c_layout(tmp_path):
        cls = getattr(capi, s)
        if what == "sizeof":
            assert ctypes.sizeof(cls) == int(val), s
        else:
            assert getattr(cls, what).offset == int(val), (s, what)


def test_header_compiles_as_c_and_cpp(tmp_path):
    src = tmp_path / "h.c"
    src.write_text(f'#include "{HEADER}"\nint main(void){{return 0;}}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-c", str(src), "-o",
                    str(tmp_path / "h.o")], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-x", "c++", "-c",
                    str(src), "-o", str(tmp_path / "hpp.o")], check=True)


# ---- argument checks (nothing is launched) -----------------------------------

def status_of(fn, *a):
    try:
        fn(*a)
    except capi.W4A16Error as e:
        return e.status
    return capi.W4A16_OK


def test_prepack_bytes_rejects_unsupported_schemes():
    P = capi.W4A16_PROFILE_DECODE
    # codes + scales exactly, K in whole records of 8 groups (7168 = 28 records)
    assert capi.w4a16_prepack_bytes(P, 0, 48, 4096, 7168, 32) == 48 * 4096 * 7168 // 2 + 48 * 4096 * 224 * 2
    # K = 96: 3 groups padded to one record of 8
    assert capi.w4a16_prepack_bytes(P, 0, 1, 64, 96, 32) == 64 * 256 // 2 + 64 * 8 * 2
    assert status_of(capi.w4a16_prepack_bytes, P, 0, 1, 64, 64, 64) == capi.W4A16_ERR_UNSUPPORTED
    assert status_of(capi.w4a16_prepack_bytes, P, 0, 1, 64, 48, 32) == capi.W4A16_ERR_UNSUPPORTED
    assert status_of(capi.w4a16_prepack_bytes, P, 0, 1, 96, 64, 32) == capi.W4A16_ERR_UNSUPPORTED
    assert status_of(capi.w4a16_prepack_bytes, capi.W4A16_PROFILE_PREFILL, 0, 1, 64, 64, 32) == \
        capi.W4A16_ERR_UNSUPPORTED
    assert status_of(capi.w4a16_prepack_bytes, 7, 0, 1, 64, 64, 32) == capi.W4A16_ERR_UNSUPPORTED
    assert status_of(capi.w4a16_prepack_bytes, P, 0x80, 1, 64, 64, 32) == capi.W4A16_ERR_UNSUPPORTED
    assert status_of(capi.w4a16_prepack_bytes, P, 0, 0, 64, 64, 32) == capi.W4A16_ERR_INVALID_ARG
    assert "group" in capi.w4a16_last_error() or capi.w4a16_last_error() != ""


def test_align_capacity_and_checks():
    sc, bc, tc = capi.w4a16_moe_align_capacity(64, 8, 48, 16, 32)
    assert sc == 512 + 48 * 15 and bc == sc // 16 and tc == 16 + 48
    assert status_of(capi.w4a16_moe_align_capacity, 4, 2, 0, 16, 0) == capi.W4A16_ERR_INVALID_ARG
    assert status_of(capi.w4a16_moe_align_capacity, 4, 2, 8, 0, 0) == capi.W4A16_ERR_INVALID_ARG
    assert status_of(capi.w4a16_moe_align_capacity, 4, 2, 8, 16, 24) == capi.W4A16_ERR_INVALID_ARG
    # capacity too small -> CAPACITY, before any launch
    fake = 1 << 20
    r = capi.w4a16_routing(sorted_ids=fake, sorted_cap=8, expert_ids=fake, blocks_cap=1,
                           num_tokens_padded=fake)
    st = capi.lib().w4a16_moe_align(fake, 4, 2, 8, None, 8, 16, ctypes.byref(r), 0, None)
    assert st == capi.W4A16_ERR_CAPACITY
    st = capi.lib().w4a16_moe_align(fake, 4, 2, 8, None, 2000, 16, ctypes.byref(r), 0, None)
    assert st == capi.W4A16_ERR_INVALID_ARG
    st = capi.lib().w4a16_moe_align(fake, 4, 2, 8, None, 8, 16, None, 0, None)
    assert st == capi.W4A16_ERR_INVALID_ARG
    r2 = capi.w4a16_routing(sorted_ids=fake, sorted_cap=1000, expert_ids=fake, blocks_cap=100,
                            num_tokens_padded=fake, tiles=fake + 8, tiles_cap=100, tile_count=fake,
                            tile_m=16)
    st = capi.lib().w4a16_moe_align(fake, 4, 2, 8, None, 8, 16, ctypes.byref(r2), 0, None)
    assert st == capi.W4A16_ERR_INVALID_ARG            # misaligned tile table


def host_desc(profile=capi.W4A16_PROFILE_DECODE, flags=0, E=2, N=128, K=64):
    codes = np.zeros((E, N, K // 8), np.int32)
    scales = np.zeros((E, N, K // 32), np.uint16)
    nb = capi.w4a16_prepack_bytes(profile, flags, E, N, K)
    packed = np.zeros(nb, np.uint8)
    return capi.w4a16_prepack_host(profile, flags, codes, scales, E, N, K, 32, packed)


def gemm_args(desc, **kw):
    fake = 1 << 20
    a = capi.w4a16_gemm_args()
    a.layout = capi.W4A16_LAYOUT_INDEXED
    a.A, a.A_rows, a.out, a.out_rows = fake, 64, fake, 4096
    a.packed = fake
    a.desc = ctypes.pointer(desc)
    a.sorted_ids, a.sorted_cap, a.num_tokens_padded = fake, 256, fake
    a.tiles, a.tiles_cap, a.tile_count, a.tile_m = fake, 8, fake, 32
    a.num_slots, a.top_k = 64, 2
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def ws_status(a):
    return status_of(capi.w4a16_gemm_workspace_bytes, a)


def test_gemm_argument_checks():
    d = host_desc()
    assert ws_status(gemm_args(d)) == capi.W4A16_OK
    bad = capi.w4a16_desc.from_buffer_copy(d)
    bad.magic = 0
    assert ws_status(gemm_args(bad)) == capi.W4A16_ERR_MODE_MISMATCH
    bad = capi.w4a16_desc.from_buffer_copy(d)
    bad.bytes += 256
    assert ws_status(gemm_args(bad)) == capi.W4A16_ERR_MODE_MISMATCH
    assert ws_status(gemm_args(d, A=(1 << 20) + 2)) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, packed=(1 << 20) + 64)) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, tile_m=24)) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, tile_m=512)) == capi.W4A16_ERR_UNSUPPORTED
    assert ws_status(gemm_args(d, out_rows=10)) == capi.W4A16_ERR_CAPACITY
    assert ws_status(gemm_args(d, epilogue=capi.W4A16_EPI_SILU_MUL,
                               flags=capi.W4A16_GEMM_F32_OUT)) == capi.W4A16_ERR_INVALID_ARG
    # interleaved W13 with a plain store: the columns would come out permuted
    di = host_desc(flags=capi.W4A16_PACK_GATE_UP_INTERLEAVE)
    assert ws_status(gemm_args(di)) == capi.W4A16_ERR_MODE_MISMATCH
    # interleaved W13 with the SiLU epilogue: applied in the GEMM, no staging
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(di, epilogue=capi.W4A16_EPI_SILU_MUL)) == 0
    # a plain W13 with the SiLU epilogue stages bf16 Y13 [sorted_cap, N]
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(d, epilogue=capi.W4A16_EPI_SILU_MUL)) == \
        256 * 128 * 2
    # a PREFILL weight: the large-M kernel's work-queue counters, one 256-byte
    # block before the Y13 staging
    dp = host_desc(profile=capi.W4A16_PROFILE_PREFILL)
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(dp)) == 256
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(dp, epilogue=capi.W4A16_EPI_SILU_MUL)) == \
        256 + 256 * 128 * 2
    # masked: expected_m must be positive; split_k overrides are refused
    m = dict(layout=capi.W4A16_LAYOUT_MASKED, masked_m=1 << 20, max_m=32, expected_m=32,
             A_rows=64, out_rows=64)
    assert ws_status(gemm_args(d, **m)) == capi.W4A16_OK
    assert ws_status(gemm_args(d, **{**m, "expected_m": 0})) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, **{**m, "split_k": 2})) == capi.W4A16_ERR_MODE_MISMATCH
    assert ws_status(gemm_args(d, **{**m, "A_rows": 10})) == capi.W4A16_ERR_CAPACITY
    # K splits are whole 8-group records: one record cannot be split
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(d, split_k=2)) == 0
    # two splits: arrival counters (one per tile x part x column group of four
    # 64-column chunks, 256-byte granular), then fp32 partials [2, sorted_cap, N]
    d512 = host_desc(K=512)
    a = gemm_args(d512, split_k=2)
    counters = -(-8 * 4 * 1 * 4 // 256) * 256
    assert capi.w4a16_gemm_workspace_bytes(a) == counters + 2 * 256 * 128 * 4
    # launching with a too-small workspace fails before the launch
    assert capi.lib().w4a16_moe_w4a16_gemm(ctypes.byref(a), None) == capi.W4A16_ERR_CAPACITY


def test_split_k_partials_stay_below_4gib():
    """A split's fp32 partial [sorted_cap, N] is addressed with 32-bit byte
    offsets: a forced split whose partial reaches 4 GiB is refused before any
    launch, and the automatic choice runs unsplit instead (no partials in the
    workspace)."""
    d = host_desc(E=8, N=4096, K=1024)
    big = dict(sorted_cap=300000, out_rows=300000, tiles_cap=20000, num_slots=262144, top_k=8,
               A_rows=32768)
    assert 300000 * 4096 * 4 >= 1 << 32
    assert ws_status(gemm_args(d, split_k=2, **big)) == capi.W4A16_ERR_UNSUPPORTED
    assert "4 GiB" in capi.w4a16_last_error()
    # automatic: no split, so no counters and no partials
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(d, **big)) == 0
    # the same forced split on a partial below 4 GiB is accepted
    small = dict(big, sorted_cap=200000, out_rows=200000)
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(d, split_k=2, **small)) >= 2 * 200000 * 4096 * 4


def test_split_sizing_without_row_hint_uses_sorted_cap():
    """With no rows_hint the automatic split sizes its partials from the
    routing capacity (every split writes an fp32 partial of sorted_cap rows),
    not from one row per expert: a large capacity gets fewer splits."""
    d = host_desc(E=8, N=256, K=4096)
    ws_small = capi.w4a16_gemm_workspace_bytes(gemm_args(d, sorted_cap=64, out_rows=64))
    ws_large = capi.w4a16_gemm_workspace_bytes(gemm_args(d, sorted_cap=65536, out_rows=65536))
    # small capacity: split (partials present); large: the partials would
    # exceed a quarter of the weight stream, so it runs unsplit
    assert ws_small > 0
    assert ws_large == 0


def test_combine_and_silu_checks():
    fake = 1 << 20
    assert capi.lib().w4a16_moe_combine(fake, 4, 12, fake, fake, 1, 1, fake, None) == \
        capi.W4A16_ERR_INVALID_ARG
    assert capi.lib().w4a16_moe_combine(fake + 2, 4, 16, fake, fake, 1, 1, fake, None) == \
        capi.W4A16_ERR_INVALID_ARG
    assert capi.lib().w4a16_moe_silu_mul(fake, 4, None, 12, fake, None) == \
        capi.W4A16_ERR_INVALID_ARG


# ---- host prepack = documented layout -------------------------------------------

def decode_packed_prefill(packed, desc):
    """PREFILL layout (32x32x16 MFMA operands): per expert and 128-column
    chunk, records of 8 groups = codes [8 groups][2 halves h][64 lanes][4
    words v] then scales [2 h][32 columns][8 groups][2] bf16.  Word (h, lane,
    v) holds column 32*(h + 2*(v//2)) + lane%32, K offsets 16*(v%2) +
    8*(lane//32) + o in nibble o; scale (h, c32, group, jj) is column
    32*(h + 2*jj) + c32."""
    E, N, K = desc.E, desc.N, desc.K
    NC, KS, KSP = N // 128, K // 32, desc.k_groups
    R = KSP // 8
    rec = packed.view(np.uint32).reshape(E, NC, R, 4608)
    # axes: e, chunk, record, group, h, K octet (lane//32), c32, jj, step
    w = rec[..., :4096].reshape(E, NC, R, 8, 2, 2, 32, 2, 2)
    # -> e, chunk, jj, h, c32 (column 64 jj + 32 h + c32) | record, group, step, octet
    w = w.transpose(0, 1, 7, 4, 6, 2, 3, 8, 5).reshape(E, N, KSP * 4)
    assert not w[:, :, K // 8:].any()                       # padding codes are zero
    codes = np.ascontiguousarray(w[:, :, : K // 8])
    sc = np.ascontiguousarray(rec[..., 4096:]).view(np.uint16)
    # axes: e, chunk, record, h, c32, group, jj -> e, chunk, jj, h, c32 | record, group
    sc = sc.reshape(E, NC, R, 2, 32, 8, 2).transpose(0, 1, 6, 3, 4, 2, 5).reshape(E, N, KSP)
    assert not sc[:, :, KS:].any()                          # padding scales are zero
    return codes.view(np.int32), sc[:, :, :KS]


def decode_packed(packed, desc):
    """Read the packed buffer back into canonical codes and scales, from the
    layout as documented in the library.  DECODE: per expert and chunk,
    records of 8 groups, each = codes [8][64 lanes][CW/16 words] (nibble i
    holding K offset 2*(i%4) + i/4) followed by scales [8][16][CW/16] bf16;
    padding groups zero.  PREFILL: decode_packed_prefill."""
    if desc.profile == capi.W4A16_PROFILE_PREFILL:
        return decode_packed_prefill(packed, desc)
    E, N, K, CW = desc.E, desc.N, desc.K, desc.chunk_n
    NC, KS, WPL, KSP = N // CW, K // 32, CW // 16, desc.k_groups
    rec = packed.view(np.uint32).reshape(E, NC, KSP // 8, 576 * WPL)
    words = rec[..., : 512 * WPL].reshape(E, NC, KSP // 8, 8, 4, 16, WPL)
    # axes: e, chunk, record, group-in-record, K octet (lane//16), lane%16, block j
    # MXFP4 keeps the canonical nibble order (nibble i = K offset i)
    if desc.flags & capi.W4A16_PACK_MXFP4:
        off = np.arange(8)
    else:
        off = np.array([2 * (i % 4) + i // 4 for i in range(8)])
    nib = (words[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    q = np.zeros(nib.shape, np.uint32)
    q[..., off] = nib                                       # -> K offset order
    # -> [e, chunk, j, c16, record, group, octet, 8]
    q = q.transpose(0, 1, 6, 5, 2, 3, 4, 7).reshape(E, N, KSP * 32)
    assert not q[:, :, K:].any()                            # padding codes are zero
    q = q[:, :, :K]
    codes = np.zeros((E, N, K // 8), np.uint32)
    for o in range(8):
        codes |= q[:, :, o::8] << (4 * o)
    sc = np.ascontiguousarray(rec[..., 512 * WPL:]).view(np.uint16)
    sc = sc.reshape(E, NC, KSP // 8, 8, 16, WPL).transpose(0, 1, 5, 4, 2, 3).reshape(E, N, KSP)
    assert not sc[:, :, KS:].any()                          # padding scales are zero
    return codes.view(np.int32), sc[:, :, :KS]


@pytest.mark.parametrize("profile,flags", [(capi.W4A16_PROFILE_DECODE, 0),
                                           (capi.W4A16_PROFILE_PREFILL, 0),
                                           (capi.W4A16_PROFILE_DECODE, capi.W4A16_PACK_GATE_UP_INTERLEAVE),
                                           (capi.W4A16_PROFILE_PREFILL, capi.W4A16_PACK_GATE_UP_INTERLEAVE)])
def test_host_prepack_matches_documented_layout(profile, flags):
    rng = np.random.default_rng(profile * 10 + flags)
    E, N, K = 3, 256, 96
    codes = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    scales = rng.integers(0, 2**16, size=(E, N, K // 32), dtype=np.uint16)
    packed = np.zeros(capi.w4a16_prepack_bytes(profile, flags, E, N, K), np.uint8)
    desc = capi.w4a16_prepack_host(profile, flags, codes, scales, E, N, K, 32, packed)
    assert desc.magic == capi.W4A16_DESC_MAGIC and desc.profile == profile
    c2, s2 = decode_packed(packed, desc)
    if flags & capi.W4A16_PACK_GATE_UP_INTERLEAVE:
        CW = desc.chunk_n
        half = CW // 2
        perm = []
        for nn in range(N):
            c, w = divmod(nn, CW)
            perm.append(c * half + w if w < half else N // 2 + c * half + (w - half))
        codes, scales = codes[:, perm], scales[:, perm]
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2, scales)


# ---- schedule chooser -------------------------------------------------------------

def test_plan_rules():
    d13 = host_desc(E=48, N=4096, K=7168)
    d2 = host_desc(E=48, N=7168, K=2048)
    p = capi.w4a16_plan_gemm(d13, capi.W4A16_LAYOUT_INDEXED, 512)       # ~10.7 rows/expert
    # every expert in one tile of up to 32 rows, the one-stage ring (three
    # workgroups per CU)
    assert p.tile_m == 32 and p.block_m == 16 and p.split_k >= 1 and p.ring_groups == 8
    # 48+ tiles x 16 column quads already fill the resident workgroups: no K split
    assert p.split_k == 1
    p_small = capi.w4a16_plan_gemm(d13, capi.W4A16_LAYOUT_INDEXED, 96)
    assert p_small.tile_m == 16 and p_small.ring_groups == 8
    # ~21 rows per expert, deep K: two-stage ring; K of one record: one-stage ring
    d13_tp = host_desc(E=24, N=128, K=7168)
    d2_tp = host_desc(E=24, N=1024, K=256)
    p_tp = capi.w4a16_plan_gemm(d13_tp, capi.W4A16_LAYOUT_INDEXED, 512)
    assert p_tp.tile_m == 32 and p_tp.ring_groups == 16
    assert capi.w4a16_plan_gemm(d2_tp, capi.W4A16_LAYOUT_INDEXED, 512, 0, 32).ring_groups == 8
    assert capi.w4a16_plan_gemm(host_desc(profile=capi.W4A16_PROFILE_PREFILL, E=2, N=256,
                                          K=512), capi.W4A16_LAYOUT_INDEXED, 512).ring_groups == 0
    assert p_small.split_k >= p.split_k                                   # fewer tiles -> more splits
    assert capi.w4a16_plan_gemm(d13, capi.W4A16_LAYOUT_INDEXED, 0, tile_m=48).tile_m == 48
    # masked: tiles of expected_m rows, in 16-row steps
    assert capi.w4a16_plan_gemm(d13, capi.W4A16_LAYOUT_MASKED, 0, 32).tile_m == 32
    assert capi.w4a16_plan_gemm(d2, capi.W4A16_LAYOUT_MASKED, 0, 32).tile_m == 32
    assert capi.w4a16_plan_gemm(d2, capi.W4A16_LAYOUT_MASKED, 0, 20).tile_m == 32
    assert capi.w4a16_plan_gemm(d2, capi.W4A16_LAYOUT_MASKED, 0, 16).tile_m == 16
    assert status_of(capi.w4a16_plan_gemm, d13, capi.W4A16_LAYOUT_MASKED, 0, 0) == \
        capi.W4A16_ERR_INVALID_ARG
    for pl in (p, p_small):
        assert 4096 // 64 * pl.split_k >= 1 and 224 // pl.split_k >= 8


def test_contiguous_layout_checks_and_plan():
    """The grouped contiguous layout runs on PREFILL-profile weights only,
    needs m_indices and an output of m rows, refuses split_k overrides, and
    takes 128-row blocks when the grid fills the machine, else 64."""
    dp = host_desc(profile=capi.W4A16_PROFILE_PREFILL, N=4096, K=64)
    dd = host_desc(profile=capi.W4A16_PROFILE_DECODE, N=4096, K=64)
    c = dict(layout=capi.W4A16_LAYOUT_CONTIGUOUS, m_indices=1 << 20, A_rows=2048, out_rows=2048,
             tiles=None, sorted_ids=None, num_tokens_padded=None)
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(dp, **c)) == 256     # work-queue block
    assert ws_status(gemm_args(dd, **c)) == capi.W4A16_ERR_MODE_MISMATCH
    assert ws_status(gemm_args(dp, **{**c, "m_indices": None})) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(dp, **{**c, "split_k": 2})) == capi.W4A16_ERR_MODE_MISMATCH
    assert ws_status(gemm_args(dp, **{**c, "out_rows": 2047})) == capi.W4A16_ERR_CAPACITY
    # a plain W13 with the SiLU epilogue stages Y13 [m, N]
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(dp, epilogue=capi.W4A16_EPI_SILU_MUL, **c)) \
        == 256 + 2048 * 4096 * 2
    # N = 4096: 32 chunks of 128 columns, 16 column pairs; 2048 rows = 16 blocks
    # of 128 -> 256 items fill 256 CUs; 1024 rows would not
    L = capi.W4A16_LAYOUT_CONTIGUOUS
    assert capi.w4a16_plan_gemm(dp, L, 2048).tile_m == 128
    assert capi.w4a16_plan_gemm(dp, L, 1024).tile_m == 64
    assert capi.w4a16_plan_gemm(dp, L, 2048).kernel == 2
    assert status_of(capi.w4a16_plan_gemm, dd, L, 2048) == capi.W4A16_ERR_MODE_MISMATCH


def test_fused_combine_checks():
    """The fused combine needs the streaming kernel, the tile table,
    position-indexed bf16 rows, its routing buffers and comb_T * top_k ==
    num_slots; its arrival counters join the workspace's counters."""
    d = host_desc(K=64)
    fake = 1 << 20
    c = dict(comb_out=fake, comb_row_of=fake, comb_weights=fake, comb_T=32, top_k=2,
             num_slots=64)
    base = capi.w4a16_gemm_workspace_bytes(gemm_args(d))
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(d, **c)) == base + 256   # 32 tokens x 1 group
    assert ws_status(gemm_args(d, **{**c, "comb_T": 31})) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, **{**c, "comb_row_of": None})) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, orow=capi.W4A16_OROW_SLOT, **c)) == capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, flags=capi.W4A16_GEMM_F32_OUT, **c)) == \
        capi.W4A16_ERR_INVALID_ARG
    assert ws_status(gemm_args(d, tiles=None, expert_ids=fake, blocks_cap=16, block_m=16, **c)) \
        == capi.W4A16_ERR_INVALID_ARG
    dp = host_desc(profile=capi.W4A16_PROFILE_PREFILL, K=64)
    assert ws_status(gemm_args(dp, **c)) == capi.W4A16_ERR_UNSUPPORTED


def test_host_prepack_mxfp4_matches_documented_layout():
    """MXFP4 weights: the DECODE layout with the codes' canonical nibble order
    and each E8M0 byte b stored as the bf16 2^(b - 127) (0x0040 for b = 0,
    NaN for 255); the interleave permutes columns as for INT4; the PREFILL
    profile and the INT4 packers refuse MXFP4."""
    rng = np.random.default_rng(9)
    E, N, K = 2, 128, 288
    codes = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    b = rng.integers(0, 256, size=(E, N, K // 32)).astype(np.uint8)
    b[0, 0, 0], b[0, 1, 0], b[1, 2, 3] = 0, 255, 127
    for flags in (0, capi.W4A16_PACK_GATE_UP_INTERLEAVE):
        nb = capi.w4a16_prepack_bytes(capi.W4A16_PROFILE_DECODE, flags, E, N, K)
        packed = np.zeros(nb, np.uint8)
        desc = capi.w4a16_prepack_mxfp4_host(capi.W4A16_PROFILE_DECODE, flags, codes, b, E, N, K,
                                             32, packed)
        assert desc.flags == flags | capi.W4A16_PACK_MXFP4
        got_codes, got_sc = decode_packed(packed, desc)
        if flags:
            perm = np.array([(nn // 64) * 32 + (nn % 64) if nn % 64 < 32 else
                             N // 2 + (nn // 64) * 32 + (nn % 64) - 32 for nn in range(N)])
            want_codes, want_b = codes[:, perm], b[:, perm]
        else:
            want_codes, want_b = codes, b
        assert np.array_equal(got_codes, want_codes)
        want_sc = np.where(want_b == 255, 0x7FC0,
                           np.where(want_b == 0, 0x0040, want_b.astype(np.uint32) << 7))
        assert np.array_equal(got_sc, want_sc.astype(np.uint16))
    packed = np.zeros(capi.w4a16_prepack_bytes(capi.W4A16_PROFILE_DECODE, 0, E, N, K), np.uint8)
    assert status_of(capi.w4a16_prepack_mxfp4_host, capi.W4A16_PROFILE_PREFILL, 0, codes, b, E, N,
                     K, 32, packed) == capi.W4A16_ERR_UNSUPPORTED
    sc16 = np.zeros((E, N, K // 32), np.uint16)
    assert status_of(capi.w4a16_prepack_host, capi.W4A16_PROFILE_DECODE, capi.W4A16_PACK_MXFP4,
                     codes, sc16, E, N, K, 32, packed) == capi.W4A16_ERR_INVALID_ARG


def test_host_prepack_a8w4_matches_documented_layout():
    """MXFP4 weights for MXFP8 activations (PACK_MXFP8_ACT): per record of 256
    K, the B-operand slices of the block-scaled instruction (lane l: column
    16j + l%16, 32 canonical codes from K = 256r + 128s + 32(l/16)), then one
    word of four E8M0 bytes per (step, lane); padding groups zero; the
    interleave permutes columns as for INT4.  The flag needs MXFP4."""
    rng = np.random.default_rng(19)
    E, N, K = 2, 128, 288                   # 9 groups: the second record is mostly padding
    KS, nrec, NC = K // 32, 2, N // 64
    codes = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32)
    b = rng.integers(0, 256, size=(E, N, KS)).astype(np.uint8)
    for flags in (capi.W4A16_PACK_MXFP8_ACT,
                  capi.W4A16_PACK_MXFP8_ACT | capi.W4A16_PACK_GATE_UP_INTERLEAVE):
        nb = capi.w4a16_prepack_bytes(capi.W4A16_PROFILE_DECODE, flags | capi.W4A16_PACK_MXFP4,
                                      E, N, K)
        assert nb == E * NC * nrec * 544 * 4 * 4
        packed = np.zeros(nb, np.uint8)
        desc = capi.w4a16_prepack_mxfp4_host(capi.W4A16_PROFILE_DECODE, flags,
                                             codes.view(np.int32), b, E, N, K, 32, packed)
        assert desc.flags == flags | capi.W4A16_PACK_MXFP4
        if flags & capi.W4A16_PACK_GATE_UP_INTERLEAVE:
            perm = np.array([(nn // 64) * 32 + (nn % 64) if nn % 64 < 32 else
                             N // 2 + (nn // 64) * 32 + (nn % 64) - 32 for nn in range(N)])
        else:
            perm = np.arange(N)
        cw = np.zeros((E, N, nrec * 32), np.uint32)           # codes padded to whole records
        cw[:, :, :K // 8] = codes[:, perm]
        bw = np.zeros((E, N, nrec * 8), np.uint32)
        bw[:, :, :KS] = b[:, perm]
        words = packed.view(np.uint32).reshape(E, NC, nrec, 2176)
        for r in range(nrec):
            for s_ in range(2):
                for j in range(4):
                    for lane in range(64):
                        n = np.arange(NC) * 64 + 16 * j + lane % 16
                        base = ((s_ * 4 + j) * 64 + lane) * 4
                        kw = r * 32 + s_ * 16 + 4 * (lane // 16)
                        assert np.array_equal(words[:, :, r, base:base + 4], cw[:, n, kw:kw + 4])
                for lane in range(64):
                    blk = r * 8 + 4 * s_ + lane // 16
                    want = sum(bw[:, np.arange(NC) * 64 + 16 * j + lane % 16, blk] << (8 * j)
                               for j in range(4))
                    assert np.array_equal(words[:, :, r, 2048 + s_ * 64 + lane], want)
    packed = np.zeros(capi.w4a16_prepack_bytes(capi.W4A16_PROFILE_DECODE, 0, E, N, K), np.uint8)
    sc16 = np.zeros((E, N, KS), np.uint16)
    assert status_of(capi.w4a16_prepack_host, capi.W4A16_PROFILE_DECODE,
                     capi.W4A16_PACK_MXFP8_ACT, codes.view(np.int32), sc16, E, N, K, 32,
                     packed) == capi.W4A16_ERR_UNSUPPORTED


def test_prepare_weight_refuses_codes_it_would_misread():
    """The packer sizes its reads from the codes' shape (eight 4-bit codes per
    int32 word): codes of another dtype, or scales of another shape or dtype,
    are refused on the host before any kernel runs."""
    import torch
    import w4a16_int4_mixture_amd as m
    E, N, K = 2, 64, 256
    good_c = torch.zeros((E, N, K // 8), dtype=torch.int32)
    good_s = torch.zeros((E, N, K // 32), dtype=torch.int16)
    for c, s in [(torch.zeros((E, N, K), dtype=torch.uint8), good_s),        # one code per byte
                 (good_c.to(torch.int64), good_s),
                 (good_c, torch.zeros((E, N, K // 16), dtype=torch.int16)),  # wrong group count
                 (good_c, good_s.to(torch.float32)),
                 (good_c[0], good_s[0])]:
        with pytest.raises(ValueError):
            m.prepare_weight(c, s, m.PROFILE_DECODE)
    with pytest.raises(ValueError):
        m.prepare_weight_mxfp4(good_c, good_s)                               # E8M0 scales are bytes
    with pytest.raises(ValueError):
        m.prepare_weight_mxfp4(torch.zeros((E, N, K), dtype=torch.uint8),
                               torch.zeros((E, N, K // 32), dtype=torch.uint8))


def test_a8w4_argument_checks():
    """A weight packed for MXFP8 activations needs A_scales, and A_scales needs
    such a weight (MODE_MISMATCH either way); A8W4 runs the indexed layout
    without K splits (an override is ignored: no workspace) and without the
    fused combine; the quantizer refuses a K that is not a multiple of 32."""
    E, N, K = 2, 128, 256
    codes = np.zeros((E, N, K // 8), np.int32)
    b = np.zeros((E, N, K // 32), np.uint8)
    fl = capi.W4A16_PACK_MXFP8_ACT
    packed = np.zeros(capi.w4a16_prepack_bytes(capi.W4A16_PROFILE_DECODE,
                                               fl | capi.W4A16_PACK_MXFP4, E, N, K), np.uint8)
    d8 = capi.w4a16_prepack_mxfp4_host(capi.W4A16_PROFILE_DECODE, fl, codes, b, E, N, K, 32,
                                       packed)
    fake = 1 << 20
    assert ws_status(gemm_args(d8, A_scales=fake)) == capi.W4A16_OK
    assert ws_status(gemm_args(d8)) == capi.W4A16_ERR_MODE_MISMATCH
    assert ws_status(gemm_args(host_desc(K=K), A_scales=fake)) == capi.W4A16_ERR_MODE_MISMATCH
    assert capi.w4a16_gemm_workspace_bytes(gemm_args(d8, A_scales=fake, split_k=2)) == 0
    m = dict(layout=capi.W4A16_LAYOUT_MASKED, masked_m=fake, max_m=32, expected_m=32,
             A_rows=64, out_rows=64, A_scales=fake)
    assert ws_status(gemm_args(d8, **m)) == capi.W4A16_ERR_UNSUPPORTED
    assert ws_status(gemm_args(d8, A_scales=fake, comb_out=fake, comb_row_of=fake,
                               comb_weights=fake, comb_T=32)) == capi.W4A16_ERR_UNSUPPORTED
    for bad_k in (0, 48):
        assert capi.lib().w4a16_quantize_mxfp8(fake, 4, None, bad_k, fake, fake, None) == \
            capi.W4A16_ERR_INVALID_ARG
