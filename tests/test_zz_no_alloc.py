"""The allocation-free GEMM entry point (w4a16_moe_w4a16_gemm_noalloc) against
the entry point that takes a caller's workspace.

Both run the same kernels with the same schedule, so their outputs must be
bit-identical.  Each case makes two calls in a row through the C ABI, the
second with a smaller input, so the static scratch keeps the first call's
bytes (counters, partials, staged rows) when the second starts.  The cases
cover every part of the scratch: split-K arrival counters and fp32 partials,
the bf16 gate/up staging of a plain W13 with the SiLU epilogue, and the
large-M kernel's work-queue counters.
"""
import ctypes

import numpy as np
import pytest

import synth

ROWS_GUARD = 0x1234


def test_noalloc_refuses_calls_above_its_scratch_before_launching():
    """Host check, no GPU needed: a call whose workspace exceeds the static
    scratch returns CAPACITY before anything is launched."""
    capi = pytest.importorskip("w4a16_int4_mixture_amd._capi")
    E, N, K = 8, 4096, 1024
    codes = np.zeros((E, N, K // 8), np.int32)
    scales = np.zeros((E, N, K // 32), np.uint16)
    packed = np.zeros(capi.w4a16_prepack_bytes(1, 0, E, N, K), np.uint8)
    desc = capi.w4a16_prepack_host(1, 0, codes, scales, E, N, K, 32, packed)
    fake = 1 << 20
    a = capi.w4a16_gemm_args()
    a.layout = capi.W4A16_LAYOUT_INDEXED
    a.epilogue = capi.W4A16_EPI_SILU_MUL        # plain W13: Y13 staged in the scratch
    a.A, a.A_rows, a.out = fake, 4096, fake
    a.packed, a.desc = fake, ctypes.pointer(desc)
    a.sorted_ids, a.sorted_cap, a.num_tokens_padded = fake, 8192, fake
    a.tiles, a.tiles_cap, a.tile_count, a.tile_m = fake, 1024, fake, 16
    a.num_slots, a.top_k, a.out_rows = 8192, 2, 8192
    need = capi.w4a16_gemm_workspace_bytes(a)
    assert need > 32 << 20
    st = capi.lib().w4a16_moe_w4a16_gemm_noalloc(ctypes.byref(a), None)
    assert st == capi.W4A16_ERR_CAPACITY
    assert "scratch" in capi.w4a16_last_error()


@pytest.fixture(scope="module")
def m():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a16_int4_mixture_amd as mod
    return mod


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _host(t):
    return t.detach().cpu().numpy().view(np.uint16)


def _both(m, make_args):
    """Run the call through both entry points into separate outputs; return
    the two outputs and the workspace size of the call."""
    import torch
    from w4a16_int4_mixture_amd import _capi
    a_ws, out_ws = make_args()
    need = _capi.w4a16_gemm_workspace_bytes(a_ws)
    m.run_gemm(a_ws, "cuda")
    a_na, out_na = make_args()
    a_na.workspace, a_na.workspace_bytes = None, 0
    _capi.w4a16_moe_w4a16_gemm_noalloc(a_na)
    torch.cuda.synchronize()
    return _host(out_ws), _host(out_na), need


@pytest.mark.gpu
@pytest.mark.parametrize("profile,interleave,split", [(1, False, 3), (1, True, 2), (2, True, 0)])
def test_noalloc_indexed_equals_workspace_entry_point(m, profile, interleave, split):
    import torch
    from w4a16_int4_mixture_amd import _capi
    E, H, I, k = (6, 768, 256, 3) if profile == 1 else (40, 512, 1024, 4)
    w = synth.random_small(121 + profile, E, H, I, 8, k)
    flags = m.PACK_GATE_UP_INTERLEAVE if interleave else 0
    w13 = m.prepare_weight(_dev(w["codes13"]), _dev(w["scales13"]), profile, flags)
    for call, T in enumerate((600 if profile == 2 else 90, 37)):      # second call smaller
        d = synth.random_small(130 + 10 * profile + call, E, H, I, T, k)
        if profile == 2:
            # skewed routing: tiles of many heights and more items than
            # workgroups, so the large-M kernel takes its items from the
            # work-queue counters
            rng = np.random.default_rng(131 + call)
            p = 1.0 / np.arange(1, E + 1) ** 0.8
            p /= p.sum()
            d["topk_ids"] = np.stack([rng.choice(E, size=k, replace=False, p=p)
                                      for _ in range(T)]).astype(np.int32)
        plan = _capi.w4a16_plan_gemm(w13.desc, _capi.W4A16_LAYOUT_INDEXED, T * k, 0, 0)
        r = m.Routing(T, k, E, plan.block_m, plan.tile_m, "cuda")
        r.align(_dev(d["topk_ids"]), E)
        X = _dev(d["X"])

        def make_args():
            out = torch.full((r.sorted_cap, I), ROWS_GUARD, dtype=torch.int16, device="cuda")
            a = m.gemm_args_indexed(w13, X, r, out, _capi.W4A16_AROW_TOKEN,
                                    epilogue=_capi.W4A16_EPI_SILU_MUL, split_k=split,
                                    rows_hint=T * k)
            return a, out

        got_ws, got_na, need = _both(m, make_args)
        print(f"noalloc indexed: profile={profile} interleave={interleave} split={split} "
              f"call={call} T={T} workspace={need} B", flush=True)
        assert need > 0
        assert np.array_equal(got_ws, got_na), f"call {call}: outputs differ"
        s = r.sorted_ids.cpu().numpy()
        n = int(r.num_tokens_padded.cpu().numpy()[0])
        valid = np.nonzero(s[:n] < T * k)[0]
        assert valid.size > 0 and np.all(got_na[valid] != ROWS_GUARD), "a routed row not written"


@pytest.mark.gpu
def test_noalloc_masked_equals_workspace_entry_point(m):
    import torch
    from w4a16_int4_mixture_amd import _capi
    G, H, I, max_m = 5, 512, 256, 64
    w = synth.random_small(141, G, H, I, 8, 1)
    w13 = m.prepare_weight(_dev(w["codes13"]), _dev(w["scales13"]), 1, 0)
    rng = np.random.default_rng(142)
    for call, counts in enumerate(([64, 0, 33, 17, 50], [5, 9, 0, 2, 1])):
        counts = np.array(counts, np.int32)
        a3 = np.full((G * max_m, H), synth.BF16_NAN, np.uint16)
        for g, c in enumerate(counts):
            a3[g * max_m: g * max_m + c] = synth.random_activations(rng, c, H)
        A, mm = _dev(a3), _dev(counts)

        def make_args():
            out = torch.full((G * max_m, I), ROWS_GUARD, dtype=torch.int16, device="cuda")
            a = m.gemm_args_masked(w13, A, mm, max_m, 16, out,
                                   epilogue=_capi.W4A16_EPI_SILU_MUL)
            return a, out

        got_ws, got_na, need = _both(m, make_args)
        print(f"noalloc masked: call={call} counts={counts.tolist()} workspace={need} B",
              flush=True)
        assert need > 0
        valid = np.concatenate([g * max_m + np.arange(c) for g, c in enumerate(counts)])
        assert np.array_equal(got_ws[valid], got_na[valid]), f"call {call}: outputs differ"
        invalid = np.setdiff1d(np.arange(G * max_m), valid)
        assert np.all(got_na[invalid] == ROWS_GUARD), "padding rows were written"
