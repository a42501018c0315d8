"""The allocation-free logits + top-16 (GPU): dflash2_logits_topk_noalloc,
called through the C ABI, against dflash2_logits_topk on the same inputs,
bit for bit, on two calls in a row (the second smaller, so the fixed
scratch still holds the first call's tile maxima) and for each dtype."""
import ctypes

import numpy as np
import pytest
import torch

import block_drafting_amd as bd

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call_noalloc(h, Wp, code, V, M, H):
    z = torch.full((M, V), float("nan"), dtype=torch.float32, device=DEV)
    tv = torch.full((M, 16), -7.0, dtype=torch.float32, device=DEV)
    ti = torch.full((M, 16), -7, dtype=torch.int32, device=DEV)
    st = bd.lib().dflash2_logits_topk_noalloc(
        ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(Wp), ctypes.c_void_p(z.data_ptr()),
        ctypes.c_void_p(tv.data_ptr()), ctypes.c_void_p(ti.data_ptr()), M, H, V, 16, code,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, bd.lib().dflash2_strerror(st)
    return z, tv, ti


def _call_workspace(h, Wp, code, V, M, H):
    z = torch.empty((M, V), dtype=torch.float32, device=DEV)
    tv = torch.empty((M, 16), dtype=torch.float32, device=DEV)
    ti = torch.empty((M, 16), dtype=torch.int32, device=DEV)
    need = int(bd.lib().dflash2_logits_topk_workspace(M, H, V, 16, code, 1))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    st = bd.lib().dflash2_logits_topk(
        ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(Wp), ctypes.c_void_p(z.data_ptr()),
        ctypes.c_void_p(tv.data_ptr()), ctypes.c_void_p(ti.data_ptr()), M, H, V, 16, code,
        ctypes.c_void_p(ws.data_ptr()), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, bd.lib().dflash2_strerror(st)
    return z, tv, ti


@pytest.mark.parametrize("dt,code", [("bf16", 1), ("packed", 2), ("f32", 0)])
def test_noalloc_matches_the_workspace_call_twice(dt, code):
    g = torch.Generator(device=DEV).manual_seed(5)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    # first call: the larger problem; second: smaller, with fewer tiles per row
    for (M, H, V) in ((700, 1032, 100003), (37, 520, 4099)):
        h = torch.randn((M, H), generator=g, device=DEV).to(tdt)
        W = (torch.randn((V, H), generator=g, device=DEV) / H ** 0.5).to(tdt)
        Wp = bd.lmhead_pack(W) if code == 2 else None
        wptr = Wp.data.data_ptr() if code == 2 else W.data_ptr()
        print(f"\\n[noalloc] dtype {dt} M={M} H={H} V={V}", flush=True)
        za, tva, tia = _call_noalloc(h, wptr, code, V, M, H)
        zb, tvb, tib = _call_workspace(h, wptr, code, V, M, H)
        torch.cuda.synchronize()
        assert torch.equal(za, zb)
        assert torch.equal(tva, tvb)
        assert torch.equal(tia, tib)
        # the top-16 is the rows' 16 largest (value desc, id asc), on a few rows
        rows = [0, M // 2, M - 1]
        zc = za[rows].double().cpu().numpy()
        ref = np.lexsort((np.broadcast_to(np.arange(V), zc.shape), -zc), axis=1)[:, :16]
        np.testing.assert_array_equal(tia[rows].cpu().numpy(), ref)


def test_noalloc_refuses_more_than_its_scratch():
    h = torch.zeros((8, 16), dtype=torch.bfloat16, device=DEV)
    # 7062 rows of 151936 tokens need more tile maxima than the scratch holds;
    # refused on the host before any launch (no buffers of that size are made)
    st = bd.lib().dflash2_logits_topk_noalloc(
        ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(h.data_ptr() + 4096),
        ctypes.c_void_p(h.data_ptr() + 8192), ctypes.c_void_p(h.data_ptr() + 16384),
        ctypes.c_void_p(h.data_ptr() + 32768), 7062, 16, 151936, 16, 1, None)
    assert st == -5
