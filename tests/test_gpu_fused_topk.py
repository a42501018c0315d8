"""LM-head GEMM + top-16 without materialised logits (GPU).

dflash2_logits_topk with logits == NULL and bf16 operands runs the GEMM's
candidate form: a row of an N tile stores its 256 logits only while the row
has no lower bound theta on its 16th value yet (16 group maxima, all filled),
or when more than four of its values reach theta; otherwise it leaves just
those values and their columns.  The top-16 then reads stored tiles or
slots.  The same GEMM accumulators feed both forms, so the bar is bit for
bit: ids and value bits equal to the materialised path's, and equal to the
oracle's top-16 of the materialised logits (ties by lower id, NaN as -inf).
Cases: ragged M and V, fewer than 16 tiles (every tile stored), ties spread
over tiles, a tile with exactly four and one with five values at the top
(slots full, slots overflowing), rows of zeros, NaN and +inf, packed and
row-major W.
"""
import numpy as np
import pytest
import torch

import block_drafting_amd as bd
import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def _both(h, W):
    """(fused top_val, top_idx), (materialised top_val, top_idx), logits."""
    M, V = h.shape[0], (W.V if isinstance(W, bd.PackedWeight) else W.shape[0])
    z = torch.empty((M, V), dtype=torch.float32, device=DEV)
    v1, i1 = bd.logits_topk(h, W)            # candidate form (logits in the workspace)
    v0, i0 = bd.logits_topk(h, W, logits=z)  # logits materialised
    torch.cuda.synchronize()
    return (v1, i1), (v0, i0), z


def _assert_same(a, b):
    assert torch.equal(a[1], b[1])
    assert torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))


def _oracle_rows(fused, z, rows):
    zh = z[rows].cpu().numpy()
    wv, wi = O.topk16(zh)
    np.testing.assert_array_equal(fused[1][rows].cpu().numpy(), wi)
    np.testing.assert_array_equal(fused[0][rows].cpu().numpy().view(np.uint32),
                                  wv.view(np.uint32))


@pytest.mark.parametrize("M,H,V,packed", [
    (512, 1024, 151936, True),     # two M tiles, 594 N tiles, ragged last N tile
    (300, 136, 8000, False),       # ragged M and V, K tail
    (37, 64, 1000, True),          # 4 N tiles: no bound ever, every tile stored
    (513, 520, 4099, False),       # 17 N tiles: one beyond the 16 groups
    (1, 64, 70001, True),          # one row, odd V (scalar reads)
    (256, 192, 151936, True),      # the last round of N tiles as 128-row tiles
    (200, 136, 70001, False),      # the same with a K tail and row-major W
])
def test_fused_topk_random(M, H, V, packed):
    g = torch.Generator(device=DEV).manual_seed(M * 7 + V)
    h = _bf16(torch.randn((M, H), generator=g, device=DEV))
    W = _bf16(torch.randn((V, H), generator=g, device=DEV) / H ** 0.5)
    Wx = bd.lmhead_pack(W) if packed else W
    fused, mat, z = _both(h, Wx)
    _assert_same(fused, mat)
    rows = sorted(set([0, M - 1] + list(range(0, M, max(1, M // 12)))))
    _oracle_rows(fused, z, rows)


def test_fused_topk_ties_slots_and_specials():
    """Structured W columns, the same for every row with h[:, 0] = 1:
      - 40 tied values 64 at column 7 of tiles 300..339 (one per tile: one slot),
      - 4 values 66 in tile 450 (slots exactly full),
      - 5 values 66 in tile 460 (one more than the slots: the tile is stored),
      - 10 values 65 in tile 500.
    The top-16 is the nine 66s, then seven of the 65s (ids ascending).
    Extra rows: all zeros (every value ties at 0: every tile overflows),
    one NaN (every logit NaN), one huge h (+inf logits, ties at +inf)."""
    M, H, V = 300, 256, 151936
    g = torch.Generator(device=DEV).manual_seed(77)
    W = torch.randn((V, H), generator=g, device=DEV) / H ** 0.5
    W[:, 0] = 0.0
    a = lambda *x: torch.tensor(np.concatenate(x), device=DEV, dtype=torch.long)
    cols = {64.0: a(np.arange(300, 340) * 256 + 7), 66.0: a(450 * 256 + np.arange(4) * 9,
                                                           460 * 256 + 100 + np.arange(5)),
            65.0: a(500 * 256 + np.arange(10))}
    for val, c in cols.items():
        W[c] = 0.0                   # these logits are exactly h[:, 0] * val
        W[c, 0] = val
    h = torch.randn((M, H), generator=g, device=DEV)
    h[:, 0] = 1.0
    h[5] = 0.0                       # zero row
    h[6, 3] = float("nan")           # NaN row
    h[7] = 0.0
    h[7, 0] = 1e38                   # logits 1e38 * W[:, 0]: +inf at the tied columns
    h, W = _bf16(h), _bf16(W)
    for Wx in (W, bd.lmhead_pack(W)):
        fused, mat, z = _both(h, Wx)
        _assert_same(fused, mat)
        _oracle_rows(fused, z, [0, 1, 5, 6, 7, 150, 299])
        ids = fused[1][0].cpu().numpy()
        want = np.concatenate([450 * 256 + np.arange(4) * 9, 460 * 256 + 100 + np.arange(5),
                               500 * 256 + np.arange(7)])
        np.testing.assert_array_equal(np.sort(ids), np.sort(want))
        np.testing.assert_array_equal(fused[1][5].cpu().numpy(), np.arange(16))
        np.testing.assert_array_equal(fused[1][6].cpu().numpy(), np.arange(16))
        assert torch.isinf(fused[0][7]).all()


def test_fused_topk_repeated_calls_and_workspace_reuse():
    """The group maxima are reset by every call: a second call on other
    inputs with the same workspace (and a smaller M) gives its own result,
    not one bounded by the first call's maxima."""
    M, H, V = 512, 256, 151936
    g = torch.Generator(device=DEV).manual_seed(3)
    W = _bf16(torch.randn((V, H), generator=g, device=DEV) / H ** 0.5)
    h_big = _bf16(torch.randn((M, H), generator=g, device=DEV) * 4.0)   # large logits first
    h_small = _bf16(torch.randn((M, H), generator=g, device=DEV) * 0.25)
    need = bd.logits_topk_workspace(M, H, V, torch.bfloat16, False)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for h in (h_big, h_small, h_small[:200], h_big):
        v1, i1 = bd.logits_topk(h, W, workspace=ws)
        v0, i0 = bd.logits_topk(h, W, logits=torch.empty((h.shape[0], V), device=DEV))
        torch.cuda.synchronize()
        _assert_same((v1, i1), (v0, i0))


def test_fused_step_matches_materialised_step():
    """A whole bf16 step (conv, logits + top-16, scores, walk, verification)
    with and without materialised logits: identical outputs."""
    import workloads as WL
    from _devutil import convs_to_dev, to_dev

    w = WL.WORKLOADS[1]
    inp = WL.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if dt != torch.bfloat16:
        pytest.skip("the candidate form is the bf16 GEMM's")
    convs = convs_to_dev(inp["convs"], w.dtype)
    x, W = to_dev(inp["x"], w.dtype), to_dev(inp["W"], w.dtype)
    U, Vf = to_dev(inp["U"], w.dtype), to_dev(inp["Vf"], w.dtype)
    anc = to_dev(inp["anchor_tok"], "i32")
    tgt = torch.randint(0, w.V, (w.B, w.L + 1), device=DEV, dtype=torch.int32)
    outs = []
    for keep in (True, False):
        buf = bd.StepBuffers(w.B, w.L, w.H, w.V, dt, DEV, n_convs=w.n_convs, keep_logits=keep)
        bd.run_step(buf, x, convs, W, U, Vf, anc, tgt)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (buf.top_val, buf.top_idx, buf.path_tok,
                                         buf.accept_len, buf.next_tok)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_candidate_form_graph_replays():
    """logits + top-16 in the candidate form captured in a HIP graph (the
    group-maxima reset, GEMM and merge as three nodes): every replay, with
    eager calls on other inputs and synchronisations in between (which leave
    other group maxima in the workspace), gives the eager result; so does an
    eager call afterwards."""
    M, H, V = 512, 512, 151936
    g = torch.Generator(device=DEV).manual_seed(21)
    W = bd.lmhead_pack(_bf16(torch.randn((V, H), generator=g, device=DEV) / H ** 0.5))
    h = _bf16(torch.randn((M, H), generator=g, device=DEV))
    h_other = _bf16(torch.randn((M, H), generator=g, device=DEV) * 3.0)   # larger logits
    ws = torch.empty(bd.logits_topk_workspace(M, H, V, torch.bfloat16, False), dtype=torch.uint8,
                     device=DEV)
    tv = torch.empty((M, 16), dtype=torch.float32, device=DEV)
    ti = torch.empty((M, 16), dtype=torch.int32, device=DEV)

    def call(x):
        bd.logits_topk(x, W, top_val=tv, top_idx=ti, workspace=ws)

    call(h)
    torch.cuda.synchronize()
    want_v, want_i = tv.clone(), ti.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        call(h)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            call(h)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(4):
        call(h_other)                      # other inputs through the same workspace
        torch.cuda.synchronize()
        tv.zero_()
        ti.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ti, want_i)
        assert torch.equal(tv.view(torch.int32), want_v.view(torch.int32))
    call(h)
    torch.cuda.synchronize()
    assert torch.equal(ti, want_i)
