"""Stage-by-stage parity of the HIP library with the CPU oracle (GPU).

Every GPU stage is fed the oracle's own inputs for that stage and compared
element by element, at sizes the oracle finishes in seconds that still span
several tiles and ragged tails, plus the edge cases each stage has.

Bars (floating point from the arithmetic, integers exact):
  conv      |y - y_ora| <= ulp_storage(y_ora) + (H + 4) 2^-24 * bound, bound =
            the conv of absolute values; bf16 outputs bit-exact (the kernel
            evaluates in fp64 and rounds once)
  logits    |z - z_ora| <= 1e-3 max(|z_ora|, 1); bit-exact on dyadic inputs
  top-16    bit-exact ids and values (decided on the same fp32 logits)
  gate      |g - g_ora| <= (1/4) H 2^-24 sum_c |h_c w_c| + 4 2^-24 (fp32
            accumulation through the sigmoid's slope), mean error < 1e-6
  pairs     |S - S_ora| <= 1e-4 (gated and ungated); a gate of ones
            reproduces the ungated kernel bit for bit
  path      bit-exact slots, tokens and fp32 score for both walks (the
            oracle decides in fp32)
  sampling  slots equal wherever the uniform is more than 1e-5 from a bin
            edge of the oracle's fp64 inverse CDF (decided before the first
            closer one); |q - q_ora| <= 2e-6
  lse       |lse - lse_ora| <= (V/256 + 16) 2^-24 + 2^-23 |lse| (fp32 sums of
            V/256 terms per thread, then a tree)
  rejection accept lengths equal wherever every accept decision is clear by
            2e-4 relative; the verifier's token equal wherever u * mass is
            1e-5 of the mass away from every bin edge, else inside that
            window; emitted tokens follow the target (chi-square, GPU)
  verify    exact
  fused     scores, walk and verification in one launch: bit for bit the
            three separate calls; scores and the sampling walk in one launch:
            bit for bit the two separate calls
"""
import numpy as np
import pytest
import torch

import block_drafting_amd as bd
import oracle as O
import workloads as WL
from _devutil import bf16_ulp, to_dev, to_host_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits_or_f32(a, dt):
    return WL.to_bf16_bits(a) if dt == "bf16" else a.astype(np.float32)


# ------------------------------------------------------------------ conv
def _conv_case(B, L, H, dt, mode, groups, seed, anchor=True):
    g = np.random.default_rng(seed)
    x = _bits_or_f32(g.standard_normal((B, L, H)).astype(np.float32), dt)
    a = _bits_or_f32(g.standard_normal((B, H)).astype(np.float32), dt) if anchor else None
    k0 = (g.standard_normal(H) * 0.7).astype(np.float32)
    k1 = (g.standard_normal(H) * 0.7).astype(np.float32)
    P = (g.standard_normal((H, 2 * groups)) * np.sqrt(0.01 / H)).astype(np.float32) if mode else None
    return x, a, k0, k1, P


def _conv_check(x, a, k0, k1, P, groups, dt):
    B, L, H = x.shape
    xo = O.as_f64(x, dt)
    ao = None if a is None else O.as_f64(a, dt)
    Pd = None if P is None else P.astype(np.float64)
    want = O.round_to_dtype(O.twotap_conv(xo, ao, k0.astype(np.float64), k1.astype(np.float64),
                                          Pd, groups), dt)
    bound = O.twotap_conv(np.abs(xo), None if ao is None else np.abs(ao), np.abs(k0.astype(np.float64)),
                          np.abs(k1.astype(np.float64)), None if Pd is None else np.abs(Pd), groups)
    y = bd.twotap_conv(to_dev(x, dt), torch.from_numpy(k0).to(DEV), torch.from_numpy(k1).to(DEV),
                       None if a is None else to_dev(a, dt),
                       None if P is None else torch.from_numpy(P).to(DEV), groups)
    got = O.as_f64(to_host_bits(y), dt)
    tol = (bf16_ulp(want) if dt == "bf16" else 0.0) + (H + 4) * 2.0 ** -24 * bound
    err = np.abs(got - want)
    assert np.all(err <= tol), f"max err {err.max()} (tol {tol[err > tol][:4]})"
    return float(np.mean(got != want))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,H,mode,groups", [
    (3, 5, 64, 0, 1), (2, 1, 8, 0, 1), (4, 16, 5120, 0, 1), (5, 8, 136, 1, 1),
    (2, 16, 5120, 1, 1), (3, 4, 256, 1, 16), (2, 3, 5120, 1, 320), (1, 2, 64, 1, 64),
])
def test_conv_parity(dt, B, L, H, mode, groups):
    x, a, k0, k1, P = _conv_case(B, L, H, dt, mode, groups, seed=B * 100 + L * 10 + mode)
    frac = _conv_check(x, a, k0, k1, P, groups, dt)
    # the kernel evaluates in fp64 and rounds once (round-to-odd, then RNE):
    # only values within ~2^-52 relative of a rounding boundary can differ
    assert frac == 0.0 if dt == "bf16" else frac < 1e-4


# Shapes that reach each row-group layout of the conv kernels: several
# positions per workgroup (2, 4 or 8 with a projection; 2, or four
# pipelined single rows with static taps), with L not a multiple of the
# group so the last group is partial, no anchor, and rows wider than one
# workgroup's 1024 chunks (H = 10240, 20480: the one-row kernels).  bf16
# rows of H = 640 k <= 5120 take the ten-channels-per-thread kernel: 2 x 4,
# 2 x 2, 2 and 1 positions with a projection, 8 single rows (two groups
# ahead), 2 x 2, 2 and 1 static (the last from the 5120-channel shapes above).
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,H,mode,anchor", [
    (110, 5, 136, 0, True),      # 550 rows, static: 2 positions per workgroup, L odd
    (300, 7, 64, 0, True),       # 2100 rows, static: 4 pipelined rows, 7 = 4 + 3
    (300, 7, 64, 0, False),
    (70, 9, 520, 1, True),       # 630 rows, projection: 2 positions
    (130, 9, 64, 1, True),       # 1170 rows: 4 positions, 9 = 4 + 4 + 1
    (300, 11, 136, 1, False),    # 3300 rows: 8 positions, 11 = 8 + 3
    (2, 3, 10240, 1, True),      # wider than 8192 channels: one-row kernels
    (520, 2, 20480, 0, True),
    (230, 9, 640, 1, True),      # ten channels per thread: 2 x 4 positions, 9 = 8 + 1
    (130, 9, 1280, 1, False),    # 2 x 2, 9 = 4 + 4 + 1, no anchor
    (80, 7, 640, 1, True),       # 2 positions, 7 odd
    (300, 11, 640, 0, True),     # static, 8 single rows, 11 = 8 + 3
    (130, 9, 1280, 0, False),    # static, 2 x 2
    (110, 5, 2560, 0, True),     # static, 2 positions (4 waves)
])
def test_conv_row_groups_parity(dt, B, L, H, mode, anchor):
    x, a, k0, k1, P = _conv_case(B, L, H, dt, mode, 1, seed=B + L + H)
    if not anchor:
        a = None
    frac = _conv_check(x, a, k0, k1, P, 1, dt)
    assert frac == 0.0 if dt == "bf16" else frac < 1e-4


def test_conv_no_anchor_and_special_taps_bit_exact():
    B, L, H = 3, 6, 128
    x, a, _, _, _ = _conv_case(B, L, H, "bf16", 0, 1, seed=5)
    ones, zeros = np.ones(H, np.float32), np.zeros(H, np.float32)
    xd, ad = to_dev(x, "bf16"), to_dev(a, "bf16")
    y = to_host_bits(bd.twotap_conv(xd, torch.from_numpy(ones).to(DEV), torch.from_numpy(zeros).to(DEV), ad))
    np.testing.assert_array_equal(y, x)                                  # identity
    y = to_host_bits(bd.twotap_conv(xd, torch.from_numpy(zeros).to(DEV), torch.from_numpy(ones).to(DEV), ad))
    np.testing.assert_array_equal(y[:, 1:], x[:, :-1])                   # shift
    np.testing.assert_array_equal(y[:, 0], a)                            # anchor
    y = to_host_bits(bd.twotap_conv(xd, torch.from_numpy(zeros).to(DEV), torch.from_numpy(ones).to(DEV), None))
    assert not np.any(y[:, 0] & 0x7fff)                                  # zero anchor
    _conv_check(x, None, (np.arange(H) % 3).astype(np.float32), np.full(H, 0.5, np.float32), None, 1, "bf16")


@pytest.mark.parametrize("H,mode", [(640, 0), (640, 1), (5120, 1), (136, 0), (136, 1)])
def test_conv_bf16_rounds_once_near_midpoints(H, mode):
    """Outputs a hair above a bf16 midpoint: x alternates 2^-8 and 1 (every
    third channel negated, anchor +-1), k0 = 1, k1 = 1 + 2^-23, so every odd
    position is +-(1 + 2^-8 + 2^-31).  Its nearest fp32 is the midpoint
    1 + 2^-8 itself, whose nearest-even bf16 would be 1; the one correct
    rounding gives 1 + 2^-7.  Even positions are 1 + 2^-8 + 2^-23 (an fp32 value above the
    midpoint).  A zero projection (mode 1) runs the corrections' kernels
    with D = 0.  H = 640: ten channels per thread; H = 136: eight."""
    B, L = 3, 8
    mag = np.where(np.arange(L) % 2 == 0, 2.0 ** -8, 1.0)   # x_t
    sgn = np.where(np.arange(H) % 3 == 0, -1.0, 1.0)         # channels negated throughout
    xs = WL.to_bf16_bits((mag[None, :, None] * sgn[None, None, :] * np.ones((B, L, H))).astype(np.float32))
    a = WL.to_bf16_bits(np.broadcast_to(sgn, (B, H)).astype(np.float32))
    k0 = np.ones(H, np.float32)
    k1 = np.full(H, 1.0 + 2.0 ** -23, np.float32)
    P = np.zeros((H, 2), np.float32) if mode else None
    xo, ao = O.as_f64(xs, "bf16"), O.as_f64(a, "bf16")
    want = O.round_to_bf16(O.twotap_conv(xo, ao, k0.astype(np.float64), k1.astype(np.float64),
                                         None if P is None else P.astype(np.float64), 1))
    y = bd.twotap_conv(to_dev(xs, "bf16"), torch.from_numpy(k0).to(DEV), torch.from_numpy(k1).to(DEV),
                       to_dev(a, "bf16"), None if P is None else torch.from_numpy(P).to(DEV))
    assert np.all(np.abs(want) == 1.0 + 2.0 ** -7)  # the single rounding goes up
    got = to_host_bits(y)
    np.testing.assert_array_equal(O.as_f64(got, "bf16"), want)
    assert np.all((got & 0x7fff) == 0x3F81)
    np.testing.assert_array_equal(got[0, 1] >> 15, (sgn < 0).astype(got.dtype))


def conv_mm_tolerance(xo, ao, P, groups, want):
    """1 bf16 ulp for the final rounding, plus the fp32 accumulation of the
    corrections (|dD| <= H 2^-24 sum_c |x_c P_c|) carried through |x| and |prev|."""
    H = xo.shape[2]
    k = np.zeros(H)
    dD = O.twotap_conv(np.abs(xo), None if ao is None else np.abs(ao), k, k,
                       H * 2.0 ** -24 * np.abs(P), groups)
    return bf16_ulp(want) + dD


@pytest.mark.parametrize("B,L,H,G,anchor", [(1, 1, 64, 4, True), (3, 5, 136, 17, True),
                                            (2, 16, 5120, 320, True), (37, 1, 128, 8, False),
                                            (5, 7, 2560, 160, True), (1, 3, 256, 256, True),
                                            (4, 8, 1024, 1, True), (9, 8, 520, 65, False),
                                            (1100, 8, 1024, 64, True),    # > 256 tiles
                                            # split-K partials parked in y, then the
                                            # ten-channel mix: ragged M tile (915 rows),
                                            # 32-channel groups with a ragged N tile,
                                            # 256-thread rows
                                            (61, 15, 5120, 320, True), (267, 15, 1280, 40, False),
                                            (63, 31, 2560, 160, True)])
def test_conv_mm_parity(B, L, H, G, anchor):
    g = np.random.default_rng(B * 1000 + G)
    x = WL.to_bf16_bits(g.standard_normal((B, L, H)).astype(np.float32))
    a = WL.to_bf16_bits(g.standard_normal((B, H)).astype(np.float32)) if anchor else None
    k0 = (g.standard_normal(H) * 0.7).astype(np.float32)
    k1 = (g.standard_normal(H) * 0.7).astype(np.float32)
    pt = WL.to_bf16_bits((g.standard_normal((2 * G, H)) * np.sqrt(0.01 / H)).astype(np.float32))
    xo = O.as_f64(x, "bf16")
    ao = None if a is None else O.as_f64(a, "bf16")
    P = O.as_f64(pt, "bf16").T
    want = O.round_to_bf16(O.twotap_conv(xo, ao, k0.astype(np.float64), k1.astype(np.float64),
                                         P, G))
    y = bd.twotap_conv_mm(to_dev(x, "bf16"), torch.from_numpy(k0).to(DEV),
                          torch.from_numpy(k1).to(DEV), to_dev(pt, "bf16"),
                          None if a is None else to_dev(a, "bf16"))
    got = O.as_f64(to_host_bits(y), "bf16")
    err = np.abs(got - want)
    assert (err <= conv_mm_tolerance(xo, ao, P, G, want)).all(), err.max()
    assert (got != want).mean() <= 1e-3, (got != want).mean()


@pytest.mark.parametrize("B,L,H,G", [(3, 8, 640, 40), (61, 15, 5120, 320)])
def test_conv_mm_zero_map_is_the_static_conv_bit_exact(B, L, H, G):
    x, a, k0, k1, _ = _conv_case(B, L, H, "bf16", False, 1, seed=31)
    pt = np.zeros((2 * G, H), np.uint16)
    args = (to_dev(x, "bf16"), torch.from_numpy(k0).to(DEV), torch.from_numpy(k1).to(DEV))
    y_mm = bd.twotap_conv_mm(*args, to_dev(pt, "bf16"), to_dev(a, "bf16"))
    y_st = bd.twotap_conv(*args, to_dev(a, "bf16"))
    assert torch.equal(y_mm.view(torch.int16), y_st.view(torch.int16))


def test_conv_mm_split_graph_replays():
    """The split-K per-group conv (partials parked in y, then the mix)
    captured as a HIP graph: every replay, with eager calls on other inputs
    into the same output in between, gives the eager result."""
    B, L, H, G = 64, 16, 5120, 320          # 1024 rows: the split path
    g = torch.Generator(device=DEV).manual_seed(9)
    x = torch.randn((B, L, H), generator=g, device=DEV).to(torch.bfloat16)
    x2 = torch.randn((B, L, H), generator=g, device=DEV).to(torch.bfloat16)
    a = torch.randn((B, H), generator=g, device=DEV).to(torch.bfloat16)
    k0 = torch.randn(H, generator=g, device=DEV) * 0.7
    k1 = torch.randn(H, generator=g, device=DEV) * 0.7
    pt = (torch.randn((2 * G, H), generator=g, device=DEV) * (0.01 / H) ** 0.5).to(torch.bfloat16)
    y = torch.empty_like(x)
    want = bd.twotap_conv_mm(x, k0, k1, pt, a).clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        bd.twotap_conv_mm(x, k0, k1, pt, a, out=y)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            bd.twotap_conv_mm(x, k0, k1, pt, a, out=y)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(3):
        bd.twotap_conv_mm(x2, k0, k1, pt, a, out=y)   # other inputs, same output buffer
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16))


def test_conv_empty_batch_is_noop():
    x = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(64, device=DEV)
    assert bd.twotap_conv(x, k, k).shape == (0, 8, 64)


# ------------------------------------------------------------------ logits
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,H,V", [(1, 8, 16), (37, 64, 1000), (300, 136, 4099), (513, 520, 2048),
                                   (64, 5120, 300), (257, 2560, 777)])
def test_lmhead_parity(dt, M, H, V):
    g = np.random.default_rng(M + H + V)
    y = _bits_or_f32(g.standard_normal((M, H)).astype(np.float32), dt)
    W = _bits_or_f32((g.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32), dt)
    want = O.lm_logits(O.as_f64(y, dt), W, dt).astype(np.float64)
    got = bd.lmhead_logits(to_dev(y, dt), to_dev(W, dt)).cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    assert np.all(err <= 1e-3 * np.maximum(np.abs(want), 1.0)), err.max()


# One M tile of 129..256 rows whose last round of N tiles fills at most half
# the CUs runs that round as 128-row tiles in a second launch (594 tiles,
# 82 in the third round, at M = 256, V = 151936; one tail tile at
# V = 257 x 256 - 5; a K tail at H = 136).  Every output is the same
# sequence of MFMA accumulations whatever the tile's height, so the rows
# equal, bit for bit, those of a product of more than 256 rows (one
# launch of 256-row tiles); the tile maxima are those rows' maxima.
@pytest.mark.parametrize("M,H,V,packed", [(256, 192, 151936, True), (129, 64, 257 * 256 - 5, False),
                                          (200, 136, 70001, True)])
def test_lmhead_tail_launch_bit_exact(M, H, V, packed):
    g = torch.Generator(device=DEV).manual_seed(M + V)
    h_big = torch.randn((300, H), generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g, device=DEV) / H ** 0.5).to(torch.bfloat16)
    Wx = bd.lmhead_pack(W) if packed else W
    z_big = bd.lmhead_logits(h_big, Wx)                      # 300 rows: no tail launch
    z, tmax = bd.lmhead_logits_tilemax(h_big[:M].contiguous(), Wx)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int32), z_big[:M].view(torch.int32))
    nt = (V + 255) // 256
    zp = torch.full((M, nt * 256), -float("inf"), device=DEV)
    zp[:, :V] = z
    assert torch.equal(tmax, zp.view(M, nt, 256).amax(dim=2))
    rows = [0, 127, 128, M - 1]
    want = O.lm_logits(O.as_f64(to_host_bits(h_big[rows]), "bf16"), to_host_bits(W), "bf16")
    err = np.abs(z[rows].cpu().numpy().astype(np.float64) - want)
    assert np.all(err <= 1e-3 * np.maximum(np.abs(want), 1.0)), err.max()


def test_lmhead_one_hot_and_dyadic_bit_exact():
    M, H, V = 70, 256, 1100
    g = np.random.default_rng(3)
    W = WL.to_bf16_bits((g.standard_normal((V, H)) / 16).astype(np.float32))
    y = np.zeros((M, H), np.float32)
    cols = g.integers(0, H, M)
    y[np.arange(M), cols] = 1.0
    got = bd.lmhead_logits(to_dev(WL.to_bf16_bits(y), "bf16"), to_dev(W, "bf16")).cpu().numpy()
    np.testing.assert_array_equal(got, O.as_f64(W, "bf16")[:, cols].T.astype(np.float32))
    # small integers and 1/64 multiples: every partial sum is exact in fp32
    yi = np.clip(np.round(g.standard_normal((M, H)) * 3), -16, 16).astype(np.float32)
    Wi = (np.clip(np.round(g.standard_normal((V, H)) * 2), -8, 8) / 64).astype(np.float32)
    got = bd.lmhead_logits(to_dev(WL.to_bf16_bits(yi), "bf16"), to_dev(WL.to_bf16_bits(Wi), "bf16"))
    want = O.lm_logits(yi.astype(np.float64), WL.to_bf16_bits(Wi), "bf16")
    np.testing.assert_array_equal(got.cpu().numpy(), want)


def _pack_ref(W):
    """The packed LM-head layout written out with torch ops: W [V, H] zero-padded
    to whole 256-row x 64-column blocks, blocks ordered (row tile, column
    slice), each block row-major."""
    V, H = W.shape
    Vp, Hp = -(-V // 256) * 256, -(-H // 64) * 64
    pad = torch.zeros((Vp, Hp), dtype=W.dtype, device=W.device)
    pad[:V, :H] = W
    return pad.view(Vp // 256, 256, Hp // 64, 64).permute(0, 2, 1, 3).contiguous().view(-1)


@pytest.mark.parametrize("V,H", [(1, 8), (16, 64), (300, 136), (4099, 200), (1000, 5120)])
def test_lmhead_pack_layout(V, H):
    g = torch.Generator(device=DEV).manual_seed(V * 31 + H)
    W = torch.randn((V, H), generator=g, device=DEV).to(torch.bfloat16)
    n = bd.lib().dflash2_lmhead_pack_bytes(V, H)
    assert n == 2 * _pack_ref(W).numel()
    Wp = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)   # padding must be overwritten
    assert bd.lib().dflash2_lmhead_pack(W.data_ptr(), Wp.data_ptr(), V, H,
                                        bd._stream(W.device)) == 0
    assert torch.equal(Wp.view(torch.int16), _pack_ref(W).view(torch.int16))


@pytest.mark.parametrize("M,H,V", [(1, 8, 16), (37, 64, 1000), (300, 136, 4099), (513, 520, 2048),
                                   (257, 2560, 777)])
def test_packed_lmhead_matches_row_major_and_oracle(M, H, V):
    """Packing W changes only where the GEMM reads it from: logits, tile maxima
    and top-16 are bit for bit those of the row-major W, and the logits meet the
    oracle's bound."""
    g = np.random.default_rng(M * 3 + H + V)
    y = _bits_or_f32(g.standard_normal((M, H)).astype(np.float32), "bf16")
    Wb = _bits_or_f32((g.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32), "bf16")
    h, W = to_dev(y, "bf16"), to_dev(Wb, "bf16")
    Wp = bd.lmhead_pack(W)
    z1, t1 = bd.lmhead_logits_tilemax(h, W)
    z2, t2 = bd.lmhead_logits_tilemax(h, Wp)
    assert torch.equal(z1.view(torch.int32), z2.view(torch.int32))
    assert torch.equal(t1.view(torch.int32), t2.view(torch.int32))
    assert torch.equal(bd.lmhead_logits(h, Wp).view(torch.int32), z1.view(torch.int32))
    v1, i1 = bd.logits_topk(h, W)
    v2, i2 = bd.logits_topk(h, Wp)
    assert torch.equal(i1, i2) and torch.equal(v1.view(torch.int32), v2.view(torch.int32))
    want = O.lm_logits(O.as_f64(y, "bf16"), Wb, "bf16").astype(np.float64)
    got = z2.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-3 * np.maximum(np.abs(want), 1.0))


def test_packed_lmhead_full_vocabulary():
    """512 rows x hidden 5120 x vocabulary 151936 (a ragged last row tile):
    packed and row-major W give the same logits and tile maxima, bit for bit."""
    M, H, V = 512, 5120, 151936
    g = torch.Generator(device=DEV).manual_seed(5)
    h = torch.randn((M, H), generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g, device=DEV) / H ** 0.5).to(torch.bfloat16)
    Wp = bd.lmhead_pack(W)
    z1, t1 = bd.lmhead_logits_tilemax(h, W)
    z2, t2 = bd.lmhead_logits_tilemax(h, Wp)
    assert torch.equal(z1.view(torch.int32), z2.view(torch.int32))
    assert torch.equal(t1.view(torch.int32), t2.view(torch.int32))


def test_packed_weight_checks_its_partner():
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device=DEV)
    Wp = bd.lmhead_pack(W)
    with pytest.raises(ValueError):
        bd.lmhead_logits(torch.zeros((4, 72), dtype=torch.bfloat16, device=DEV), Wp)   # H differs
    with pytest.raises(ValueError):
        bd.lmhead_logits(torch.zeros((4, 64), dtype=torch.float32, device=DEV), Wp)    # fp32 h
    with pytest.raises(TypeError):
        bd.lmhead_pack(W.float())


# ------------------------------------------------------------------ top-16
def _topk_check(z):
    tv, ti = bd.topk16(torch.from_numpy(z).to(DEV))
    wv, wi = O.topk16(z)
    np.testing.assert_array_equal(ti.cpu().numpy(), wi)
    np.testing.assert_array_equal(tv.cpu().numpy().view(np.uint32), wv.view(np.uint32))


@pytest.mark.parametrize("M,V", [(1, 16), (3, 17), (7, 4099), (33, 151936), (512, 4096), (5, 100003)])
def test_topk_parity_random(M, V):
    g = np.random.default_rng(M * 7 + V)
    _topk_check(g.standard_normal((M, V)).astype(np.float32))


def test_topk_ties_zeros_nan_inf_and_adversarial_order():
    V = 20000
    g = np.random.default_rng(11)
    rows = [
        np.zeros(V),                                   # all tied: lowest 16 ids
        np.where(np.arange(V) % 2 == 0, 0.0, -0.0),    # +0 / -0 mix
        np.arange(V, dtype=np.float64),                # ascending: every value inserts
        -np.arange(V, dtype=np.float64),               # descending
        np.round(g.standard_normal(V) * 64) / 64,      # 1/64 grid: many ties
        np.full(V, -np.inf),
        np.where(g.random(V) < 0.5, np.nan, g.standard_normal(V)),
        np.concatenate([[np.inf, np.nan, -np.inf], g.standard_normal(V - 3)]),
    ]
    z = np.stack(rows).astype(np.float32)
    z[4, 1000:1040] = z[4].max()                       # 40-way tie at the top
    _topk_check(z)
    nan_rows = np.full((2, 64), np.nan, np.float32)    # everything ranks as -inf
    _topk_check(nan_rows)


def _tile_max(z):
    """Row maxima of 256-column tiles, NaN ignored (a tile of only NaN gives
    -inf), test-local numpy."""
    M, V = z.shape
    nt = (V + 255) // 256
    pad = np.full((M, nt * 256), -np.inf, np.float32)
    pad[:, :V] = np.where(np.isnan(z), -np.inf, z)
    return pad.reshape(M, nt, 256).max(axis=2).astype(np.float32)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,H,V", [(1, 8, 16), (37, 64, 1000), (300, 136, 4099), (64, 256, 151936)])
def test_lmhead_tilemax_is_the_max_of_the_stored_logits(dt, M, H, V):
    g = np.random.default_rng(M + V)
    h = _bits_or_f32(g.standard_normal((M, H)).astype(np.float32), dt)
    W = _bits_or_f32((g.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32), dt)
    z, tm = bd.lmhead_logits_tilemax(to_dev(h, dt), to_dev(W, dt))
    z = z.cpu().numpy()
    np.testing.assert_array_equal(tm.cpu().numpy(), _tile_max(z))
    want = O.lm_logits(O.as_f64(h, dt), W, dt).astype(np.float64)
    assert np.all(np.abs(z - want) <= 1e-3 * np.maximum(np.abs(want), 1.0))


def _topk_tilemax_check(z):
    tv, ti = bd.topk16_tilemax(torch.from_numpy(z).to(DEV), torch.from_numpy(_tile_max(z)).to(DEV))
    wv, wi = O.topk16(z)
    np.testing.assert_array_equal(ti.cpu().numpy(), wi)
    np.testing.assert_array_equal(tv.cpu().numpy().view(np.uint32), wv.view(np.uint32))


@pytest.mark.parametrize("M,V", [(1, 16), (3, 17), (7, 4099), (33, 151936), (512, 4096),
                                 (5, 100003), (4, 255), (2, 257)])
def test_topk_tilemax_parity_random(M, V):
    g = np.random.default_rng(M * V + 3)
    _topk_tilemax_check((g.standard_normal((M, V)) * 3).astype(np.float32))


def test_topk_tilemax_ties_zeros_nan_inf():
    g = np.random.default_rng(11)
    z = (np.round(g.standard_normal((6, 5000)) * 2) / 4).astype(np.float32)   # many ties
    z[0] = 1.0                                       # every tile ties at the bound
    z[1, :] = -0.0
    z[1, 700:900] = 0.0                              # +0 and -0 tie
    z[2, ::7] = np.nan
    z[3, 1000:1300] = np.nan                         # a whole tile of NaN
    z[4, 4990] = np.inf
    z[4, 3] = -np.inf
    z[5, :] = -np.inf
    z[5, 4242] = -1.0
    _topk_tilemax_check(z)
    # rows whose every tile maximum is -inf: the bound sits at -inf, so NaN
    # (ranked as -inf) must pass the filter too
    z = np.full((3, 1000), np.nan, np.float32)
    z[1, :] = -np.inf
    z[2, ::2] = -np.inf                              # NaN and -inf mixed
    _topk_tilemax_check(z)
    # top values spread over 16 different tiles vs packed in one
    z = np.zeros((2, 151936), np.float32)
    z[0, np.arange(16) * 9000] = 5.0
    z[1, 77000:77016] = 5.0
    _topk_tilemax_check(z)


def test_topk_tilemax_more_than_1024_tiles():
    """V > 262144: the tile maxima take more than one pass (1024 per pass) and
    the second bound is skipped; values planted across passes."""
    g = np.random.default_rng(9)
    V = 300007                                          # 1172 tiles, ragged last tile
    z = g.standard_normal((3, V)).astype(np.float32)
    z[0, [5, 262143, 262144, 299999, 300006]] = 7.0     # around the pass boundary and the tail
    z[1, 262144:262144 + 40] = 6.5                      # 40 ties inside the second pass
    z[2, ::1000] = np.nan
    _topk_tilemax_check(z)


def test_logits_topk_more_than_1024_tiles():
    g = np.random.default_rng(10)
    M, H, V = 5, 64, 266240                             # 1040 tiles
    h = g.standard_normal((M, H)).astype(np.float32)
    W = (g.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32)
    z, tm = bd.lmhead_logits_tilemax(to_dev(_bits_or_f32(h, "bf16"), "bf16"),
                                     to_dev(_bits_or_f32(W, "bf16"), "bf16"))
    zh = z.cpu().numpy()
    np.testing.assert_array_equal(tm.cpu().numpy(), _tile_max(zh))
    tv, ti = bd.topk16_tilemax(z, tm)
    wv, wi = O.topk16(zh)
    np.testing.assert_array_equal(ti.cpu().numpy(), wi)
    np.testing.assert_array_equal(tv.cpu().numpy().view(np.uint32), wv.view(np.uint32))


def test_topk_tilemax_bound_refinement():
    """The second bound (the 16th largest of the tile maxima that reach the
    lane-max bound) around its edges: ties at it, a graded run it cuts to 16
    tiles, and more than 64 tiles at the first bound (refinement skipped)."""
    g = np.random.default_rng(5)
    z = (g.standard_normal((4, 151936)) * 0.5).astype(np.float32)
    t = np.arange(594)
    z[0, t[:30] * 256 + 7] = 5.0                        # 30 tiles tie at the 16th maximum
    z[1, t[:40] * 256 + t[:40] % 256] = (5.0 - 0.01 * t[:40]).astype(np.float32)
    z[2, t[::8][:70] * 256 + 100] = 5.0                 # 70 tied tiles: > 64 reach the first bound
    z[3, t[:17] * 256 + 255] = 5.0                      # 17 tiles, last column of each
    z[3, 16 * 256 + 254] = 5.0                          # a second 5.0 inside the 17th tile
    _topk_tilemax_check(z)


# ------------------------------------------------------------------ pair scores
def _pair_case(B, L, V, r, dt, seed, anchor=True):
    g = np.random.default_rng(seed)
    tv = g.standard_normal((B, L, 16)).astype(np.float32)
    ti = g.integers(0, V, (B, L, 16)).astype(np.int32)
    U = _bits_or_f32((g.standard_normal((V, r)) * np.sqrt(0.1)).astype(np.float32), dt)
    Vf = _bits_or_f32((g.standard_normal((V, r)) * np.sqrt(0.1)).astype(np.float32), dt)
    at = g.integers(0, V, B).astype(np.int32) if anchor else None
    return tv, ti, at, U, Vf


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,V,r", [(1, 1, 64, 1), (3, 2, 500, 7), (4, 8, 4096, 32),
                                     (5, 16, 151936, 64), (2, 16, 2000, 128), (2, 5, 300, 256),
                                     (1, 64, 1000, 16)])
def test_pair_parity(dt, B, L, V, r):
    tv, ti, at, U, Vf = _pair_case(B, L, V, r, dt, seed=B + L + r)
    wS0, wS = O.pair_scores(tv, ti, at, U, Vf, dt)
    S0, S = bd.pair_score(torch.from_numpy(tv).to(DEV), torch.from_numpy(ti).to(DEV),
                          torch.from_numpy(at).to(DEV), to_dev(U, dt), to_dev(Vf, dt))
    assert np.abs(S0.cpu().numpy() - wS0).max() <= 1e-4
    if L > 1:
        assert np.abs(S.cpu().numpy() - wS).max() <= 1e-4


def test_pair_without_anchor_and_bad_ids_give_nan():
    tv, ti, _, U, Vf = _pair_case(2, 3, 100, 8, "f32", seed=1, anchor=False)
    wS0, wS = O.pair_scores(tv, ti, None, U, Vf, "f32")
    S0, S = bd.pair_score(torch.from_numpy(tv).to(DEV), torch.from_numpy(ti).to(DEV), None,
                          torch.from_numpy(U).to(DEV), torch.from_numpy(Vf).to(DEV))
    np.testing.assert_array_equal(S0.cpu().numpy(), wS0)
    ti_bad = ti.copy()
    ti_bad[1, 1, 5] = 100          # == V: out of range, at position 1
    ti_bad[0, 0, 3] = -7           # negative, at position 0
    S0, S = bd.pair_score(torch.from_numpy(tv).to(DEV), torch.from_numpy(ti_bad).to(DEV), None,
                          torch.from_numpy(U).to(DEV), torch.from_numpy(Vf).to(DEV))
    S, S0 = S.cpu().numpy(), S0.cpu().numpy()
    assert np.isnan(S[1, 0, :, 5]).all() and np.isnan(S[1, 0]).sum() == 16   # as current token
    assert np.isnan(S[1, 1, 5, :]).all() and np.isnan(S[1, 1]).sum() == 16   # as previous token
    assert np.isnan(S0[0, 3]) and np.isnan(S0).sum() == 1
    assert np.isnan(S[0, 0, 3, :]).all() and np.isnan(S[0, 0]).sum() == 16
    ok = ~np.isnan(S)
    np.testing.assert_allclose(S[ok], wS[ok], atol=1e-4, rtol=0)


# ------------------------------------------------------------------ context gate
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,H,r", [(1, 8, 1), (37, 136, 7), (300, 520, 64), (64, 2568, 33),
                                   (513, 5120, 256), (4096, 256, 40),
                                   (4100, 64, 100)])        # > 256 tiles: four-wave kernel
def test_context_gate_parity(dt, M, H, r):
    g = np.random.default_rng(M + H + r)
    h = _bits_or_f32(g.standard_normal((M, H)).astype(np.float32), dt)
    Wg = _bits_or_f32((g.standard_normal((r, H)) / np.sqrt(H)).astype(np.float32), dt)
    hd, Wd = O.as_f64(h, dt), O.as_f64(Wg, dt)
    want = O.context_gate(hd, Wg, dt).astype(np.float64)
    got = bd.context_gate(to_dev(h, dt), to_dev(Wg, dt)).cpu().numpy()
    err = np.abs(got - want)
    tol = 0.25 * H * 2.0 ** -24 * (np.abs(hd) @ np.abs(Wd).T) + 4 * 2.0 ** -24
    assert (err <= tol).all(), err.max()
    assert err.mean() < 1e-6, err.mean()


def test_context_gate_saturates_and_empty():
    h = np.zeros((3, 16), np.float32)
    h[0, 0], h[1, 0] = 200.0, -200.0                 # sigmoid saturates to exactly 1 and 0
    Wg = np.zeros((2, 16), np.float32)
    Wg[0, 0] = 1.0
    got = bd.context_gate(torch.from_numpy(h).to(DEV), torch.from_numpy(Wg).to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, [[1.0, 0.5], [0.0, 0.5], [0.5, 0.5]])
    out = bd.context_gate(torch.empty((0, 16), device=DEV), torch.from_numpy(Wg).to(DEV))
    assert out.shape == (0, 2)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,V,r", [(1, 1, 64, 1), (3, 2, 500, 7), (4, 8, 4096, 32),
                                     (5, 16, 151936, 64), (2, 5, 300, 256), (64, 8, 151936, 256)])
def test_gated_pair_parity(dt, B, L, V, r):
    tv, ti, at, U, Vf = _pair_case(B, L, V, r, dt, seed=B + L + r + 1)
    gate = np.random.default_rng(r).random((B, L, r)).astype(np.float32)
    wS0, wS = O.pair_scores(tv, ti, at, U, Vf, dt, gate)
    args = (torch.from_numpy(tv).to(DEV), torch.from_numpy(ti).to(DEV),
            torch.from_numpy(at).to(DEV), to_dev(U, dt), to_dev(Vf, dt))
    S0, S = bd.pair_score(*args, gate=torch.from_numpy(gate).to(DEV))
    assert np.abs(S0.cpu().numpy() - wS0).max() <= 1e-4
    if L > 1:
        assert np.abs(S.cpu().numpy() - wS).max() <= 1e-4
    # a gate of ones is the ungated kernel, bit for bit
    G0, G = bd.pair_score(*args, gate=torch.ones((B, L, r), device=DEV))
    P0, P = bd.pair_score(*args)
    assert torch.equal(G0, P0) and torch.equal(G, P)


# ------------------------------------------------------------------ path walk
@pytest.mark.parametrize("B,L,dyadic", [(1, 1, False), (7, 2, True), (64, 8, False), (64, 8, True),
                                        (33, 16, True), (5, 64, False), (300, 3, True)])
def test_path_select_bit_exact(B, L, dyadic):
    g = np.random.default_rng(B * L)
    if dyadic:
        S0 = (np.round(g.standard_normal((B, 16)) * 2) / 4).astype(np.float32)
        S = (np.round(g.standard_normal((B, L - 1, 16, 16)) * 2) / 4).astype(np.float32)
    else:
        S0 = g.standard_normal((B, 16)).astype(np.float32) * 4
        S = g.standard_normal((B, L - 1, 16, 16)).astype(np.float32)
    ti = g.integers(0, 151936, (B, L, 16)).astype(np.int32)
    ws, wt, wsc = O.path_select(S0, S, ti)
    slot, tok, score = bd.path_select(torch.from_numpy(S0).to(DEV),
                                      torch.from_numpy(S).to(DEV) if L > 1 else None,
                                      torch.from_numpy(ti).to(DEV))
    np.testing.assert_array_equal(slot.cpu().numpy(), ws)
    np.testing.assert_array_equal(tok.cpu().numpy(), wt)
    np.testing.assert_array_equal(score.cpu().numpy().view(np.uint32), wsc.view(np.uint32))


@pytest.mark.parametrize("B,L,dyadic", [(1, 1, False), (7, 2, True), (64, 8, False), (64, 8, True),
                                        (33, 16, True), (5, 64, False), (5, 64, True), (300, 3, True)])
def test_path_greedy_bit_exact(B, L, dyadic):
    g = np.random.default_rng(B * L + 1)
    if dyadic:
        S0 = (np.round(g.standard_normal((B, 16)) * 2) / 4).astype(np.float32)
        S = (np.round(g.standard_normal((B, L - 1, 16, 16)) * 2) / 4).astype(np.float32)
    else:
        S0 = g.standard_normal((B, 16)).astype(np.float32) * 4
        S = g.standard_normal((B, L - 1, 16, 16)).astype(np.float32)
    ti = g.integers(0, 151936, (B, L, 16)).astype(np.int32)
    ws, wt, wsc = O.path_select_greedy(S0, S, ti)
    slot, tok, score = bd.path_select(torch.from_numpy(S0).to(DEV),
                                      torch.from_numpy(S).to(DEV) if L > 1 else None,
                                      torch.from_numpy(ti).to(DEV), mode="greedy")
    np.testing.assert_array_equal(slot.cpu().numpy(), ws)
    np.testing.assert_array_equal(tok.cpu().numpy(), wt)
    np.testing.assert_array_equal(score.cpu().numpy().view(np.uint32), wsc.view(np.uint32))


def test_path_greedy_trap_and_ties():
    # the pins' hand case: greedy [0, 3, 7] (score 5), max-plus [1, 2, 5] (score 9)
    S0 = np.zeros((1, 16), np.float32)
    S0[0, 0], S0[0, 1] = 5.0, 4.0
    S = np.full((1, 2, 16, 16), -10.0, np.float32)
    S[0, 0, 0, 3], S[0, 0, 1, 2], S[0, 0, 3, 0] = -1.0, 3.0, 8.0
    S[0, 1] = 0.0
    S[0, 1, 2, 5], S[0, 1, 3, 7] = 2.0, 1.0
    d0, d = torch.from_numpy(S0).to(DEV), torch.from_numpy(S).to(DEV)
    slot, _, score = bd.path_select(d0, d, None, mode="greedy")
    assert slot.cpu().tolist() == [[0, 3, 7]] and score.cpu().tolist() == [5.0]
    slot, _, score = bd.path_select(d0, d, None, mode="viterbi")
    assert slot.cpu().tolist() == [[1, 2, 5]] and score.cpu().tolist() == [9.0]
    z0 = torch.zeros((3, 16), device=DEV)
    z = torch.zeros((3, 4, 16, 16), device=DEV)
    slot, _, score = bd.path_select(z0, z, None, mode="greedy")
    assert (slot.cpu().numpy() == 0).all() and (score.cpu().numpy() == 0).all()


def test_path_select_all_tied_takes_slot_zero():
    B, L = 4, 8
    S0 = np.zeros((B, 16), np.float32)
    S = np.zeros((B, L - 1, 16, 16), np.float32)
    slot, _, score = bd.path_select(torch.from_numpy(S0).to(DEV), torch.from_numpy(S).to(DEV), None)
    assert (slot.cpu().numpy() == 0).all() and (score.cpu().numpy() == 0).all()


# ------------------------------------------------------------------ sampling + rejection
SAMPLE_TOL = 1e-5


def decided_prefix(margin, tol):
    """Per block, the number of leading positions whose decision is clear."""
    bad = margin <= tol
    return np.where(bad.any(axis=1), bad.argmax(axis=1), margin.shape[1])


@pytest.mark.parametrize("B,L,T", [(1, 1, 1.0), (7, 2, 0.7), (64, 8, 1.0), (33, 16, 2.0),
                                   (5, 64, 1.0), (300, 3, 0.3)])
def test_path_sample_parity(B, L, T):
    g = np.random.default_rng(B * L + 7)
    S0 = (g.standard_normal((B, 16)) * 2).astype(np.float32)
    S = g.standard_normal((B, L - 1, 16, 16)).astype(np.float32)
    ti = g.integers(0, 151936, (B, L, 16)).astype(np.int32)
    u = g.random((B, L)).astype(np.float32)
    ws, wt, wq = O.sample_path(S0, S, ti, T, u)
    slot, tok, q = bd.path_sample(torch.from_numpy(S0).to(DEV),
                                  torch.from_numpy(S).to(DEV) if L > 1 else None,
                                  torch.from_numpy(ti).to(DEV), torch.from_numpy(u).to(DEV), T)
    slot, tok, q = slot.cpu().numpy(), tok.cpu().numpy(), q.cpu().numpy()
    k = decided_prefix(O.sample_margin(wq, u), SAMPLE_TOL)
    assert (k == L).mean() >= 0.95
    for b in range(B):
        assert slot[b, :k[b]].tolist() == ws[b, :k[b]].tolist(), b
        assert tok[b, :k[b]].tolist() == wt[b, :k[b]].tolist(), b
        upto = min(k[b] + 1, L)                 # q of the first undecided position still matches
        assert np.abs(q[b, :upto] - wq[b, :upto]).max() <= 2e-6, b
    np.testing.assert_allclose(q.sum(axis=2), 1.0, atol=2e-6)


def joint_sample_tol(S0, S, T):
    """Bound on |q_gpu - q_oracle| for whole-path draws.  The backward
    message beta_t is a chain of L - 1 - t fp32 log-sum-exps over values of
    magnitude at most max|S| / T + beta_{t+1}; each adds a few roundings of
    2^-24 relative, so |d beta| <= 4 2^-24 L (max|S| / T + log 16) and
    |dq| <= 2 |da| q.  Twice that again for the softmax's own roundings; an
    fp32 emulation of the kernel stays 10x or more inside it."""
    L = (S.shape[1] if S is not None and S.ndim == 4 else 0) + 1
    smax = max(float(np.abs(S0).max()), float(np.abs(S).max()) if L > 1 else 0.0)
    return 8 * 2.0 ** -24 * L * (smax / T + 4.0)


@pytest.mark.parametrize("B,L,T", [(1, 1, 1.0), (7, 2, 0.7), (64, 8, 1.0), (33, 16, 2.0),
                                   (5, 64, 1.0), (300, 3, 0.3), (64, 16, 0.5)])
def test_path_sample_whole_path_parity(B, L, T):
    """Whole-path draws (backward messages, forward draws) against the
    oracle's fp64 sampler: slots equal wherever the uniform is clear of every
    bin edge by the fp32 messages' error bound, proposals within it."""
    g = np.random.default_rng(B * L + 11)
    S0 = (g.standard_normal((B, 16)) * 2).astype(np.float32)
    S = (g.standard_normal((B, L - 1, 16, 16)) * 1.5).astype(np.float32)
    ti = g.integers(0, 151936, (B, L, 16)).astype(np.int32)
    u = g.random((B, L)).astype(np.float32)
    ws, wt, wq = O.sample_path_joint(S0, S, ti, T, u)
    slot, tok, q = bd.path_sample(torch.from_numpy(S0).to(DEV),
                                  torch.from_numpy(S).to(DEV) if L > 1 else None,
                                  torch.from_numpy(ti).to(DEV), torch.from_numpy(u).to(DEV), T,
                                  mode="path")
    slot, tok, q = slot.cpu().numpy(), tok.cpu().numpy(), q.cpu().numpy()
    tol = joint_sample_tol(S0, S, T)
    k = decided_prefix(O.sample_margin(wq, u), tol)
    # a position is undecided with probability ~32 tol (~1% at L = 64), so
    # long blocks are compared up to their first undecided position
    assert k.mean() >= min(0.9 * L, 16), k.mean()
    for b in range(B):
        assert slot[b, :k[b]].tolist() == ws[b, :k[b]].tolist(), b
        assert tok[b, :k[b]].tolist() == wt[b, :k[b]].tolist(), b
        upto = min(k[b] + 1, L)
        assert np.abs(q[b, :upto] - wq[b, :upto]).max() <= tol, b
    np.testing.assert_allclose(q.sum(axis=2), 1.0, atol=2e-6)
    if L == 1:                                  # one position: the chain sampler's draw
        c = bd.path_sample(torch.from_numpy(S0).to(DEV), None, torch.from_numpy(ti).to(DEV),
                           torch.from_numpy(u).to(DEV), T)
        np.testing.assert_array_equal(c[0].cpu().numpy(), slot)


def test_whole_path_draws_follow_the_path_distribution_on_gpu():
    """GPU draws of whole paths (L = 3, one score set, 200,000 blocks) against
    the enumerated distribution exp(score / T) over all 4096 paths."""
    from scipy.stats import chisquare
    import itertools

    g = np.random.default_rng(44)
    N, L, T = 200000, 3, 1.0
    S0 = (g.standard_normal(16) * 1.5).astype(np.float32)
    S = (g.standard_normal((L - 1, 16, 16)) * 1.5).astype(np.float32)
    paths = np.array(list(itertools.product(range(16), repeat=L)))
    sc = S0[paths[:, 0]].astype(np.float64)
    for t in range(1, L):
        sc = sc + S[t - 1, paths[:, t - 1], paths[:, t]]
    probs = np.exp((sc - sc.max()) / T)
    probs /= probs.sum()
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    slot, _, _ = bd.path_sample(d(np.broadcast_to(S0, (N, 16))),
                                d(np.broadcast_to(S, (N, L - 1, 16, 16))), None,
                                d(g.random((N, L)).astype(np.float32)), T, mode="path")
    idx = (slot.cpu().numpy().astype(np.int64) * np.array([256, 16, 1])).sum(axis=1)
    counts = np.bincount(idx, minlength=4096)
    exp = probs * N
    big = exp >= 5
    obs = np.concatenate([counts[big], [counts[~big].sum()]])
    ex = np.concatenate([exp[big], [exp[~big].sum()]])
    assert chisquare(obs, ex).pvalue > 1e-4


@pytest.mark.parametrize("R,V,T,neg", [(1, 16, 1.0, False), (7, 1001, 0.7, False),
                                       (64, 151936, 1.0, False), (3, 4096, 2.0, True)])
def test_target_lse_parity(R, V, T, neg):
    g = np.random.default_rng(R + V)
    z = (g.standard_normal((R, V)) * 3).astype(np.float32)
    if neg:
        z[:, ::3] = -np.inf                     # tokens with no mass
    want = O.target_lse(z, T)
    got = bd.target_lse(torch.from_numpy(z).to(DEV), T).cpu().numpy()
    tol = (V / 256 + 16) * 2.0 ** -24 + 2.0 ** -23 * np.abs(want)
    assert (np.abs(got - want) <= tol).all(), np.abs(got - want).max()


def _spec_case(g, B, L, V, T):
    """Candidates, a sampled path with its proposals (fp32), target logits
    where some drafted tokens are likely under the target, and uniforms."""
    ti = np.stack([np.stack([g.choice(V, 16, replace=False) for _ in range(L)])
                   for _ in range(B)]).astype(np.int32)
    S0 = g.standard_normal((B, 16)).astype(np.float32)
    S = g.standard_normal((B, L - 1, 16, 16)).astype(np.float32)
    u = g.random((B, L)).astype(np.float32)
    slot, tok, q = O.sample_path(S0, S, ti, T, u)
    q = q.astype(np.float32)
    z = g.standard_normal((B, L + 1, V)).astype(np.float32)
    bump = g.random((B, L)) < 0.6
    for b in range(B):
        for t in range(L):
            if bump[b, t]:
                z[b, t, tok[b, t]] += np.float32(np.log(V) + g.standard_normal())
    return ti, slot, tok, q, z, g.random((B, L)).astype(np.float32), g.random(B).astype(np.float32)


# Window for the verifier's token: the GPU's fp32 inverse CDF (4-term lane
# sums and a 6-level tree per 256-token tile, a chunked scan over the tiles,
# a 6-level scan inside the chosen tile, 2-ulp exponentials) stays within
# about 40 2^-24 of the mass; 1e-5 of the mass is 4x that.  At V = 151936
# one token's bin (~7e-6 of the mass) is narrower than the window, so there
# the token is checked against the window only.
RES_WIN = 1e-5


def check_rejection(ti, slot, tok, q, z, T, ua, ur, acc, nxt):
    """Compare GPU (acc, nxt) with the oracle under the margin rules; returns
    how many blocks were compared exactly."""
    B, L = tok.shape
    V = z.shape[-1]
    wa, wn = O.rejection_verify(tok, q.astype(np.float64), ti, z, T, ua.astype(np.float64),
                                ur.astype(np.float64))
    lse = O.target_lse(z, T)
    exact = 0
    for b in range(B):
        clear = True
        for t in range(min(wa[b], L)):           # every decision the oracle took
            px = np.exp(z[b, t, tok[b, t]] / T - lse[b, t])
            d = float(ua[b, t]) * float(q[b, t, slot[b, t]]) - px
            if abs(d) <= 2e-4 * px:
                clear = False
                break
        if not clear:
            continue
        assert acc[b] == wa[b], b
        n = wa[b] - 1
        p = np.exp(z[b, n] / T - lse[b, n])
        if n < L:
            qv = np.zeros(V)
            np.add.at(qv, ti[b, n], q[b, n].astype(np.float64))
            r = np.maximum(p - qv, 0.0)
        else:
            r = p
        cum = np.cumsum(r)
        target = float(ur[b]) * cum[-1]
        win = RES_WIN * cum[-1]
        v = int(nxt[b])
        assert 0 <= v < V and r[v] > 0, b
        lo = cum[v - 1] if v > 0 else 0.0
        assert lo - win <= target <= cum[v] + win, b
        edges = np.concatenate([[0.0], cum])
        if np.min(np.abs(edges - target)) > win:
            assert v == wn[b], b
            exact += 1
    return exact


@pytest.mark.parametrize("B,L,V,T", [(50, 1, 16, 1.0), (200, 4, 1000, 1.0), (24, 8, 151936, 1.0),
                                     (31, 3, 4099, 0.5)])
def test_verify_rejection_parity(B, L, V, T):
    g = np.random.default_rng(B + L + V)
    ti, slot, tok, q, z, ua, ur = _spec_case(g, B, L, V, T)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    zd = d(z)
    lse = bd.target_lse(zd, T)
    acc, nxt = bd.verify_rejection(d(slot), d(tok), d(q), d(ti), zd, lse, T, d(ua), d(ur))
    exact = check_rejection(ti, slot, tok, q, z, T, ua, ur, acc.cpu().numpy(), nxt.cpu().numpy())
    if V <= 10000:                      # bins wider than the window: most draws decided
        assert exact >= 0.9 * B, exact
    a = acc.cpu().numpy()
    assert ((a >= 1) & (a <= L + 1)).all() and len(np.unique(a)) > 1


@pytest.mark.parametrize("B,L,V,T", [(50, 1, 16, 1.0), (200, 4, 1000, 1.0), (24, 8, 151936, 1.0),
                                     (31, 3, 4099, 0.5), (40, 64, 300, 1.0), (90, 2, 1001, 2.0)])
def test_verify_rejection_lazy_parity(B, L, V, T):
    g = np.random.default_rng(B + L + V + 7)
    ti, slot, tok, q, z, ua, ur = _spec_case(g, B, L, V, T)
    if L > 8:
        # long acceptance runs of every length: block b's drafted tokens are
        # likely under the target up to a position drawn per block
        cut = g.integers(0, L + 1, B)
        for b in range(B):
            for t in range(cut[b]):
                z[b, t, tok[b, t]] += np.float32(2 * np.log(V))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    acc, nxt = bd.verify_rejection_lazy(d(slot), d(tok), d(q), d(ti), d(z), T, d(ua), d(ur))
    exact = check_rejection(ti, slot, tok, q, z, T, ua, ur, acc.cpu().numpy(), nxt.cpu().numpy())
    if V <= 10000:
        assert exact >= 0.9 * B, exact
    a = acc.cpu().numpy()
    assert ((a >= 1) & (a <= L + 1)).all() and len(np.unique(a)) > 1


def test_verify_rejection_lazy_bad_tokens_and_neg_inf():
    # a token outside [0, V) or a slot outside [0, 16) fails its test; -inf
    # logits carry no mass and are never drawn
    g = np.random.default_rng(3)
    B, L, V, T = 6, 3, 700, 1.0
    ti, slot, tok, q, z, ua, ur = _spec_case(g, B, L, V, T)
    z[:, :, 100:400] = -np.inf
    tok[0, 0] = V
    slot[1, 0] = 16
    tok[2, 1] = -1
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    acc, nxt = bd.verify_rejection_lazy(d(slot), d(tok), d(q), d(ti), d(z), T, d(ua), d(ur))
    a, nx = acc.cpu().numpy(), nxt.cpu().numpy()
    assert a[0] == 1 and a[1] == 1 and a[2] <= 2
    assert ((nx < 100) | (nx >= 400)).all() and ((nx >= 0) & (nx < V)).all()
    # the two-call verification takes the same decisions here
    lse = bd.target_lse(d(z), T)
    acc2, _ = bd.verify_rejection(d(slot), d(tok), d(q), d(ti), d(z), lse, T, d(ua), d(ur))
    np.testing.assert_array_equal(a, acc2.cpu().numpy())


@pytest.mark.parametrize("B,L,V,T,rows", [
    (50, 1, 16, 1.0, 1), (50, 1, 16, 1.0, 2),          # every row staged (L + 1 = 2)
    (200, 4, 1000, 1.0, 2), (200, 4, 1000, 1.0, 5),
    (24, 8, 151936, 1.0, 2), (24, 8, 151936, 1.0, 9),
    (31, 3, 4099, 0.5, 2),                             # V % 4 != 0: scalar loads
    (40, 64, 300, 1.0, 2), (40, 64, 300, 1.0, 65),     # long acceptance runs
    (90, 2, 1001, 2.0, 3), (64, 8, 151936, 1.0, 1)])
def test_verify_rejection_staged_matches_lazy(B, L, V, T, rows):
    """The staged verification sums the first `rows` rows of every block up
    front with the lazy verification's arithmetic and merge order: accept
    lengths and drawn tokens equal the lazy call's bit for bit, and follow
    the oracle under the margin rules."""
    g = np.random.default_rng(B + L + V + rows)
    ti, slot, tok, q, z, ua, ur = _spec_case(g, B, L, V, T)
    if L > 8:
        cut = g.integers(0, L + 1, B)
        for b in range(B):
            for t in range(cut[b]):
                z[b, t, tok[b, t]] += np.float32(2 * np.log(V))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = (d(slot), d(tok), d(q), d(ti), d(z), T, d(ua), d(ur))
    acc0, nxt0 = bd.verify_rejection_lazy(*args)
    ws = torch.full((bd.verify_rejection_staged_workspace(B, L, V, rows),), 255, dtype=torch.uint8,
                    device=DEV)
    for _ in range(2):                        # the records are rewritten by every call
        acc1, nxt1 = bd.verify_rejection_staged(*args, rows=rows, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(acc0, acc1)
        assert torch.equal(nxt0, nxt1)
    a = acc1.cpu().numpy()
    check_rejection(ti, slot, tok, q, z, T, ua, ur, a, nxt1.cpu().numpy())
    assert ((a >= 1) & (a <= L + 1)).all()


def test_verify_rejection_staged_graph_replays():
    """The staged verification's two launches captured in a HIP graph: every
    replay, with eager calls on other inputs through the same workspace and
    synchronisations in between, gives the eager result."""
    g = np.random.default_rng(17)
    B, L, V, T = 64, 8, 151936, 1.0
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    case = [d(a) for a in _spec_case(g, B, L, V, T)]
    other = [d(a) for a in _spec_case(g, B, L, V, T)]

    def args(c):
        ti, slot, tok, q, z, ua, ur = c
        return (slot, tok, q, ti, z, T, ua, ur)

    ws = torch.empty(bd.verify_rejection_staged_workspace(B, L, V, 2), dtype=torch.uint8, device=DEV)
    acc = torch.empty((B,), dtype=torch.int32, device=DEV)
    nxt = torch.empty((B,), dtype=torch.int32, device=DEV)
    bd.verify_rejection_staged(*args(case), acc, nxt, rows=2, workspace=ws)
    torch.cuda.synchronize()
    want = (acc.clone(), nxt.clone())
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        bd.verify_rejection_staged(*args(case), acc, nxt, rows=2, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            bd.verify_rejection_staged(*args(case), acc, nxt, rows=2, workspace=ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(4):
        a2, n2 = bd.verify_rejection_staged(*args(other), rows=2, workspace=ws)
        torch.cuda.synchronize()
        acc.fill_(-7)
        nxt.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, want[0]) and torch.equal(nxt, want[1])


def test_verify_rejection_staged_bad_tokens_and_neg_inf():
    g = np.random.default_rng(3)
    B, L, V, T = 6, 3, 700, 1.0
    ti, slot, tok, q, z, ua, ur = _spec_case(g, B, L, V, T)
    z[:, :, 100:400] = -np.inf
    z[3, 0, :] = -np.inf                      # a staged row whose mass sits on one token
    z[3, 0, 5] = 0.0
    tok[0, 0] = V
    slot[1, 0] = 16
    tok[2, 1] = -1
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = (d(slot), d(tok), d(q), d(ti), d(z), T, d(ua), d(ur))
    acc0, nxt0 = bd.verify_rejection_lazy(*args)
    acc1, nxt1 = bd.verify_rejection_staged(*args)
    assert torch.equal(acc0, acc1) and torch.equal(nxt0, nxt1)
    a = acc1.cpu().numpy()
    assert a[0] == 1 and a[1] == 1 and a[2] <= 2


@pytest.mark.parametrize("lazy", [False, True, "staged"])
def test_verify_rejection_draw_past_the_last_prefix(lazy):
    """u_res at 1 or one ulp below it, with the row's last 256-token tile all
    -inf (V = 151936): when u * mass passes every tile prefix the draw takes
    the last token with residual mass, as the oracle does, and never emits an
    id outside [0, V).  Regression: the draw once fell back to the last tile
    without checking its mass and emitted -1."""
    g = np.random.default_rng(91)
    B, L, V, T = 16, 3, 151936, 1.0
    ti, slot, tok, q, z, ua, _ = _spec_case(g, B, L, V, T)
    last_tile = (V - 1) // 256 * 256
    z[:, :, last_tile:] = -np.inf
    # u = 1 is one past the uniforms' range [0, 1): the largest value
    # rounding of u * mass can reach
    ur = np.where(np.arange(B) % 2 == 0, np.float32(1.0),
                  np.nextafter(np.float32(1.0), np.float32(0.0))).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    if lazy == "staged":
        acc, nxt = bd.verify_rejection_staged(d(slot), d(tok), d(q), d(ti), d(z), T, d(ua), d(ur))
    elif lazy:
        acc, nxt = bd.verify_rejection_lazy(d(slot), d(tok), d(q), d(ti), d(z), T, d(ua), d(ur))
    else:
        lse = bd.target_lse(d(z), T)
        acc, nxt = bd.verify_rejection(d(slot), d(tok), d(q), d(ti), d(z), lse, T, d(ua), d(ur))
    a, nx = acc.cpu().numpy(), nxt.cpu().numpy()
    assert ((nx >= 0) & (nx < last_tile)).all(), nx
    check_rejection(ti, slot, tok, q, z, T, ua, ur, a, nx)
    wa, wn = O.rejection_verify(tok, q.astype(np.float64), ti, z, T, ua.astype(np.float64),
                                ur.astype(np.float64))
    same = (a == wa) & (ur == 1.0)
    assert same.sum() >= 4
    np.testing.assert_array_equal(nx[same], wn[same])      # the last token with mass


@pytest.mark.parametrize("lazy,mode", [(False, "chain"), (True, "chain"), (True, "path"),
                                       ("staged", "chain")])
def test_rejection_sampling_is_lossless_on_gpu(lazy, mode):
    # the whole sampled walk + verification on the GPU: emitted tokens follow
    # the target's softmax (chi-square on a 24-token vocabulary)
    from scipy.stats import chisquare

    g = np.random.default_rng(41)
    N, L, V, T = 60000, 2, 24, 1.0
    S0 = np.broadcast_to(g.standard_normal(16).astype(np.float32), (N, 16)).copy()
    S = np.broadcast_to(g.standard_normal((L - 1, 16, 16)).astype(np.float32),
                        (N, L - 1, 16, 16)).copy()
    ti = np.broadcast_to(np.stack([g.permutation(V)[:16] for _ in range(L)]).astype(np.int32),
                         (N, L, 16)).copy()
    zt = (g.standard_normal((L + 1, V)) * 1.5).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    slot, tok, q = bd.path_sample(d(S0), d(S), d(ti), d(g.random((N, L)).astype(np.float32)), T,
                                  mode=mode)
    zd = d(np.broadcast_to(zt, (N, L + 1, V)))
    ua, ur = d(g.random((N, L)).astype(np.float32)), d(g.random(N).astype(np.float32))
    if lazy == "staged":
        acc, nxt = bd.verify_rejection_staged(slot, tok, q, d(ti), zd, T, ua, ur)
    elif lazy:
        acc, nxt = bd.verify_rejection_lazy(slot, tok, q, d(ti), zd, T, ua, ur)
    else:
        lse = bd.target_lse(zd, T)
        acc, nxt = bd.verify_rejection(slot, tok, q, d(ti), zd, lse, T, ua, ur)
    acc, nxt, tok = acc.cpu().numpy(), nxt.cpu().numpy(), tok.cpu().numpy()
    p = np.exp(zt / T - O.target_lse(zt, T)[:, None])
    first = np.where(acc > 1, tok[:, 0], nxt)
    assert chisquare(np.bincount(first, minlength=V), p[0] * N).pvalue > 1e-4
    has2 = acc >= 2
    second = np.where(acc > 2, tok[:, 1], nxt)[has2]
    assert chisquare(np.bincount(second, minlength=V), p[1] * has2.sum()).pvalue > 1e-4


# ------------------------------------------------------------------ verify
def test_verify_parity():
    g = np.random.default_rng(5)
    for B, L in ((1, 1), (100, 8), (1000, 16), (3, 64)):
        path = g.integers(0, 3, (B, L)).astype(np.int32)
        tgt = g.integers(0, 3, (B, L + 1)).astype(np.int32)
        tgt[: B // 3, :L] = path[: B // 3]            # some full blocks
        wa, wn = O.verify_greedy(path, tgt)
        a, n = bd.verify_greedy(torch.from_numpy(path).to(DEV), torch.from_numpy(tgt).to(DEV))
        np.testing.assert_array_equal(a.cpu().numpy(), wa)
        np.testing.assert_array_equal(n.cpu().numpy(), wn)


# ------------------------------------------------------------------ fused scores + walk + verify
def _plant_targets(path_tok, V, seed):
    """Targets that follow the walked tokens for a random prefix of each block
    (every length from 0 to L occurs), then differ."""
    g = np.random.default_rng(seed)
    B, L = path_tok.shape
    tgt = np.empty((B, L + 1), np.int32)
    tgt[:, :L] = path_tok
    tgt[:, L] = g.integers(0, V, B)
    n = np.arange(B) % (L + 1)
    for b in range(B):
        if n[b] < L:
            tgt[b, n[b]] = (path_tok[b, n[b]] + 1 + g.integers(0, V - 1)) % V
    return tgt


@pytest.mark.parametrize("mode", ["viterbi", "greedy"])
@pytest.mark.parametrize("dt,B,L,V,r,gated,ties", [
    ("f32", 1, 1, 64, 1, False, False), ("bf16", 3, 2, 500, 7, True, False),
    ("bf16", 64, 8, 4096, 32, False, True), ("f32", 5, 16, 151936, 64, True, False),
    ("bf16", 40, 16, 151936, 256, False, False), ("bf16", 9, 17, 2000, 128, True, False),
    ("f32", 2, 5, 300, 256, False, False), ("bf16", 3, 64, 1000, 16, False, True),
    ("bf16", 5, 64, 3000, 256, True, False), ("f32", 300, 3, 700, 8, False, False)])
def test_fused_pair_walk_verify_matches_the_separate_calls(mode, dt, B, L, V, r, gated, ties):
    tv, ti, at, U, Vf = _pair_case(B, L, V, r, dt, seed=B * 7 + L + r)
    if ties:                                   # dyadic scores, no pair term: ties everywhere
        tv = (np.round(tv * 2) / 4).astype(np.float32)
        U = np.zeros_like(U)
    gate = (np.random.default_rng(r).random((B, L, r)).astype(np.float32) if gated else None)
    d = dict(tv=torch.from_numpy(tv).to(DEV), ti=torch.from_numpy(ti).to(DEV),
             at=torch.from_numpy(at).to(DEV), U=to_dev(U, dt), Vf=to_dev(Vf, dt),
             gate=None if gate is None else torch.from_numpy(gate).to(DEV))
    S0, S = bd.pair_score(d["tv"], d["ti"], d["at"], d["U"], d["Vf"], gate=d["gate"])
    slot, tok, score = bd.path_select(S0, S if L > 1 else None, d["ti"], mode=mode)
    tgt = _plant_targets(tok.cpu().numpy(), V, seed=B + L)
    tg = torch.from_numpy(tgt).to(DEV)
    acc, nxt = bd.verify_greedy(tok, tg)
    # fused, scores written out
    fS0 = torch.full_like(S0, 7.0)
    fS = torch.full_like(S, 7.0)
    f = bd.pair_select_verify(d["tv"], d["ti"], d["at"], d["U"], d["Vf"], tg, d["gate"], mode,
                              fS0, fS)
    assert torch.equal(fS0, S0) and torch.equal(fS, S)
    for got, want in zip(f, (slot, tok, score, acc, nxt)):
        assert torch.equal(got, want)
    # fused, scores kept on chip: the same outputs
    g2 = bd.pair_select_verify(d["tv"], d["ti"], d["at"], d["U"], d["Vf"], tg, d["gate"], mode)
    for got, want in zip(g2, (slot, tok, score, acc, nxt)):
        assert torch.equal(got, want)
    # and the acceptance follows the oracle's rule on the walked tokens
    wa, wn = O.verify_greedy(f[1].cpu().numpy(), tgt)
    np.testing.assert_array_equal(f[3].cpu().numpy(), wa)
    np.testing.assert_array_equal(f[4].cpu().numpy(), wn)
    if B >= L + 1:
        assert set(np.unique(wa)) == set(range(1, L + 2))


def test_fused_pair_walk_verify_against_the_oracle():
    B, L, V, r, dt = 6, 16, 4096, 64, "bf16"
    tv, ti, at, U, Vf = _pair_case(B, L, V, r, dt, seed=11)
    wS0, wS = O.pair_scores(tv, ti, at, U, Vf, dt)
    d = [torch.from_numpy(tv).to(DEV), torch.from_numpy(ti).to(DEV), torch.from_numpy(at).to(DEV),
         to_dev(U, dt), to_dev(Vf, dt)]
    S0 = torch.empty((B, 16), device=DEV)
    S = torch.empty((B, L - 1, 16, 16), device=DEV)
    probe = bd.pair_select_verify(*d, torch.zeros((B, L + 1), dtype=torch.int32, device=DEV),
                                  None, "viterbi", S0, S)
    assert np.abs(S0.cpu().numpy() - wS0).max() <= 1e-4
    assert np.abs(S.cpu().numpy() - wS).max() <= 1e-4
    # the walk is exact on the scores the kernel computed
    ws, wt, wsc = O.path_select(S0.cpu().numpy(), S.cpu().numpy(), ti)
    np.testing.assert_array_equal(probe[0].cpu().numpy(), ws)
    np.testing.assert_array_equal(probe[1].cpu().numpy(), wt)
    np.testing.assert_array_equal(probe[2].cpu().numpy().view(np.uint32), wsc.view(np.uint32))
    tgt = _plant_targets(wt, V, seed=3)
    out = bd.pair_select_verify(*d, torch.from_numpy(tgt).to(DEV), None, "viterbi")
    wa, wn = O.verify_greedy(wt, tgt)
    np.testing.assert_array_equal(out[3].cpu().numpy(), wa)
    np.testing.assert_array_equal(out[4].cpu().numpy(), wn)
    gs, gt, gsc = O.path_select_greedy(S0.cpu().numpy(), S.cpu().numpy(), ti)
    out = bd.pair_select_verify(*d, torch.from_numpy(tgt).to(DEV), None, "greedy")
    np.testing.assert_array_equal(out[0].cpu().numpy(), gs)
    np.testing.assert_array_equal(out[2].cpu().numpy().view(np.uint32), gsc.view(np.uint32))
    ga, gn = O.verify_greedy(gt, tgt)
    np.testing.assert_array_equal(out[3].cpu().numpy(), ga)
    np.testing.assert_array_equal(out[4].cpu().numpy(), gn)


@pytest.mark.parametrize("mode", ["viterbi", "greedy"])
def test_fused_verify_at_the_longest_block(mode):
    """L = 64, the longest walk: first mismatch at 0, 1, 62, 63, and no
    mismatch at all (the bonus target then sits past the last lane of the
    wave and comes from memory), checked against the oracle's rule."""
    B, L, V, r, dt = 5, 64, 3000, 16, "bf16"
    tv, ti, at, U, Vf = _pair_case(B, L, V, r, dt, seed=64)
    d = [torch.from_numpy(tv).to(DEV), torch.from_numpy(ti).to(DEV), torch.from_numpy(at).to(DEV),
         to_dev(U, dt), to_dev(Vf, dt)]
    probe = bd.pair_select_verify(*d, torch.zeros((B, L + 1), dtype=torch.int32, device=DEV),
                                  None, mode)
    tok = probe[1].cpu().numpy()
    g = np.random.default_rng(9)
    tgt = np.empty((B, L + 1), np.int32)
    tgt[:, :L] = tok
    tgt[:, L] = g.integers(0, V, B)                    # the bonus token
    for b, cut in enumerate([0, 1, 62, 63, None]):
        if cut is not None:
            tgt[b, cut] = (tok[b, cut] + 1) % V        # first mismatch at `cut`
    out = bd.pair_select_verify(*d, torch.from_numpy(tgt).to(DEV), None, mode)
    wa, wn = O.verify_greedy(tok, tgt)
    np.testing.assert_array_equal(out[3].cpu().numpy(), wa)
    np.testing.assert_array_equal(out[4].cpu().numpy(), wn)
    np.testing.assert_array_equal(wa, [1, 2, 63, 64, 65])
    assert wn[4] == tgt[4, L]


def test_fused_pair_walk_verify_empty_batch():
    U = torch.zeros((64, 8), device=DEV)
    e = torch.empty((0, 4, 16), device=DEV)
    out = bd.pair_select_verify(e, e.to(torch.int32), None, U, U,
                                torch.empty((0, 5), dtype=torch.int32, device=DEV))
    assert all(t.shape[0] == 0 for t in out)


@pytest.mark.parametrize("mode", ["chain", "path"])
@pytest.mark.parametrize("dt,B,L,V,r,gated,T", [
    ("f32", 1, 1, 64, 1, False, 1.0), ("bf16", 3, 2, 500, 7, True, 0.7),
    ("bf16", 64, 8, 4096, 32, False, 1.0), ("f32", 5, 16, 151936, 64, True, 2.0),
    ("bf16", 40, 8, 151936, 64, False, 1.0), ("bf16", 9, 17, 2000, 128, True, 1.0),
    ("bf16", 3, 64, 1000, 256, False, 0.5), ("f32", 300, 3, 700, 8, False, 1.0)])
def test_fused_pair_sample_matches_the_separate_calls(dt, B, L, V, r, gated, T, mode):
    tv, ti, at, U, Vf = _pair_case(B, L, V, r, dt, seed=B * 5 + L + r)
    g = np.random.default_rng(B + L)
    gate = g.random((B, L, r)).astype(np.float32) if gated else None
    u = g.random((B, L)).astype(np.float32)
    d = dict(tv=torch.from_numpy(tv).to(DEV), ti=torch.from_numpy(ti).to(DEV),
             at=torch.from_numpy(at).to(DEV), U=to_dev(U, dt), Vf=to_dev(Vf, dt),
             gate=None if gate is None else torch.from_numpy(gate).to(DEV),
             u=torch.from_numpy(u).to(DEV))
    S0, S = bd.pair_score(d["tv"], d["ti"], d["at"], d["U"], d["Vf"], gate=d["gate"])
    slot, tok, q = bd.path_sample(S0, S if L > 1 else None, d["ti"], d["u"], T, mode=mode)
    fS0 = torch.full_like(S0, 7.0)
    fS = torch.full_like(S, 7.0)
    f = bd.pair_sample(d["tv"], d["ti"], d["at"], d["U"], d["Vf"], d["u"], T, d["gate"], fS0, fS,
                       mode=mode)
    assert torch.equal(fS0, S0) and torch.equal(fS, S)
    for got, want in zip(f, (slot, tok, q)):
        assert torch.equal(got, want)
    g2 = bd.pair_sample(d["tv"], d["ti"], d["at"], d["U"], d["Vf"], d["u"], T, d["gate"],
                        mode=mode)
    for got, want in zip(g2, (slot, tok, q)):
        assert torch.equal(got, want)
    # the walk follows the oracle's sampling rule on the kernel's scores
    S0n, Sn = S0.cpu().numpy(), S.cpu().numpy()
    if mode == "path":
        ws, wt, wq = O.sample_path_joint(S0n, Sn, ti, T, u)
        tol = joint_sample_tol(S0n, Sn, T)
    else:
        ws, wt, wq = O.sample_path(S0n, Sn, ti, T, u)
        tol = SAMPLE_TOL
    k = decided_prefix(O.sample_margin(wq, u), tol)
    s_np = f[0].cpu().numpy()
    for b in range(B):
        np.testing.assert_array_equal(s_np[b, :k[b]], ws[b, :k[b]])
    if B >= 20:
        assert (k == L).mean() >= 0.9


def test_fused_pair_sample_empty_batch():
    U = torch.zeros((64, 8), device=DEV)
    e = torch.empty((0, 4, 16), device=DEV)
    out = bd.pair_sample(e, e.to(torch.int32), None, U, U, torch.empty((0, 4), device=DEV), 1.0)
    assert all(t.shape[0] == 0 for t in out)


@pytest.mark.parametrize("mode", ["viterbi", "greedy"])
def test_fused_calls_without_anchor_and_with_bad_ids(mode):
    # no anchor token (no match term at t = 0) and candidate ids outside
    # [0, V) (NaN scores): the fused calls still equal the separate ones bit
    # for bit, and every slot stays in [0, 16)
    B, L, V, r = 6, 5, 300, 16
    tv, ti, _, U, Vf = _pair_case(B, L, V, r, "f32", seed=77, anchor=False)
    ti[1, 2, 4] = V
    ti[3, 0, 0] = -5
    d = [torch.from_numpy(tv).to(DEV), torch.from_numpy(ti).to(DEV), None,
         torch.from_numpy(U).to(DEV), torch.from_numpy(Vf).to(DEV)]
    S0, S = bd.pair_score(*d)
    slot, tok, score = bd.path_select(S0, S, d[1], mode=mode)
    tg = torch.from_numpy(_plant_targets(tok.cpu().numpy(), V, seed=8)).to(DEV)
    acc, nxt = bd.verify_greedy(tok, tg)
    f = bd.pair_select_verify(*d, tg, None, mode)
    for got, want in zip(f, (slot, tok, score, acc, nxt)):
        assert torch.equal(got, want) or (got.dtype == torch.float32 and
                                          torch.equal(torch.isnan(got), torch.isnan(want)) and
                                          torch.equal(got[~torch.isnan(got)], want[~torch.isnan(want)]))
    s = f[0].cpu().numpy()
    assert ((s >= 0) & (s < 16)).all()
    u = torch.from_numpy(np.random.default_rng(2).random((B, L)).astype(np.float32)).to(DEV)
    ps, pt, pq = bd.path_sample(S0, S, d[1], u, 1.0)
    fs = bd.pair_sample(*d, u, 1.0)
    assert torch.equal(fs[0], ps) and torch.equal(fs[1], pt)
    assert torch.equal(torch.isnan(fs[2]), torch.isnan(pq))
    assert torch.equal(fs[2][~torch.isnan(pq)], pq[~torch.isnan(pq)])
