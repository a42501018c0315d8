"""C-ABI checks that need no GPU: the library loads, exports every function
include/dflash2.h declares, and rejects bad arguments on the host before any
launch (fake device addresses are safe here: validation fails first)."""
import ctypes
import os
import re
import subprocess

import pytest

import block_drafting_amd as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")

EINVAL, EUNSUP, EHIP, EWS, ESCRATCH = -1, -2, -3, -4, -5
P = 0x7f0000001000          # 4 KiB-aligned fake device address (never dereferenced)
Q = 0x7f0000100000          # another, far from P


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dflash2_\w+)\s*\(", text, re.M)))


def test_header_declares_the_five_step_calls():
    names = _declared()
    for n in ("dflash2_twotap_conv", "dflash2_logits_topk", "dflash2_pair_score",
              "dflash2_path_select", "dflash2_verify_greedy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = bd.lib()
    for n in _declared():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", bd.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dflash2_\w+)", out))
    assert exported == set(_declared())      # nothing undeclared leaks out


def test_version_and_strerror():
    L = bd.lib()
    assert L.dflash2_version() >= 10000
    for s in (0, EINVAL, EUNSUP, EHIP, EWS, ESCRATCH):
        assert len(L.dflash2_strerror(s)) > 0
    assert L.dflash2_strerror(12345) == b"unknown status"


def test_conv_validation():
    f = bd.lib().dflash2_twotap_conv
    ok = dict(x=P, a=None, y=Q, k0=P + 0x80000, k1=P + 0x90000, pr=None, g=1, B=2, L=8, H=64, dt=1)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["a"], a["y"], a["k0"], a["k1"], a["pr"], a["g"], a["B"], a["L"],
                 a["H"], a["dt"], None)

    assert call(B=0) == 0                     # empty batch: nothing to do
    assert call(x=None) == EINVAL
    assert call(k1=None) == EINVAL
    assert call(L=0) == EINVAL
    assert call(H=12) == EINVAL               # H % 8
    assert call(dt=7) == EINVAL
    assert call(y=P) == EINVAL                # y aliases x
    assert call(y=P + 64) == EINVAL           # partial overlap
    assert call(y=Q, k0=Q + 0x100) == EINVAL  # y overlaps a tap vector
    assert call(y=Q, k1=Q + 0x7f0) == EINVAL
    assert call(y=Q, pr=Q + 0x10, g=1) == EINVAL   # ... or the projection
    assert call(x=P + 4) == EINVAL            # misaligned
    assert call(pr=P + 0xa0000, g=3) == EINVAL   # groups must divide H
    assert call(pr=P + 0xa0000, g=0) == EINVAL
    assert call(B=-1) == EINVAL
    # one workgroup per row with a projection: B*L must fit the grid
    assert call(pr=P + 0xa0000, B=40_000_000, L=64, H=8) == EUNSUP


def test_conv_mm_validation():
    f = bd.lib().dflash2_twotap_conv_mm
    ok = dict(x=P, a=None, y=Q, k0=P + 0x80000, k1=P + 0x90000, pt=P + 0xa0000, g=4, B=2, L=8,
              H=64, dt=1)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["a"], a["y"], a["k0"], a["k1"], a["pt"], a["g"], a["B"], a["L"],
                 a["H"], a["dt"], None)

    assert call(B=0) == 0
    assert call(dt=0) == EUNSUP               # matrix cores take bf16
    assert call(pt=None) == EINVAL
    assert call(pt=P + 0xa0004) == EINVAL     # misaligned map
    assert call(g=3) == EINVAL                # groups must divide H
    assert call(g=0) == EINVAL
    assert call(y=P + 0xa0000) == EINVAL      # y overlaps the map
    assert call(y=P) == EINVAL                # y aliases x
    assert call(y=Q, k0=Q + 0x100) == EINVAL  # y overlaps a tap vector (it holds partial sums)
    assert call(y=Q, k1=Q + 0x7f0) == EINVAL
    assert call(H=12) == EINVAL
    assert call(H=(1 << 21) + 64, g=1) == EUNSUP


def test_lmhead_and_topk_validation():
    L = bd.lib()
    assert L.dflash2_lmhead_logits(P, Q, P + 0x10000000, 8, 64, 15, 1, None) == EINVAL  # V < 16
    assert L.dflash2_lmhead_logits(P, Q, P + 0x10000000, 8, 60, 64, 1, None) == EINVAL  # H % 8
    assert L.dflash2_lmhead_logits(P, Q, None, 8, 64, 64, 1, None) == EINVAL
    assert L.dflash2_lmhead_logits(P, Q, P, 8, 64, 64, 1, None) == EINVAL              # aliasing
    assert L.dflash2_lmhead_logits(P, Q, None, 0, 64, 64, 1, None) == 0                 # M == 0
    assert L.dflash2_topk16(P, Q, Q + 4096, 4, 100, 8, None, 0, None) == EINVAL         # K != 16
    assert L.dflash2_topk16(P, None, Q, 4, 100, 16, None, 0, None) == EINVAL
    need = L.dflash2_topk16_workspace(64, 151936, 16)     # short batch: rows split
    assert need > 0 and L.dflash2_topk16_workspace(64, 151936, 8) == 0
    big = 0x7e0000000000
    assert L.dflash2_topk16(big, Q, Q + 65536, 64, 151936, 16, None, 0, None) == EWS
    assert L.dflash2_topk16(big, Q, Q + 65536, 64, 151936, 16, P, need - 1, None) == EWS
    assert L.dflash2_topk16(big, Q, Q + 65536, 64, 151936, 16, P + 16, need, None) == EWS  # align
    ws_given = L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 0, 1)
    ws_none = L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 0, 0)
    assert ws_none - ws_given == 512 * 151936 * 4                  # fp32: the logits
    # bf16 without logits: + group maxima [M, 16], counts [M, 594], slots [M, 594, 4] x 8 bytes
    cand = 512 * 16 * 4 + 512 * 594 * 4 + 512 * 594 * 32
    assert (L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 1, 0) ==
            L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 1, 1) + cand + 512 * 151936 * 4)
    assert L.dflash2_logits_topk(P, Q, None, P + 4096, P + 8192, 512, 5120, 151936, 16, 1,
                                 None, 0, None) == EWS                             # no room for logits


def test_lmhead_pack_validation():
    L = bd.lib()
    nb = L.dflash2_lmhead_pack_bytes
    assert nb(151936, 5120) == 594 * 80 * 256 * 64 * 2       # whole 256 x 64 blocks
    assert nb(1, 8) == nb(256, 64) == 32768
    assert nb(257, 72) == 2 * 2 * 32768
    assert nb(0, 64) == 0 and nb(100, 60) == 0 and nb(100, 0) == 0
    assert nb(1, (1 << 21) + 8) == 0                          # beyond 32-bit tile offsets
    pk = L.dflash2_lmhead_pack
    far = P + 0x10000000
    assert pk(P, far, 0, 64, None) == EINVAL                  # V < 1
    assert pk(P, far, 100, 60, None) == EINVAL                # H % 8
    assert pk(None, far, 100, 64, None) == EINVAL
    assert pk(P, None, 100, 64, None) == EINVAL
    assert pk(P, far + 8, 100, 64, None) == EINVAL            # misaligned
    assert pk(P, P + 8192, 100, 64, None) == EINVAL           # inside W (12800 bytes)
    assert pk(P + 16384, P, 100, 64, None) == EINVAL          # W inside the 32 KiB of Wp
    assert pk(P, far, 1, (1 << 21) + 8, None) == EUNSUP
    # packed W spans whole blocks: a logits buffer past V * H * 2 bytes but
    # inside the packed size overlaps it
    z = Q + 16384
    assert L.dflash2_lmhead_logits(P, Q, z, 8, 64, 100, 2, None) == EINVAL
    assert L.dflash2_lmhead_logits_tilemax(P, Q, z, far, 8, 64, 100, 2, None) == EINVAL
    assert L.dflash2_lmhead_logits(P, Q, far, 8, 64, 100, 3, None) == EINVAL   # unknown dtype
    assert L.dflash2_lmhead_logits(P, Q, None, 0, 64, 100, 2, None) == 0
    assert (L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 2, 0) ==
            L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 1, 0))
    assert L.dflash2_logits_topk(P, Q, z, far, far + 4096, 8, 64, 100, 16, 2, far + 65536,
                                 1 << 20, None) == EINVAL
    # the packed code belongs to the LM head only
    assert L.dflash2_pair_score(P, P, None, P, P, 2, 4, 1000, 8, 2, P, P, None) == EINVAL
    assert L.dflash2_context_gate(P, Q, far, 8, 64, 8, 2, None) == EINVAL


def test_tilemax_validation():
    L = bd.lib()
    f = L.dflash2_lmhead_logits_tilemax
    z, tm = P + 0x10000000, P + 0x20000000
    assert f(P, Q, z, None, 8, 64, 1000, 1, None) == EINVAL              # tilemax missing
    assert f(P, Q, z, z + 64, 8, 64, 1000, 1, None) == EINVAL            # overlaps the logits
    assert f(P, Q, z, tm + 2, 8, 64, 1000, 1, None) == EINVAL            # misaligned
    assert f(P, Q, z, tm, 8, 60, 1000, 1, None) == EINVAL                # H % 8
    assert f(P, Q, z, tm, 0, 64, 1000, 1, None) == 0
    k = L.dflash2_topk16_tilemax
    assert k(z, tm, P, P + 4096, 8, 1000, 8, None) == EINVAL             # K != 16
    assert k(z, None, P, P + 4096, 8, 1000, 16, None) == EINVAL
    assert k(z, tm, tm, P + 4096, 8, 1000, 16, None) == EINVAL           # top_val over tilemax
    assert k(z, tm, P, P, 8, 1000, 16, None) == EINVAL                   # outputs alias
    assert k(z, tm, P, P + 4096, 0, 1000, 16, None) == 0
    assert L.dflash2_logits_topk_workspace(512, 5120, 151936, 16, 1, 1) >= 512 * 594 * 4


def test_pair_select_verify_validation():
    L = bd.lib()
    ps = L.dflash2_pair_score
    #        tv  ti          anc   U   V             B  L  V    r  dt S0           S
    args = [P, P + 0x10000, None, Q, Q + 0x100000, 2, 4, 100, 8, 1, P + 0x20000, P + 0x30000]
    assert ps(*args[:8], 0, *args[9:], None) == EINVAL       # r = 0
    assert ps(*args[:8], 257, *args[9:], None) == EINVAL     # r > 256
    assert ps(*args[:6], 65, *args[7:], None) == EINVAL      # L > 64
    assert ps(*args[:6], 0, *args[7:], None) == EINVAL       # L = 0
    assert ps(*args[:7], 15, *args[8:], None) == EINVAL      # V < 16
    bad = list(args)
    bad[11] = P                                              # S overlaps top_val
    assert ps(*bad, None) == EINVAL
    bad = list(args)
    bad[11] = None                                           # S missing with L > 1
    assert ps(*bad, None) == EINVAL
    bad = list(args)
    bad[11] = P + 0x30004                                    # S misaligned
    assert ps(*bad, None) == EINVAL
    assert ps(*args[:5], 0, *args[6:], None) == 0            # B = 0

    sel = L.dflash2_path_select
    assert sel(P, Q, None, 2, 0, P + 0x1000, None, P + 0x2000, None) == EINVAL
    assert sel(P, Q, None, 2, 65, P + 0x1000, None, P + 0x2000, None) == EINVAL
    assert sel(P, Q, P + 0x9000, 2, 4, P + 0x1000, None, P + 0x2000, None) == EINVAL  # tok pair
    assert sel(P, None, None, 2, 4, P + 0x1000, None, P + 0x2000, None) == EINVAL     # S missing
    assert sel(P, Q, None, 2, 4, P + 0x1000, None, P + 0x1000, None) == EINVAL        # outs alias
    assert sel(P, Q, None, 0, 4, P + 0x1000, None, P + 0x2000, None) == 0

    ver = L.dflash2_verify_greedy
    assert ver(P, Q, 4, 0, P + 0x1000, None, None) == EINVAL
    assert ver(None, Q, 4, 8, P + 0x1000, None, None) == EINVAL
    assert ver(P, Q, 4, 8, P, None, None) == EINVAL           # accept_len aliases path_tok
    assert ver(P, Q, 4, 8, P + 0x1000, P + 0x1000, None) == EINVAL
    assert ver(P, Q, 0, 8, P + 0x1000, None, None) == 0


def test_fused_pair_walk_verify_validation():
    f = bd.lib().dflash2_pair_select_verify
    ok = dict(tv=P, ti=P + 0x10000, anc=None, U=Q, Vf=Q + 0x100000, gate=None, tg=P + 0x50000,
              B=2, L=4, V=100, r=8, dt=1, mode=0, S0=P + 0x20000, S=P + 0x30000,
              slot=P + 0x60000, tok=P + 0x61000, score=P + 0x62000, acc=P + 0x63000,
              nt=P + 0x64000)

    def call(**kw):
        a = dict(ok, **kw)
        return f(*(a[k] for k in ok), None)

    # every call below is rejected (or empty) before anything is launched

    assert call(B=0) == 0
    assert call(B=-1) == EINVAL
    assert call(mode=2) == EINVAL
    assert call(mode=-1) == EINVAL
    assert call(L=0) == EINVAL
    assert call(L=65) == EINVAL
    assert call(r=0) == EINVAL
    assert call(r=257) == EINVAL
    assert call(V=15) == EINVAL
    assert call(dt=3) == EINVAL
    for k in ("tv", "ti", "U", "Vf", "tg", "slot", "score", "acc"):
        assert call(**{k: None}) == EINVAL, k
    assert call(tg=P + 0x50002) == EINVAL        # misaligned target
    assert call(U=Q + 1) == EINVAL                # odd bf16 factor address
    assert call(acc=P + 0x50004) == EINVAL        # accept_len overlaps target
    assert call(S=P) == EINVAL                    # S overlaps top_val
    assert call(S0=P + 0x30000 + 64) == EINVAL    # S0 inside S
    assert call(tok=P + 0x60000) == EINVAL        # path_tok aliases path_slot
    assert call(nt=P + 0x63000) == EINVAL         # next_tok aliases accept_len
    assert call(gate=P + 0x20000) == EINVAL       # gate overlaps S0
    assert call(slot=Q + 0x100000) == EINVAL      # output over a factor
    assert call(S0=None, S=None, B=0) == 0        # scores may stay on chip


def test_fused_pair_sample_validation():
    f = bd.lib().dflash2_pair_sample
    ok = dict(tv=P, ti=P + 0x10000, anc=None, U=Q, Vf=Q + 0x100000, gate=None, u=P + 0x50000,
              T=1.0, B=2, L=4, V=100, r=8, dt=1, S0=P + 0x20000, S=P + 0x30000,
              slot=P + 0x60000, tok=P + 0x61000, q=P + 0x62000)

    def call(**kw):
        a = dict(ok, **kw)
        return f(*(a[k] for k in ok), None)

    # every call below is rejected (or empty) before anything is launched
    assert call(B=0) == 0
    assert call(B=-1) == EINVAL
    assert call(T=0.0) == EINVAL
    assert call(T=float("inf")) == EINVAL
    assert call(L=0) == EINVAL
    assert call(L=65) == EINVAL
    assert call(r=257) == EINVAL
    assert call(V=15) == EINVAL
    for k in ("tv", "ti", "U", "Vf", "u", "slot", "q"):
        assert call(**{k: None}) == EINVAL, k
    assert call(u=P + 0x50002) == EINVAL          # misaligned uniforms
    assert call(q=P + 0x50000) == EINVAL          # q over the uniforms
    assert call(S=P) == EINVAL                    # S over top_val
    assert call(tok=P + 0x60000) == EINVAL        # path_tok aliases path_slot
    assert call(S0=None, S=None, B=0) == 0


def test_lazy_rejection_validation():
    f = bd.lib().dflash2_verify_rejection_lazy
    #     slot  tok         q            ti           z   T    ua           ur
    ok = [P, P + 0x1000, P + 0x2000, P + 0x4000, Q, 1.0, P + 0x6000, P + 0x7000,
          4, 2, 1000, P + 0x8000, P + 0x9000]
    #     B  L  V     acc          nxt

    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a, None)

    # every call below is rejected (or empty) before anything is launched
    assert call(8, 0) == 0                        # B = 0
    assert call(8, -1) == EINVAL
    assert call(9, 0) == EINVAL                   # L = 0
    assert call(9, 65) == EINVAL                  # L > 64
    assert call(10, 15) == EINVAL                 # V < 16
    assert call(10, 2097152 + 256) == EUNSUP      # tiles exceed 64 KiB of LDS
    assert call(5, 0.0) == EINVAL                 # T must be > 0
    assert call(5, float("nan")) == EINVAL
    for i in (0, 1, 2, 3, 4, 6, 7, 11, 12):
        assert call(i, None) == EINVAL, i
    assert call(11, Q + 64) == EINVAL             # accept_len inside z
    assert call(12, P + 0x8000) == EINVAL         # next_tok aliases accept_len
    assert call(0, P + 2) == EINVAL               # misaligned


def test_staged_rejection_validation():
    f = bd.lib().dflash2_verify_rejection_staged
    need = bd.lib().dflash2_verify_rejection_staged_workspace(4, 2, 1000, 2)
    assert need == 4 * 2 * (2 * 4 + 2 * 1) * 4            # [B, rows] records of 4 tiles, 1 batch
    assert bd.lib().dflash2_verify_rejection_staged_workspace(4, 2, 1000, 0) == 0
    assert bd.lib().dflash2_verify_rejection_staged_workspace(4, 2, 1000, 4) == 0   # rows > L + 1
    W = P + 0x20000
    #     slot  tok         q            ti           z   T    ua           ur
    ok = [P, P + 0x1000, P + 0x2000, P + 0x4000, Q, 1.0, P + 0x6000, P + 0x7000,
          4, 2, 1000, 2, W, need, P + 0x8000, P + 0x9000]
    #     B  L  V    rows ws need  acc          nxt

    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a, None)

    assert call(8, 0) == 0                        # B = 0
    assert call(11, 0) == EINVAL                  # rows < 1
    assert call(11, 4) == EINVAL                  # rows > L + 1
    assert call(12, None) == EINVAL               # no workspace
    assert call(13, need - 4) == EINVAL           # workspace too small
    assert call(12, W + 2) == EINVAL              # misaligned workspace
    assert call(12, Q + 64) == EINVAL             # workspace inside z
    assert call(12, P + 0x8000 - 16) == EINVAL    # workspace over accept_len
    assert call(10, 2097152 + 256) == EUNSUP      # tiles exceed 64 KiB of LDS
    assert call(5, 0.0) == EINVAL
    for i in (0, 1, 2, 3, 4, 6, 7, 14, 15):
        assert call(i, None) == EINVAL, i
    assert call(14, Q + 64) == EINVAL             # accept_len inside z


def test_gate_and_gated_pair_validation():
    L = bd.lib()
    cg = L.dflash2_context_gate
    #          h  Wg          gate          M   H    r   dt
    ok = [P, P + 0x100000, Q, 8, 64, 16, 1]
    assert cg(*ok[:4], 60, *ok[5:], None) == EINVAL              # H % 8
    assert cg(*ok[:5], 0, 1, None) == EINVAL                     # r = 0
    assert cg(*ok[:5], 257, 1, None) == EINVAL                   # r > 256
    assert cg(*ok[:6], 3, None) == EINVAL                        # dtype
    assert cg(None, *ok[1:], None) == EINVAL
    assert cg(P + 4, *ok[1:], None) == EINVAL                    # h misaligned
    assert cg(P, P + 0x100000, P + 64, 8, 64, 16, 1, None) == EINVAL   # gate overlaps h
    assert cg(P, P + 0x100000, Q, 8, (1 << 21) + 8, 16, 1, None) == EUNSUP
    assert cg(*ok[:3], 0, *ok[4:], None) == 0                    # M = 0
    pg = L.dflash2_pair_score_gated
    #       tv  ti          anc   U   V             gate          B  L  V    r  dt S0           S
    args = [P, P + 0x10000, None, Q, Q + 0x100000, P + 0x40000, 2, 4, 100, 8, 1, P + 0x20000,
            P + 0x30000]
    bad = list(args)
    bad[5] = None                                                # gate required
    assert pg(*bad, None) == EINVAL
    bad[5] = P + 0x40002                                         # misaligned
    assert pg(*bad, None) == EINVAL
    bad[5] = P + 0x30000                                         # gate overlaps S
    assert pg(*bad, None) == EINVAL
    bad = list(args)
    bad[9] = 300                                                 # r > 256
    assert pg(*bad, None) == EINVAL
    assert pg(*args[:6], 0, *args[7:], None) == 0                # B = 0


def test_path_select_mode_validation():
    sm = bd.lib().dflash2_path_select_mode
    assert sm(P, Q, None, 2, 4, 2, P + 0x1000, None, P + 0x2000, None) == EINVAL   # mode
    assert sm(P, Q, None, 2, 4, -1, P + 0x1000, None, P + 0x2000, None) == EINVAL
    assert sm(P, Q + 4, None, 2, 4, 1, P + 0x1000, None, P + 0x2000, None) == EINVAL  # S align
    assert sm(P, Q, None, 2, 65, 1, P + 0x1000, None, P + 0x2000, None) == EINVAL
    assert sm(P, Q, None, 2, 4, 1, P + 0x1000, None, P + 0x1000, None) == EINVAL     # alias
    assert sm(P, Q, None, 0, 4, 1, P + 0x1000, None, P + 0x2000, None) == 0
    assert bd.PATH_MODES == {"viterbi": 0, "greedy": 1}
    text = open(HEADER).read()
    assert "DFLASH2_PATH_VITERBI = 0" in text and "DFLASH2_PATH_GREEDY = 1" in text


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 8, 64), dtype=torch.bfloat16)
    k = torch.zeros(64)
    with pytest.raises(ValueError):
        bd.twotap_conv(x, k, k)


def test_logits_topk_noalloc_validation():
    """The allocation-free logits + top-16: the logits are required, and a
    problem whose tile maxima exceed the fixed scratch is refused with its
    own status before anything touches the device."""
    f = bd.lib().dflash2_logits_topk_noalloc
    MB = 1 << 20
    h, W, z, tv, ti = P, P + 512 * MB, P + 4096 * MB, P + 16384 * MB, P + 16400 * MB

    def call(M=512, H=5120, V=151936, K=16, dt=1, z_=z, h_=h):
        return f(h_, W, z_, tv, ti, M, H, V, K, dt, None)

    assert call(M=0) == 0
    assert call(K=8) == EINVAL
    assert call(z_=None) == EINVAL                       # logits are a caller-given output
    assert call(z_=z + 4) == EINVAL                      # 16-byte alignment
    assert call(h_=None) == EINVAL
    assert call(z_=h) == EINVAL                          # logits overlap h
    assert call(M=7062) == ESCRATCH                      # 7062 * 594 * 4 > 16 MiB
    assert call(M=4096, V=1 << 20) == ESCRATCH
    assert bd.lib().dflash2_strerror(ESCRATCH).startswith(b"problem larger")


def test_sample_mode_validation():
    """The sampling calls' mode argument: chain (0) or whole path (1); any
    other value is refused before any launch."""
    L = bd.lib()
    f = L.dflash2_path_sample_mode
    S0, S, u, slot, q = P, P + 0x10000, P + 0x80000, P + 0x90000, P + 0xA0000
    assert f(S0, S, None, u, 1.0, 0, 4, 1, slot, None, q, None) == 0      # empty batch
    assert f(S0, S, None, u, 1.0, 2, 4, 2, slot, None, q, None) == EINVAL
    assert f(S0, S, None, u, 1.0, 2, 4, -1, slot, None, q, None) == EINVAL
    assert f(S0, S, None, u, 0.0, 2, 4, 1, slot, None, q, None) == EINVAL  # T must be > 0
    g = L.dflash2_pair_sample_mode
    tv, ti, U, Vf = P, P + 0x10000, P + 0x100000, P + 0x200000
    args = lambda mode, B=2: (tv, ti, None, U, Vf, None, u + 0x400000, 1.0, B, 4, 1000, 8, 1,
                              mode, None, None, slot + 0x400000, None, q + 0x400000, None)
    assert g(*args(1, B=0)) == 0
    assert g(*args(3)) == EINVAL


def test_candidate_form_validation():
    """dflash2_lmhead_candidates / dflash2_topk16_candidates reject bad
    arguments on the host before any launch."""
    L = bd.lib()
    g, t = L.dflash2_lmhead_candidates, L.dflash2_topk16_candidates
    need = L.dflash2_logits_topk_workspace(64, 256, 4096, 16, 1, 0)
    assert need == L.dflash2_logits_topk_workspace(64, 256, 4096, 16, 2, 0)
    ws = P + 0x40000000
    #       h  W   M   H    V     dt ws  bytes
    assert g(P, Q, 64, 256, 4096, 0, ws, need, None) == EUNSUP            # fp32 operands
    assert g(P, Q, 64, 256, 4096, 1, None, 0, None) == EWS
    assert g(P, Q, 64, 256, 4096, 1, ws, need - 1, None) == EWS
    assert g(P, Q, 64, 256, 4096, 1, ws + 16, need, None) == EWS          # 256-byte alignment
    assert g(P, Q, 64, 256, 4096, 1, P, need, None) == EINVAL             # over h
    assert g(P, Q, 64, 60, 4096, 1, ws, need, None) == EINVAL             # H % 8
    assert g(P, Q, 0, 256, 4096, 1, None, 0, None) == 0                   # M == 0
    out = P + 0x80000000
    #       ws  bytes  top_val  top_idx     M   H    V     K
    assert t(ws, need, out, out + 8192, 64, 256, 4096, 8, None) == EINVAL  # K != 16
    assert t(ws, need - 1, out, out + 8192, 64, 256, 4096, 16, None) == EWS
    assert t(None, 0, out, out + 8192, 64, 256, 4096, 16, None) == EWS
    assert t(ws, need, ws, out + 8192, 64, 256, 4096, 16, None) == EINVAL  # top_val in the workspace
    assert t(ws, need, out, out, 64, 256, 4096, 16, None) == EINVAL        # outputs alias
    assert t(ws, need, None, out, 64, 256, 4096, 16, None) == EINVAL
    assert t(ws, need, out, out + 8192, 0, 256, 4096, 16, None) == 0
