"""DFlash 2 draft-select-verify step on MI355X (gfx950): Python binding.

A thin ctypes layer over libdflash2.so (include/dflash2.h).  It checks the
torch tensors it is given (device, dtype, shape, contiguity), passes raw
device pointers and the current HIP stream, and raises on a non-zero status.
Every stage of the step runs in the library's HIP kernels; PyTorch only
provides device memory and streams.  There is no fallback: without the built
library every call raises.

The five stages (names as in the C ABI):
  twotap_conv     two-tap local conv around the drafter's sublayers
                  (twotap_conv_mm: one correction per 16 channels, on the
                  matrix cores)
  logits_topk     LM-head logits and per-position top-16 candidates
                  (= lmhead_logits then topk16; W may be a PackedWeight from
                  lmhead_pack, the GEMM's tile layout, made once per weight)
  pair_score      16x16 scores of neighbouring candidates (optionally
                  weighted by a context gate from context_gate)
  path_select     max-plus walk (or the greedy best-successor walk) to one
                  path per block
  verify_greedy   greedy verification, acceptance length
At T > 0: path_sample (sampled walk), target_lse + verify_rejection (lossless
speculative-sampling verification against target logits), or
verify_rejection_lazy (the same rule, each target row's log-sum-exp computed
only for the rows the accept test reaches) or verify_rejection_staged (the
lazy rule with every block's first rows summed up front, all blocks at once;
the same results bit for bit).
One launch for several stages: pair_select_verify (scores, either walk and
greedy verification) and pair_sample (scores and the sampling walk).
run_step chains a whole step on preallocated StepBuffers.

Example (one greedy-verified step of 64 blocks of 8 positions):
    buf = StepBuffers(64, 8, H, V, torch.bfloat16, "cuda")
    run_step(buf, x, [dict(k0=k0, k1=k1, anchor_h=a)], W, U, Vf, anchor_tok, target)
    buf.accept_len, buf.next_tok      # int32 [64] each
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "DFlash2Error", "lib", "library_path", "twotap_conv", "twotap_conv_mm", "lmhead_logits",
    "lmhead_logits_tilemax", "lmhead_pack", "PackedWeight", "topk16", "topk16_tilemax",
    "topk16_workspace", "logits_topk", "logits_topk_workspace", "logits_topk_noalloc",
    "lmhead_candidates", "topk16_candidates",
    "context_gate", "pair_score",
    "path_select", "pair_select_verify", "pair_sample", "path_sample", "SAMPLE_MODES", "target_lse", "verify_rejection", "verify_rejection_lazy", "verify_rejection_staged", "verify_rejection_staged_workspace", "STAGED_ROWS", "verify_greedy", "StepBuffers", "run_step", "TOPK", "PATH_MODES",
]

TOPK = 16
PATH_MODES = {"viterbi": 0, "greedy": 1}
SAMPLE_MODES = {"chain": 0, "path": 1}
_HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH2_LIBRARY selects another build of the same library (the host
# AddressSanitizer build that the CPU tests load, for instance)
library_path = os.environ.get("DFLASH2_LIBRARY") or os.path.join(_HERE, "libdflash2.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

_SIGS = {
    "dflash2_version": ([], _I),
    "dflash2_strerror": ([_I], ctypes.c_char_p),
    "dflash2_twotap_conv": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "dflash2_twotap_conv_mm": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "dflash2_lmhead_logits": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "dflash2_lmhead_logits_tilemax": ([_P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "dflash2_lmhead_pack_bytes": ([_I, _I], _Z),
    "dflash2_lmhead_pack": ([_P, _P, _I, _I, _P], _I),
    "dflash2_topk16_tilemax": ([_P, _P, _P, _P, _I, _I, _I, _P], _I),
    "dflash2_topk16_workspace": ([_I, _I, _I], _Z),
    "dflash2_topk16": ([_P, _P, _P, _I, _I, _I, _P, _Z, _P], _I),
    "dflash2_logits_topk_workspace": ([_I, _I, _I, _I, _I, _I], _Z),
    "dflash2_logits_topk": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P], _I),
    "dflash2_logits_topk_noalloc": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "dflash2_lmhead_candidates": ([_P, _P, _I, _I, _I, _I, _P, _Z, _P], _I),
    "dflash2_topk16_candidates": ([_P, _Z, _P, _P, _I, _I, _I, _I, _P], _I),
    "dflash2_probe_mfma_operand_bytes": ([_I], _Z),
    "dflash2_probe_mfma": ([_P, _I, _I, _P, _P], _I),
    "dflash2_pair_score": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "dflash2_context_gate": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "dflash2_pair_score_gated": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "dflash2_path_select": ([_P, _P, _P, _I, _I, _P, _P, _P, _P], _I),
    "dflash2_path_select_mode": ([_P, _P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
    "dflash2_verify_greedy": ([_P, _P, _I, _I, _P, _P, _P], _I),
    "dflash2_pair_sample": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _I, _I, _P,
                             _P, _P, _P, _P, _P], _I),
    "dflash2_pair_select_verify": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P,
                                    _P, _P, _P, _P, _P, _P], _I),
    "dflash2_path_sample": ([_P, _P, _P, _P, ctypes.c_float, _I, _I, _P, _P, _P, _P], _I),
    "dflash2_path_sample_mode": ([_P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _P, _P, _P, _P], _I),
    "dflash2_pair_sample_mode": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _I, _I,
                                  _I, _P, _P, _P, _P, _P, _P], _I),
    "dflash2_target_lse": ([_P, _I, _I, ctypes.c_float, _P, _P], _I),
    "dflash2_verify_rejection": ([_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _I,
                                  _P, _P, _P], _I),
    "dflash2_verify_rejection_lazy": ([_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _I,
                                       _P, _P, _P], _I),
    "dflash2_verify_rejection_staged_workspace": ([_I, _I, _I, _I], ctypes.c_size_t),
    "dflash2_verify_rejection_staged": ([_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _I,
                                         _I, _P, ctypes.c_size_t, _P, _P, _P], _I),
}


class DFlash2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().dflash2_strerror(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libdflash2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is not built; run `python -m block_drafting_amd.build` "
                "(the HIP library is required, there is no fallback)")
        L = ctypes.CDLL(library_path)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise DFlash2Error(fn, status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype == torch.float32:
        return 0
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(*ts: Optional[torch.Tensor]):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must share one device")
    return dev


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _shape(t: torch.Tensor, shape, name: str, dtype=None):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _opt(t: Optional[torch.Tensor], shape, name: str, dtype=None):
    """_shape for a tensor the caller may leave out (None)."""
    if t is not None:
        _shape(t, shape, name, dtype)


def _rank(t: torch.Tensor, nd: int, name: str, dtype=None):
    if t.dim() != nd:
        raise ValueError(f"{name}: expected {nd} dimensions, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


# ---------------------------------------------------------------- stages
def twotap_conv(x: torch.Tensor, k0: torch.Tensor, k1: torch.Tensor,
                anchor_h: Optional[torch.Tensor] = None, proj: Optional[torch.Tensor] = None,
                groups: int = 1, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = two-tap conv of x [B, L, H] (bf16 or fp32); see dflash2_twotap_conv."""
    B, L, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _shape(out, x.shape, "out", x.dtype)
    _shape(k0, (H,), "k0", torch.float32)
    _shape(k1, (H,), "k1", torch.float32)
    if anchor_h is not None:
        _shape(anchor_h, (B, H), "anchor_h", x.dtype)
    if proj is not None:
        _shape(proj, (H, 2 * groups), "proj", torch.float32)
    dev = _dev(x, k0, k1, anchor_h, proj, out)
    _check("dflash2_twotap_conv", lib().dflash2_twotap_conv(
        _ptr(x), _ptr(anchor_h), _ptr(out), _ptr(k0), _ptr(k1), _ptr(proj), groups,
        B, L, H, _dt(x), _stream(dev)))
    return out


def twotap_conv_mm(x: torch.Tensor, k0: torch.Tensor, k1: torch.Tensor, projT: torch.Tensor,
                   anchor_h: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Two-tap conv with one correction pair per group computed on the matrix
    cores: projT [2 * groups, H] bf16; see dflash2_twotap_conv_mm."""
    B, L, H = x.shape
    if projT.dim() != 2 or projT.shape[1] != H or projT.shape[0] % 2:
        raise ValueError(f"projT: expected [2 * groups, {H}], got {tuple(projT.shape)}")
    groups = projT.shape[0] // 2
    if out is None:
        out = torch.empty_like(x)
    _shape(out, x.shape, "out", x.dtype)
    _shape(k0, (H,), "k0", torch.float32)
    _shape(k1, (H,), "k1", torch.float32)
    _shape(projT, (2 * groups, H), "projT", x.dtype)
    if anchor_h is not None:
        _shape(anchor_h, (B, H), "anchor_h", x.dtype)
    dev = _dev(x, k0, k1, anchor_h, projT, out)
    _check("dflash2_twotap_conv_mm", lib().dflash2_twotap_conv_mm(
        _ptr(x), _ptr(anchor_h), _ptr(out), _ptr(k0), _ptr(k1), _ptr(projT), groups,
        B, L, H, _dt(x), _stream(dev)))
    return out


class PackedWeight:
    """An LM-head weight [V, H] bf16 in the bf16 GEMM's tile layout
    (dflash2_lmhead_pack): `data` holds the packed bytes.  The LM-head calls
    take it wherever they take W, with bit-identical logits."""

    def __init__(self, data: torch.Tensor, V: int, H: int):
        self.data, self.V, self.H = data, V, H
        self.dtype = torch.bfloat16
        self.device = data.device
        self.shape = (V, H)


def lmhead_pack(W: torch.Tensor) -> PackedWeight:
    """Copy W [V, H] bf16 into the GEMM's tile layout (one launch)."""
    if W.dim() != 2 or W.dtype != torch.bfloat16:
        raise TypeError("W must be a 2-D bf16 tensor")
    V, H = W.shape
    n = int(lib().dflash2_lmhead_pack_bytes(V, H))
    if n == 0:
        raise ValueError(f"no packed layout for V={V}, H={H}")
    data = torch.empty(n, dtype=torch.uint8, device=W.device)
    dev = _dev(W, data)
    _check("dflash2_lmhead_pack", lib().dflash2_lmhead_pack(
        _ptr(W), _ptr(data), V, H, _stream(dev)))
    return PackedWeight(data, V, H)


def _weight(W, h: torch.Tensor):
    """(pointer, V, dtype code, tensor) of an LM-head weight for h [M, H]."""
    H = h.shape[1]
    if isinstance(W, PackedWeight):
        if h.dtype != torch.bfloat16 or W.H != H:
            raise ValueError(f"packed W is bf16 [{W.V}, {W.H}]; h is {h.dtype} [*, {H}]")
        return W.data.data_ptr(), W.V, 2, W.data
    V = W.shape[0]
    _shape(W, (V, H), "W", h.dtype)
    return W.data_ptr(), V, _dt(h), W


def lmhead_logits(h: torch.Tensor, W, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """logits [M, V] fp32 = h [M, H] . W [V, H]^T (W a tensor or a PackedWeight)."""
    M, H = h.shape
    wp, V, code, wt = _weight(W, h)
    if out is None:
        out = torch.empty((M, V), dtype=torch.float32, device=h.device)
    _shape(out, (M, V), "out", torch.float32)
    dev = _dev(h, wt, out)
    _check("dflash2_lmhead_logits", lib().dflash2_lmhead_logits(
        _ptr(h), wp, _ptr(out), M, H, V, code, _stream(dev)))
    return out


TILEMAX_COLS = 256


def lmhead_logits_tilemax(h: torch.Tensor, W, out: Optional[torch.Tensor] = None,
                          tilemax: Optional[torch.Tensor] = None):
    """Logits [M, V] and their 256-column tile maxima [M, ceil(V / 256)]."""
    M, H = h.shape
    wp, V, code, wt = _weight(W, h)
    nt = (V + TILEMAX_COLS - 1) // TILEMAX_COLS
    if out is None:
        out = torch.empty((M, V), dtype=torch.float32, device=h.device)
    if tilemax is None:
        tilemax = torch.empty((M, nt), dtype=torch.float32, device=h.device)
    _shape(out, (M, V), "logits", torch.float32)
    _shape(tilemax, (M, nt), "tilemax", torch.float32)
    dev = _dev(h, wt, out, tilemax)
    _check("dflash2_lmhead_logits_tilemax", lib().dflash2_lmhead_logits_tilemax(
        _ptr(h), wp, _ptr(out), _ptr(tilemax), M, H, V, code, _stream(dev)))
    return out, tilemax


def topk16_tilemax(logits: torch.Tensor, tilemax: torch.Tensor, top_val=None, top_idx=None):
    """Top-16 of logits [M, V] that reads only the tiles its maxima allow."""
    _rank(logits, 2, "logits", torch.float32)
    M, V = logits.shape
    _shape(tilemax, (M, (V + TILEMAX_COLS - 1) // TILEMAX_COLS), "tilemax", torch.float32)
    _opt(top_val, (M, TOPK), "top_val", torch.float32)
    _opt(top_idx, (M, TOPK), "top_idx", torch.int32)
    dev = logits.device
    if top_val is None:
        top_val = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    if top_idx is None:
        top_idx = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    _dev(logits, tilemax, top_val, top_idx)
    _check("dflash2_topk16_tilemax", lib().dflash2_topk16_tilemax(
        _ptr(logits), _ptr(tilemax), _ptr(top_val), _ptr(top_idx), M, V, TOPK, _stream(dev)))
    return top_val, top_idx


def topk16_workspace(M: int, V: int) -> int:
    return int(lib().dflash2_topk16_workspace(M, V, TOPK))


def _workspace(nbytes: int, dev, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace smaller than {nbytes} bytes")
    return ws


def topk16(logits: torch.Tensor, top_val: Optional[torch.Tensor] = None,
           top_idx: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-row top-16 (value desc, id asc) of fp32 logits [M, V]."""
    _rank(logits, 2, "logits", torch.float32)
    M, V = logits.shape
    dev = logits.device
    if top_val is None:
        top_val = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    if top_idx is None:
        top_idx = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    _shape(top_val, (M, TOPK), "top_val", torch.float32)
    _shape(top_idx, (M, TOPK), "top_idx", torch.int32)
    need = topk16_workspace(M, V)
    ws = _workspace(need, dev, workspace)
    _dev(logits, top_val, top_idx, ws)
    _check("dflash2_topk16", lib().dflash2_topk16(
        _ptr(logits), _ptr(top_val), _ptr(top_idx), M, V, TOPK, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(dev)))
    return top_val, top_idx


def logits_topk_workspace(M: int, H: int, V: int, dtype: torch.dtype, logits_given: bool) -> int:
    return int(lib().dflash2_logits_topk_workspace(
        M, H, V, TOPK, 1 if dtype == torch.bfloat16 else 0, int(bool(logits_given))))


def logits_topk(h: torch.Tensor, W, logits: Optional[torch.Tensor] = None,
                top_val: Optional[torch.Tensor] = None, top_idx: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None):
    """LM-head logits (into `logits` when given, else into the workspace) and
    the per-row top-16.  Returns (top_val, top_idx)."""
    _rank(h, 2, "h")
    M, H = h.shape
    wp, V, code, wt = _weight(W, h)
    dev = h.device
    _opt(logits, (M, V), "logits", torch.float32)
    _opt(top_val, (M, TOPK), "top_val", torch.float32)
    _opt(top_idx, (M, TOPK), "top_idx", torch.int32)
    if top_val is None:
        top_val = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    if top_idx is None:
        top_idx = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    need = logits_topk_workspace(M, H, V, h.dtype, logits is not None)
    ws = _workspace(need, dev, workspace)
    _dev(h, wt, logits, top_val, top_idx, ws)
    _check("dflash2_logits_topk", lib().dflash2_logits_topk(
        _ptr(h), wp, _ptr(logits), _ptr(top_val), _ptr(top_idx), M, H, V, TOPK, code,
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(dev)))
    return top_val, top_idx


def lmhead_candidates(h: torch.Tensor, W, workspace: torch.Tensor) -> torch.Tensor:
    """The GEMM of logits_topk without a logits buffer (bf16 h; W a tensor or
    a PackedWeight): its candidate form into `workspace`
    (logits_topk_workspace(M, H, V, bf16, False) bytes).  Returns workspace."""
    _rank(h, 2, "h")
    M, H = h.shape
    wp, V, code, wt = _weight(W, h)
    if h.dtype != torch.bfloat16:
        raise TypeError("the candidate form takes bf16 operands")
    ws = _workspace(logits_topk_workspace(M, H, V, h.dtype, False), h.device, workspace)
    _dev(h, wt, ws)
    _check("dflash2_lmhead_candidates", lib().dflash2_lmhead_candidates(
        _ptr(h), wp, M, H, V, code, _ptr(ws), ws.numel() * ws.element_size(), _stream(h.device)))
    return ws


def topk16_candidates(workspace: torch.Tensor, M: int, H: int, V: int,
                      top_val: Optional[torch.Tensor] = None,
                      top_idx: Optional[torch.Tensor] = None):
    """The top-16 of logits_topk without a logits buffer, from the workspace
    lmhead_candidates filled for the same M, H, V.  Returns (top_val, top_idx)."""
    dev = workspace.device
    _opt(top_val, (M, TOPK), "top_val", torch.float32)
    _opt(top_idx, (M, TOPK), "top_idx", torch.int32)
    if top_val is None:
        top_val = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    if top_idx is None:
        top_idx = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    _dev(workspace, top_val, top_idx)
    _check("dflash2_topk16_candidates", lib().dflash2_topk16_candidates(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(top_val),
        _ptr(top_idx), M, H, V, TOPK, _stream(dev)))
    return top_val, top_idx


def logits_topk_noalloc(h: torch.Tensor, W, logits: torch.Tensor,
                        top_val: torch.Tensor, top_idx: torch.Tensor):
    """logits_topk without a workspace, for callers that cannot allocate:
    the tile maxima live in the library's fixed device scratch (shared by
    every call on one GPU; overlapping calls on one GPU race).  Every output
    is caller-given.  Returns (top_val, top_idx)."""
    _rank(h, 2, "h")
    M, H = h.shape
    wp, V, code, wt = _weight(W, h)
    _shape(logits, (M, V), "logits", torch.float32)
    _shape(top_val, (M, TOPK), "top_val", torch.float32)
    _shape(top_idx, (M, TOPK), "top_idx", torch.int32)
    dev = _dev(h, wt, logits, top_val, top_idx)
    _check("dflash2_logits_topk_noalloc", lib().dflash2_logits_topk_noalloc(
        _ptr(h), wp, _ptr(logits), _ptr(top_val), _ptr(top_idx), M, H, V, TOPK, code,
        _stream(dev)))
    return top_val, top_idx


def probe_mfma(operands: torch.Tensor, workgroups: int, iters: int,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Measurement aid (not a step): the GEMM's matrix-core work without its
    memory traffic, `workgroups` x 8 waves x `iters` x 8 bf16 32x32x16
    MFMAs on register operands loaded once from `operands` (uint8 or bf16
    bits, probe_mfma_operand_bytes(workgroups) bytes).  Returns out
    [workgroups * 512] fp32."""
    need = int(lib().dflash2_probe_mfma_operand_bytes(workgroups))
    if operands.numel() * operands.element_size() < need:
        raise ValueError(f"operands: need {need} bytes")
    if out is None:
        out = torch.empty(workgroups * 512, dtype=torch.float32, device=operands.device)
    _shape(out, (workgroups * 512,), "out", torch.float32)
    dev = _dev(operands, out)
    _check("dflash2_probe_mfma", lib().dflash2_probe_mfma(
        _ptr(operands), workgroups, iters, _ptr(out), _stream(dev)))
    return out


def probe_mfma_operand_bytes(workgroups: int) -> int:
    return int(lib().dflash2_probe_mfma_operand_bytes(workgroups))


def context_gate(h: torch.Tensor, Wg: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Context gate sigmoid(h . Wg^T): h [M, H], Wg [r, H] -> fp32 [M, r]."""
    M, H = h.shape
    r = Wg.shape[0]
    _shape(Wg, (r, H), "Wg", h.dtype)
    if out is None:
        out = torch.empty((M, r), dtype=torch.float32, device=h.device)
    _shape(out, (M, r), "gate", torch.float32)
    dev = _dev(h, Wg, out)
    _check("dflash2_context_gate", lib().dflash2_context_gate(
        _ptr(h), _ptr(Wg), _ptr(out), M, H, r, _dt(h), _stream(dev)))
    return out


def pair_score(top_val: torch.Tensor, top_idx: torch.Tensor, anchor_tok: Optional[torch.Tensor],
               U: torch.Tensor, Vf: torch.Tensor, S0: Optional[torch.Tensor] = None,
               S: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None):
    """S0 [B, 16], S [B, L-1, 16, 16] from candidates [B, L, 16] and factors
    [V, r]; with `gate` ([B, L, r] or [B*L, r] fp32) the gated scores."""
    _rank(top_val, 3, "top_val", torch.float32)
    _rank(U, 2, "U")
    B, L, K = top_val.shape
    V, r = U.shape
    _shape(top_val, (B, L, TOPK), "top_val", torch.float32)
    _shape(top_idx, (B, L, K), "top_idx", torch.int32)
    _shape(Vf, (V, r), "Vf", U.dtype)
    if anchor_tok is not None:
        _shape(anchor_tok, (B,), "anchor_tok", torch.int32)
    if gate is not None:
        if gate.dim() == 2:
            gate = gate.view(B, L, r) if gate.shape[0] == B * L else gate
        _shape(gate, (B, L, r), "gate", torch.float32)
    dev = top_val.device
    if S0 is None:
        S0 = torch.empty((B, TOPK), dtype=torch.float32, device=dev)
    if S is None:
        S = torch.empty((B, max(L - 1, 0), TOPK, TOPK), dtype=torch.float32, device=dev)
    _shape(S0, (B, TOPK), "S0", torch.float32)
    _shape(S, (B, L - 1, TOPK, TOPK), "S", torch.float32)
    _dev(top_val, top_idx, anchor_tok, U, Vf, S0, S, gate)
    if gate is None:
        _check("dflash2_pair_score", lib().dflash2_pair_score(
            _ptr(top_val), _ptr(top_idx), _ptr(anchor_tok), _ptr(U), _ptr(Vf), B, L, V, r,
            _dt(U), _ptr(S0), _ptr(S) if L > 1 else None, _stream(dev)))
    else:
        _check("dflash2_pair_score_gated", lib().dflash2_pair_score_gated(
            _ptr(top_val), _ptr(top_idx), _ptr(anchor_tok), _ptr(U), _ptr(Vf), _ptr(gate), B, L,
            V, r, _dt(U), _ptr(S0), _ptr(S) if L > 1 else None, _stream(dev)))
    return S0, S


def path_select(S0: torch.Tensor, S: Optional[torch.Tensor], top_idx: Optional[torch.Tensor],
                path_slot=None, path_tok=None, path_score=None, mode: str = "viterbi"):
    """Best path per block: max-plus ("viterbi") or best-successor ("greedy").
    Returns (path_slot, path_tok, path_score)."""
    if mode not in PATH_MODES:
        raise ValueError(f"mode must be one of {sorted(PATH_MODES)}, got {mode!r}")
    _rank(S0, 2, "S0", torch.float32)
    B = S0.shape[0]
    if top_idx is not None:
        _rank(top_idx, 3, "top_idx", torch.int32)
        L = top_idx.shape[1]
    else:
        L = 1 if S is None else S.shape[1] + 1
    _shape(S0, (B, TOPK), "S0", torch.float32)
    _opt(top_idx, (B, L, TOPK), "top_idx", torch.int32)
    if L > 1:
        if S is None:
            raise ValueError("S: the scores are needed for L > 1")
        _shape(S, (B, L - 1, TOPK, TOPK), "S", torch.float32)
    _opt(path_slot, (B, L), "path_slot", torch.int32)
    _opt(path_tok, (B, L), "path_tok", torch.int32)
    _opt(path_score, (B,), "path_score", torch.float32)
    dev = S0.device
    if path_slot is None:
        path_slot = torch.empty((B, L), dtype=torch.int32, device=dev)
    if path_tok is None and top_idx is not None:
        path_tok = torch.empty((B, L), dtype=torch.int32, device=dev)
    if path_score is None:
        path_score = torch.empty((B,), dtype=torch.float32, device=dev)
    _dev(S0, S, top_idx, path_slot, path_tok, path_score)
    _check("dflash2_path_select_mode", lib().dflash2_path_select_mode(
        _ptr(S0), _ptr(S) if L > 1 else None, _ptr(top_idx), B, L, PATH_MODES[mode],
        _ptr(path_slot), _ptr(path_tok), _ptr(path_score), _stream(dev)))
    return path_slot, path_tok, path_score


def verify_greedy(path_tok: torch.Tensor, target: torch.Tensor, accept_len=None, next_tok=None):
    """Greedy verification: (accept_len [B], next_tok [B])."""
    _rank(path_tok, 2, "path_tok", torch.int32)
    B, L = path_tok.shape
    _shape(target, (B, L + 1), "target", torch.int32)
    _opt(accept_len, (B,), "accept_len", torch.int32)
    _opt(next_tok, (B,), "next_tok", torch.int32)
    dev = path_tok.device
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(path_tok, target, accept_len, next_tok)
    _check("dflash2_verify_greedy", lib().dflash2_verify_greedy(
        _ptr(path_tok), _ptr(target), B, L, _ptr(accept_len), _ptr(next_tok), _stream(dev)))
    return accept_len, next_tok


def pair_select_verify(top_val: torch.Tensor, top_idx: torch.Tensor,
                       anchor_tok: Optional[torch.Tensor], U: torch.Tensor, Vf: torch.Tensor,
                       target: torch.Tensor, gate: Optional[torch.Tensor] = None,
                       mode: str = "viterbi", S0: Optional[torch.Tensor] = None,
                       S: Optional[torch.Tensor] = None, path_slot=None, path_tok=None,
                       path_score=None, accept_len=None, next_tok=None):
    """pair_score, path_select and verify_greedy in one launch.  The scores
    are written to S0 / S only when those are given.  Returns (path_slot,
    path_tok, path_score, accept_len, next_tok)."""
    if mode not in PATH_MODES:
        raise ValueError(f"mode must be one of {sorted(PATH_MODES)}, got {mode!r}")
    _rank(top_val, 3, "top_val", torch.float32)
    _rank(U, 2, "U")
    B, L, K = top_val.shape
    V, r = U.shape
    _shape(top_val, (B, L, TOPK), "top_val", torch.float32)
    _shape(top_idx, (B, L, K), "top_idx", torch.int32)
    _shape(Vf, (V, r), "Vf", U.dtype)
    _shape(target, (B, L + 1), "target", torch.int32)
    _opt(path_slot, (B, L), "path_slot", torch.int32)
    _opt(path_tok, (B, L), "path_tok", torch.int32)
    _opt(path_score, (B,), "path_score", torch.float32)
    _opt(accept_len, (B,), "accept_len", torch.int32)
    _opt(next_tok, (B,), "next_tok", torch.int32)
    if anchor_tok is not None:
        _shape(anchor_tok, (B,), "anchor_tok", torch.int32)
    if gate is not None:
        if gate.dim() == 2 and gate.shape[0] == B * L:
            gate = gate.view(B, L, r)
        _shape(gate, (B, L, r), "gate", torch.float32)
    if S0 is not None:
        _shape(S0, (B, TOPK), "S0", torch.float32)
    if S is not None:
        _shape(S, (B, L - 1, TOPK, TOPK), "S", torch.float32)
    dev = top_val.device
    if path_slot is None:
        path_slot = torch.empty((B, L), dtype=torch.int32, device=dev)
    if path_tok is None:
        path_tok = torch.empty((B, L), dtype=torch.int32, device=dev)
    if path_score is None:
        path_score = torch.empty((B,), dtype=torch.float32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(top_val, top_idx, anchor_tok, U, Vf, target, gate, S0, S, path_slot, path_tok,
         path_score, accept_len, next_tok)
    _check("dflash2_pair_select_verify", lib().dflash2_pair_select_verify(
        _ptr(top_val), _ptr(top_idx), _ptr(anchor_tok), _ptr(U), _ptr(Vf), _ptr(gate),
        _ptr(target), B, L, V, r, _dt(U), PATH_MODES[mode], _ptr(S0),
        _ptr(S) if L > 1 else None, _ptr(path_slot), _ptr(path_tok), _ptr(path_score),
        _ptr(accept_len), _ptr(next_tok), _stream(dev)))
    return path_slot, path_tok, path_score, accept_len, next_tok


def pair_sample(top_val: torch.Tensor, top_idx: torch.Tensor, anchor_tok: Optional[torch.Tensor],
                U: torch.Tensor, Vf: torch.Tensor, u: torch.Tensor, temperature: float,
                gate: Optional[torch.Tensor] = None, S0: Optional[torch.Tensor] = None,
                S: Optional[torch.Tensor] = None, path_slot=None, path_tok=None, q=None,
                mode: str = "chain"):
    """pair_score and path_sample in one launch.  The scores are written to
    S0 / S only when those are given.  mode "chain" draws each position from
    its predecessor's row, "path" the whole path from exp(score / T).
    Returns (path_slot, path_tok, q)."""
    if mode not in SAMPLE_MODES:
        raise ValueError(f"mode must be one of {sorted(SAMPLE_MODES)}, got {mode!r}")
    _rank(top_val, 3, "top_val", torch.float32)
    _rank(U, 2, "U")
    B, L, K = top_val.shape
    V, r = U.shape
    _shape(top_val, (B, L, TOPK), "top_val", torch.float32)
    _shape(top_idx, (B, L, K), "top_idx", torch.int32)
    _shape(Vf, (V, r), "Vf", U.dtype)
    _shape(u, (B, L), "u", torch.float32)
    _opt(path_slot, (B, L), "path_slot", torch.int32)
    _opt(path_tok, (B, L), "path_tok", torch.int32)
    _opt(q, (B, L, TOPK), "q", torch.float32)
    if anchor_tok is not None:
        _shape(anchor_tok, (B,), "anchor_tok", torch.int32)
    if gate is not None:
        if gate.dim() == 2 and gate.shape[0] == B * L:
            gate = gate.view(B, L, r)
        _shape(gate, (B, L, r), "gate", torch.float32)
    if S0 is not None:
        _shape(S0, (B, TOPK), "S0", torch.float32)
    if S is not None:
        _shape(S, (B, L - 1, TOPK, TOPK), "S", torch.float32)
    dev = top_val.device
    if path_slot is None:
        path_slot = torch.empty((B, L), dtype=torch.int32, device=dev)
    if path_tok is None:
        path_tok = torch.empty((B, L), dtype=torch.int32, device=dev)
    if q is None:
        q = torch.empty((B, L, TOPK), dtype=torch.float32, device=dev)
    _dev(top_val, top_idx, anchor_tok, U, Vf, u, gate, S0, S, path_slot, path_tok, q)
    _check("dflash2_pair_sample_mode", lib().dflash2_pair_sample_mode(
        _ptr(top_val), _ptr(top_idx), _ptr(anchor_tok), _ptr(U), _ptr(Vf), _ptr(gate), _ptr(u),
        float(temperature), B, L, V, r, _dt(U), SAMPLE_MODES[mode], _ptr(S0),
        _ptr(S) if L > 1 else None, _ptr(path_slot), _ptr(path_tok), _ptr(q), _stream(dev)))
    return path_slot, path_tok, q


def path_sample(S0: torch.Tensor, S: Optional[torch.Tensor], top_idx: Optional[torch.Tensor],
                u: torch.Tensor, temperature: float, path_slot=None, path_tok=None, q=None,
                mode: str = "chain"):
    """Sampling walk at temperature T with uniforms u [B, L]: mode "chain"
    draws each position from its predecessor's row, "path" the whole path
    from exp(score / T).  Returns (path_slot, path_tok, q [B, L, 16])."""
    if mode not in SAMPLE_MODES:
        raise ValueError(f"mode must be one of {sorted(SAMPLE_MODES)}, got {mode!r}")
    _rank(S0, 2, "S0", torch.float32)
    _rank(u, 2, "u", torch.float32)
    B = S0.shape[0]
    L = u.shape[1]
    _shape(S0, (B, TOPK), "S0", torch.float32)
    _shape(u, (B, L), "u", torch.float32)
    if L > 1:
        if S is None:
            raise ValueError("S: the scores are needed for L > 1")
        _shape(S, (B, L - 1, TOPK, TOPK), "S", torch.float32)
    _opt(top_idx, (B, L, TOPK), "top_idx", torch.int32)
    _opt(path_slot, (B, L), "path_slot", torch.int32)
    _opt(path_tok, (B, L), "path_tok", torch.int32)
    _opt(q, (B, L, TOPK), "q", torch.float32)
    dev = S0.device
    if path_slot is None:
        path_slot = torch.empty((B, L), dtype=torch.int32, device=dev)
    if path_tok is None and top_idx is not None:
        path_tok = torch.empty((B, L), dtype=torch.int32, device=dev)
    if q is None:
        q = torch.empty((B, L, TOPK), dtype=torch.float32, device=dev)
    _dev(S0, S, top_idx, u, path_slot, path_tok, q)
    _check("dflash2_path_sample_mode", lib().dflash2_path_sample_mode(
        _ptr(S0), _ptr(S) if L > 1 else None, _ptr(top_idx), _ptr(u), float(temperature), B, L,
        SAMPLE_MODES[mode], _ptr(path_slot), _ptr(path_tok), _ptr(q), _stream(dev)))
    return path_slot, path_tok, q


def target_lse(z: torch.Tensor, temperature: float, out: Optional[torch.Tensor] = None):
    """log sum exp(z / T) over the last axis of fp32 target logits."""
    if z.dtype != torch.float32 or z.dim() < 1:
        raise TypeError(f"z: expected fp32 logits, got {z.dtype} of shape {tuple(z.shape)}")
    V = z.shape[-1]
    R = z.numel() // V
    if out is None:
        out = torch.empty(z.shape[:-1], dtype=torch.float32, device=z.device)
    if out.numel() != R or out.dtype != torch.float32:
        raise ValueError("lse: expected one fp32 value per row")
    dev = _dev(z, out)
    _check("dflash2_target_lse", lib().dflash2_target_lse(
        _ptr(z), R, V, float(temperature), _ptr(out), _stream(dev)))
    return out


def verify_rejection(path_slot: torch.Tensor, path_tok: torch.Tensor, q: torch.Tensor,
                     top_idx: torch.Tensor, z: torch.Tensor, lse: torch.Tensor,
                     temperature: float, u_acc: torch.Tensor, u_res: torch.Tensor,
                     accept_len=None, next_tok=None):
    """Speculative-sampling verification: (accept_len [B], next_tok [B])."""
    _rank(path_tok, 2, "path_tok", torch.int32)
    B, L = path_tok.shape
    V = z.shape[-1]
    _shape(path_slot, (B, L), "path_slot", torch.int32)
    _shape(q, (B, L, TOPK), "q", torch.float32)
    _shape(top_idx, (B, L, TOPK), "top_idx", torch.int32)
    _shape(z, (B, L + 1, V), "z", torch.float32)
    _shape(lse, (B, L + 1), "lse", torch.float32)
    _shape(u_acc, (B, L), "u_acc", torch.float32)
    _shape(u_res, (B,), "u_res", torch.float32)
    _opt(accept_len, (B,), "accept_len", torch.int32)
    _opt(next_tok, (B,), "next_tok", torch.int32)
    dev = path_tok.device
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(path_slot, path_tok, q, top_idx, z, lse, u_acc, u_res, accept_len, next_tok)
    _check("dflash2_verify_rejection", lib().dflash2_verify_rejection(
        _ptr(path_slot), _ptr(path_tok), _ptr(q), _ptr(top_idx), _ptr(z), _ptr(lse),
        float(temperature), _ptr(u_acc), _ptr(u_res), B, L, V, _ptr(accept_len), _ptr(next_tok),
        _stream(dev)))
    return accept_len, next_tok


def verify_rejection_lazy(path_slot: torch.Tensor, path_tok: torch.Tensor, q: torch.Tensor,
                          top_idx: torch.Tensor, z: torch.Tensor, temperature: float,
                          u_acc: torch.Tensor, u_res: torch.Tensor, accept_len=None,
                          next_tok=None):
    """verify_rejection that computes each row's log-sum-exp itself, only for
    the rows the accept test reaches: (accept_len [B], next_tok [B])."""
    _rank(path_tok, 2, "path_tok", torch.int32)
    B, L = path_tok.shape
    V = z.shape[-1]
    _shape(path_slot, (B, L), "path_slot", torch.int32)
    _shape(q, (B, L, TOPK), "q", torch.float32)
    _shape(top_idx, (B, L, TOPK), "top_idx", torch.int32)
    _shape(z, (B, L + 1, V), "z", torch.float32)
    _shape(u_acc, (B, L), "u_acc", torch.float32)
    _shape(u_res, (B,), "u_res", torch.float32)
    _opt(accept_len, (B,), "accept_len", torch.int32)
    _opt(next_tok, (B,), "next_tok", torch.int32)
    dev = path_tok.device
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(path_slot, path_tok, q, top_idx, z, u_acc, u_res, accept_len, next_tok)
    _check("dflash2_verify_rejection_lazy", lib().dflash2_verify_rejection_lazy(
        _ptr(path_slot), _ptr(path_tok), _ptr(q), _ptr(top_idx), _ptr(z), float(temperature),
        _ptr(u_acc), _ptr(u_res), B, L, V, _ptr(accept_len), _ptr(next_tok), _stream(dev)))
    return accept_len, next_tok


STAGED_ROWS = 2   # target rows per block the staged verification sums up front


def verify_rejection_staged_workspace(B: int, L: int, V: int, rows: int = STAGED_ROWS) -> int:
    return int(lib().dflash2_verify_rejection_staged_workspace(B, L, V, rows))


def verify_rejection_staged(path_slot: torch.Tensor, path_tok: torch.Tensor, q: torch.Tensor,
                            top_idx: torch.Tensor, z: torch.Tensor, temperature: float,
                            u_acc: torch.Tensor, u_res: torch.Tensor, accept_len=None,
                            next_tok=None, rows: Optional[int] = None,
                            workspace: Optional[torch.Tensor] = None):
    """verify_rejection_lazy with the first `rows` target rows of every block
    (default min(2, L + 1)) summed up front, all blocks at once; the same
    (accept_len [B], next_tok [B]) bit for bit."""
    _rank(path_tok, 2, "path_tok", torch.int32)
    B, L = path_tok.shape
    V = z.shape[-1]
    rows = min(STAGED_ROWS, L + 1) if rows is None else int(rows)
    _shape(path_slot, (B, L), "path_slot", torch.int32)
    _shape(q, (B, L, TOPK), "q", torch.float32)
    _shape(top_idx, (B, L, TOPK), "top_idx", torch.int32)
    _shape(z, (B, L + 1, V), "z", torch.float32)
    _shape(u_acc, (B, L), "u_acc", torch.float32)
    _shape(u_res, (B,), "u_res", torch.float32)
    _opt(accept_len, (B,), "accept_len", torch.int32)
    _opt(next_tok, (B,), "next_tok", torch.int32)
    dev = path_tok.device
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    need = verify_rejection_staged_workspace(B, L, V, rows) if 1 <= rows <= L + 1 else 0
    ws = _workspace(need, dev, workspace)
    _dev(path_slot, path_tok, q, top_idx, z, u_acc, u_res, accept_len, next_tok,
         *([ws] if ws is not None else []))
    _check("dflash2_verify_rejection_staged", lib().dflash2_verify_rejection_staged(
        _ptr(path_slot), _ptr(path_tok), _ptr(q), _ptr(top_idx), _ptr(z), float(temperature),
        _ptr(u_acc), _ptr(u_res), B, L, V, rows, _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _ptr(accept_len),
        _ptr(next_tok), _stream(dev)))
    return accept_len, next_tok


# ---------------------------------------------------------------- whole step
class StepBuffers:
    """Preallocated device buffers for one step shape (B, L, H, V) so repeated
    steps allocate nothing.  `keep_logits` materialises the [M, V] logits in
    their own tensor (else they live in the workspace)."""

    def __init__(self, B: int, L: int, H: int, V: int, dtype: torch.dtype, device,
                 n_convs: int = 1, keep_logits: bool = True, gate_rank: int = 0,
                 sample: bool = False):
        M = B * L
        kw = dict(device=device)
        self.B, self.L, self.H, self.V = B, L, H, V
        self.y = [torch.empty((B, L, H), dtype=dtype, **kw) for _ in range(min(n_convs, 2))]
        self.logits = torch.empty((M, V), dtype=torch.float32, **kw) if keep_logits else None
        ws = logits_topk_workspace(M, H, V, dtype, keep_logits)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, **kw)
        self.top_val = torch.empty((M, TOPK), dtype=torch.float32, **kw)
        self.top_idx = torch.empty((M, TOPK), dtype=torch.int32, **kw)
        self.S0 = torch.empty((B, TOPK), dtype=torch.float32, **kw)
        self.S = torch.empty((B, max(L - 1, 0), TOPK, TOPK), dtype=torch.float32, **kw)
        self.path_slot = torch.empty((B, L), dtype=torch.int32, **kw)
        self.path_tok = torch.empty((B, L), dtype=torch.int32, **kw)
        self.path_score = torch.empty((B,), dtype=torch.float32, **kw)
        self.accept_len = torch.empty((B,), dtype=torch.int32, **kw)
        self.next_tok = torch.empty((B,), dtype=torch.int32, **kw)
        self.gate = (torch.empty((M, gate_rank), dtype=torch.float32, **kw)
                     if gate_rank else None)
        self.q = torch.empty((B, L, TOPK), dtype=torch.float32, **kw) if sample else None
        self.lse = torch.empty((B, L + 1), dtype=torch.float32, **kw) if sample else None
        sw = verify_rejection_staged_workspace(B, L, V, min(STAGED_ROWS, L + 1)) if sample else 0
        self.staged = torch.empty(max(sw, 1), dtype=torch.uint8, **kw) if sample else None


def run_step(buf: StepBuffers, x: torch.Tensor, convs, W, U: torch.Tensor,
             Vf: torch.Tensor, anchor_tok: Optional[torch.Tensor],
             target: Optional[torch.Tensor], Wg: Optional[torch.Tensor] = None,
             walk: str = "viterbi", temperature: float = 0.0,
             u_path: Optional[torch.Tensor] = None, z_target: Optional[torch.Tensor] = None,
             u_acc: Optional[torch.Tensor] = None,
             u_res: Optional[torch.Tensor] = None) -> StepBuffers:
    """One draft-select-verify step: the conv chain (each entry of `convs` is a
    dict with k0, k1, anchor_h and either proj + groups, or projT for the
    matrix-core corrections), logits + top-16 (W a tensor or a PackedWeight),
    pair scores
    (context-gated from the final hidden states when `Wg` is given), the path
    walk (`walk`: "viterbi", "greedy", "sample" (each position from its
    predecessor's row) or "sample-path" (the whole path from exp(score / T))
    at `temperature` with the uniforms `u_path`) and verification: greedy against `target` argmax ids,
    or, for a sampled walk given target logits `z_target` [B, L+1, V], the
    lossless rejection rule with uniforms `u_acc`, `u_res` (the first two target
    rows of every block summed up front, further rows only where the accept
    test reaches them).  A walk that is
    not sampled, with targets given, runs scores, walk and verification in
    one launch (pair_select_verify); a sampled walk runs scores and walk in
    one launch (pair_sample).  Every call is enqueued on the current
    stream; nothing is synchronised."""
    B, L, H, V = buf.B, buf.L, buf.H, buf.V
    cur = x
    for j, c in enumerate(convs):
        out = buf.y[j % len(buf.y)]
        if c.get("projT") is not None:
            twotap_conv_mm(cur, c["k0"], c["k1"], c["projT"], c.get("anchor_h"), out=out)
        else:
            twotap_conv(cur, c["k0"], c["k1"], c.get("anchor_h"), c.get("proj"),
                        c.get("groups", 1), out=out)
        cur = out
    M = B * L
    logits_topk(cur.view(M, H), W, buf.logits, buf.top_val, buf.top_idx, buf.workspace)
    tv = buf.top_val.view(B, L, TOPK)
    ti = buf.top_idx.view(B, L, TOPK)
    gate = None
    if Wg is not None:
        if buf.gate is None:
            raise ValueError("StepBuffers were made without gate_rank")
        gate = context_gate(cur.view(M, H), Wg, buf.gate)
    sampled = walk in ("sample", "sample-path")
    smode = "path" if walk == "sample-path" else "chain"
    if not sampled and target is not None:
        pair_select_verify(tv, ti, anchor_tok, U, Vf, target, gate, walk, buf.S0, buf.S,
                           buf.path_slot, buf.path_tok, buf.path_score, buf.accept_len,
                           buf.next_tok)
        return buf
    if sampled:
        if buf.q is None or u_path is None:
            raise ValueError("a sampled walk needs StepBuffers(sample=True) and u_path")
        pair_sample(tv, ti, anchor_tok, U, Vf, u_path, temperature, gate, buf.S0, buf.S,
                    buf.path_slot, buf.path_tok, buf.q, mode=smode)
        if z_target is not None:
            verify_rejection_staged(buf.path_slot, buf.path_tok, buf.q, ti, z_target,
                                    temperature, u_acc, u_res, buf.accept_len, buf.next_tok,
                                    workspace=buf.staged)
        return buf
    pair_score(tv, ti, anchor_tok, U, Vf, buf.S0, buf.S, gate=gate)
    path_select(buf.S0, buf.S, ti, buf.path_slot, buf.path_tok, buf.path_score, mode=walk)
    return buf
