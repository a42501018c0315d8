"""Test helpers: move seeded workload arrays to the GPU and back."""
import numpy as np
import torch


def to_dev(a, dtype: str, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) or fp32 / int32 numpy arrays -> device tensor."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.int32 or a.dtype == np.int64:
        return torch.from_numpy(a.astype(np.int32)).to(device)
    return torch.from_numpy(a.astype(np.float32)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns; fp32/int -> numpy."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def convs_to_dev(convs, dtype: str, device="cuda"):
    out = []
    for c in convs:
        out.append({
            "k0": torch.from_numpy(np.ascontiguousarray(c["k0"], np.float32)).to(device),
            "k1": torch.from_numpy(np.ascontiguousarray(c["k1"], np.float32)).to(device),
            "anchor_h": None if c["anchor_h"] is None else to_dev(c["anchor_h"], dtype, device),
            "proj": None if c.get("proj") is None
            else torch.from_numpy(np.ascontiguousarray(c["proj"], np.float32)).to(device),
            "groups": c.get("groups", 1),
            "projT": None if c.get("projT") is None else to_dev(c["projT"], dtype, device),
        })
    return out


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (fp64): 2^(e-8) for v in [2^(e-1), 2^e)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.maximum(v, 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def f32_ulp(v: np.ndarray) -> np.ndarray:
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.maximum(v, 2.0 ** -126))
    return np.ldexp(1.0, e - 24)
