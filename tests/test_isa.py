"""Properties of the generated gfx950 code (CPU: hipcc cross-compiles).

- No kernel uses packed fp32 arithmetic: the build turns the feature off,
  so hipcc never forms those instructions from ordinary float code.
- The ten-channel conv in its split-K mode reads a group's partials from the
  same y rows it then overwrites.  Its workgroup barrier waits for LDS
  operations only, so every partial load must be consumed (its wait issued)
  before the next barrier; otherwise a wave's load could still be in flight
  while other waves store into those rows.
"""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_drafting_amd import build as B  # noqa: E402


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-I", B.INCLUDE, "-I", B.CSRC, "--cuda-device-only",
           "-S", src, "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm():
    try:
        B.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    srcs = sorted(os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(min(8, len(srcs))) as ex:
            texts = list(ex.map(lambda s: _device_asm(s, d), srcs))
    return dict(zip((os.path.basename(s) for s in srcs), texts))


def _kernels(text: str, pattern: str):
    """(symbol, body lines) of every kernel whose symbol matches pattern."""
    lines = text.split("\n")
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S+):", l)
        if m and re.search(pattern, m.group(1)):
            end = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
            yield m.group(1), lines[i:end]


def test_no_packed_fp32(asm):
    pk = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    hits = {name: len(pk.findall(t)) for name, t in asm.items()}
    assert not any(hits.values()), hits


def _sources(line: str):
    """VGPR numbers read by a vector ALU instruction (operands after the first)."""
    ops = line.split(";")[0].split(",")[1:]
    regs = []
    for op in ops:
        for a, b in re.findall(r"v\[(\d+):(\d+)\]", op):
            regs += range(int(a), int(b) + 1)
        regs += [int(x) for x in re.findall(r"(?<![\w\[:])v(\d+)\b", op)]
    return regs


def test_split_conv_partials_consumed_before_barrier(asm):
    kernels = list(_kernels(asm["conv.hip"], r"conv_rows10_kernelILi\d+ELi\d+ELi\d+ELi2E"))
    assert len(kernels) >= 4
    for name, body in kernels:
        text = "\n".join(body)
        # the y descriptor: the one the kernel stores through
        y_rsrc = set(re.findall(r"buffer_store_dword\w*\s+v\S+,\s*v\d+,\s*(s\[\d+:\d+\])", text))
        assert y_rsrc, name
        loads = []
        for i, l in enumerate(body):
            m = re.search(r"buffer_load_dwordx4 v\[(\d+):(\d+)\], v\d+, (s\[\d+:\d+\])", l)
            if m and m.group(3) in y_rsrc:
                loads.append((i, range(int(m.group(1)), int(m.group(2)) + 1)))
        assert loads, name
        barriers = [i for i, l in enumerate(body) if "s_barrier" in l]
        late = []
        for i, regs in loads:
            nxt = next((b for b in barriers if b > i), None)
            if nxt is None:
                continue
            use = next((j for j in range(i + 1, len(body))
                        if body[j].split() and body[j].split()[0].startswith("v_")
                        and any(r in regs for r in _sources(body[j]))), None)
            if use is None or use > nxt:
                late.append(i)
        assert not late, f"{name}: {len(late)} of {len(loads)} partial loads consumed after a barrier"
