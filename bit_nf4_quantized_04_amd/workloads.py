"""Seeded synthetic inputs for the NF4 QLoRA linear layer.

This module only draws random numbers; it holds none of the layer's arithmetic.
Both the HIP path (tests, benchmark) and the CPU oracle consume its output.

Every stream is ``numpy.random.Generator(PCG64(1000*c + t))`` with c the
workload number and t the stream number:

    t=0 W0 (float32)     t=1 x        t=2 A        t=3 B
    t=4 dH               t=5 adapter ids           t=6 outlier mask
    t=7 outlier t-values

x, A, B and dH are drawn in float32 and converted to bfloat16 by torch's CPU
conversion (a library routine); they are returned as uint16 bit patterns.

Workloads (shapes follow the nn.Linear layout: W0 is [out, in]):

1. tiny:        W0 [256, 256] ~ N(0, 0.02^2), no double quant; x [4, 256];
                r=8, alpha=16; A He-uniform, B ~ N(0, 0.01^2).
2. decode:      W0 [4096, 4096] ~ N(0, 0.02^2), double quant; x [M, 4096],
                M in {1, 4, 16}; r=16, alpha=32.
3. 7B MLP:      W0 [11008, 4096] (4096 -> 11008), double quant; x [2048, 4096];
                r=64, alpha=16; dH [2048, 11008].
4. 70B MLP:     W0 [28672, 8192] (8192 -> 28672): with probability 0.001 an
                entry is 0.1 * Student-t(df=3), else N(0, 0.015^2); double
                quant; x [M, 8192], M in {1, 4096}; r=64, alpha=128.
5. multi-adapter: W0 [4096, 4096] ~ N(0, 0.02^2), double quant; 64 adapters
                r=16, alpha=32, A and B ~ N(0, 0.01^2); x [2048, 4096]; ids
                uniform in [0, 64).

He-uniform for A is U(-sqrt(6/in), +sqrt(6/in)) (Kaiming uniform, gain sqrt 2,
fan_in = in).  dH is N(0, 1).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SHAPES = {
    1: dict(out=256, inp=256, dq=False, r=8, alpha=16.0, M=(4,), std=0.02),
    2: dict(out=4096, inp=4096, dq=True, r=16, alpha=32.0, M=(1, 4, 16), std=0.02),
    3: dict(out=11008, inp=4096, dq=True, r=64, alpha=16.0, M=(2048,), std=0.02),
    4: dict(out=28672, inp=8192, dq=True, r=64, alpha=128.0, M=(1, 4096), std=0.015),
    5: dict(out=4096, inp=4096, dq=True, r=16, alpha=32.0, M=(2048,), std=0.02, n_adapters=64),
}


def _rng(c: int, t: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * c + t))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns through torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight(c: int, out: int | None = None, inp: int | None = None) -> np.ndarray:
    """W0 [out, in] float32 for workload ``c`` (shape overridable for small tests)."""
    sh = SHAPES[c]
    out = sh["out"] if out is None else out
    inp = sh["inp"] if inp is None else inp
    g = _rng(c, 0)
    w = g.standard_normal((out, inp), dtype=np.float32)
    w *= np.float32(sh["std"])
    if c == 4:
        mask = _rng(c, 6).random((out, inp), dtype=np.float32) < np.float32(0.001)
        n = int(mask.sum())
        tv = _rng(c, 7).standard_t(3, size=n).astype(np.float32) * np.float32(0.1)
        w[mask] = tv
    return w


def activations(c: int, M: int, inp: int | None = None) -> np.ndarray:
    inp = SHAPES[c]["inp"] if inp is None else inp
    x = _rng(c, 1).standard_normal((M, inp), dtype=np.float32)
    return to_bf16_bits(x)


def adapters(c: int, inp: int | None = None, out: int | None = None, r: int | None = None):
    """(A bits [r, in], B bits [out, r]) for single-adapter workloads 1-4."""
    sh = SHAPES[c]
    inp = sh["inp"] if inp is None else inp
    out = sh["out"] if out is None else out
    r = sh["r"] if r is None else r
    bound = math.sqrt(6.0 / inp)
    a = _rng(c, 2).uniform(-bound, bound, size=(r, inp)).astype(np.float32)
    b = (_rng(c, 3).standard_normal((out, r), dtype=np.float32) * np.float32(0.01))
    return to_bf16_bits(a), to_bf16_bits(b)


def adapter_bank(c: int = 5, n: int | None = None, inp: int | None = None,
                 out: int | None = None, r: int | None = None):
    """(A bank [n, r, in], B bank [n, out, r]) bits, both ~ N(0, 0.01^2)."""
    sh = SHAPES[c]
    n = sh.get("n_adapters", 64) if n is None else n
    inp = sh["inp"] if inp is None else inp
    out = sh["out"] if out is None else out
    r = sh["r"] if r is None else r
    a = _rng(c, 2).standard_normal((n, r, inp), dtype=np.float32) * np.float32(0.01)
    b = _rng(c, 3).standard_normal((n, out, r), dtype=np.float32) * np.float32(0.01)
    return to_bf16_bits(a), to_bf16_bits(b)


def adapter_ids(c: int, M: int, n: int) -> np.ndarray:
    return _rng(c, 5).integers(0, n, size=M, dtype=np.int32)


def upstream_grad(c: int, M: int, out: int | None = None) -> np.ndarray:
    out = SHAPES[c]["out"] if out is None else out
    return to_bf16_bits(_rng(c, 4).standard_normal((M, out), dtype=np.float32))


@dataclass
class Workload:
    c: int
    out: int
    inp: int
    r: int
    alpha: float
    dq: bool

    @property
    def scale(self) -> float:
        return self.alpha / self.r


def workload(c: int) -> Workload:
    sh = SHAPES[c]
    return Workload(c=c, out=sh["out"], inp=sh["inp"], r=sh["r"], alpha=sh["alpha"], dq=sh["dq"])
