"""Seeded sweep of layer shapes through every entry point, each against the
oracle: M, out, in, r and the scale format drawn at random (small sizes, so
the oracle is quick), which reaches the decode kernels, the few-token
backward, the small-grid GEMM and (for the larger draws) the register-dequant
kernels with and without split reductions."""

import numpy as np
import pytest

from oracle import nf4_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from bit_nf4_quantized_04_amd import nf4qlora

    return nf4qlora


def _draw(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.choice([1, 2, 5, 16, 17, 40, 300, 700]))
    out = int(rng.choice([64, 96, 250, 512, 1024, 2048, 4096]))
    inp = 64 * int(rng.choice([1, 3, 4, 8, 16, 17, 32]))
    r = int(rng.choice([1, 3, 8, 16, 24, 64, 65]))
    dq = bool(rng.integers(0, 2))
    group = int(rng.choice([256, 100])) if dq else 256
    return rng, M, out, inp, r, dq, group


@pytest.mark.parametrize("seed", range(24))
def test_layer_sweep(F, seed):
    import torch

    rng, M, out, inp, r, dq, group = _draw(1000 + seed)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    a = O.rne_bf16_bits((rng.standard_normal((r, inp)) * np.sqrt(2.0 / inp)).astype(np.float32))
    b = O.rne_bf16_bits((rng.standard_normal((out, r)) * 0.01).astype(np.float32))
    dh = O.rne_bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    s = float(rng.choice([0.25, 2.0]))
    print("case M=%d out=%d in=%d r=%d dq=%s group=%d" % (M, out, inp, r, dq, group), flush=True)
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    wm = F.qlora_merge(q, U.bf(a), U.bf(b), s)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq, dq_group=group), w.shape, dq_group=group)
    href, uref = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("u", u.cpu().numpy(), uref)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])
    U.assert_close("merged", U.bf16_to_f64(wm), O.bf16_bits_to_f32(O.merge(wb, a, b, s)).astype(np.float64))


# (tokens, out features, in features): forward grids of 256 x 256 tiles with
# and without a split partial last pass, dX grids with and without splits of
# the weight rows, and shapes that stay on the tiled kernels
_LARGE_SHAPES = [
    (1100, 2048, 512), (600, 4096, 1024), (1000, 1024, 2048), (1100, 4096, 1024), (2048, 1024, 1024),
    (700, 2048, 2048), (1500, 4096, 256), (513, 8192, 1024), (1024, 2048, 4096), (3000, 1024, 1024),
]


def _draw_large(seed):
    rng = np.random.default_rng(3000 + seed)
    M, out, inp = _LARGE_SHAPES[seed % len(_LARGE_SHAPES)]
    r = int(rng.choice([1, 8, 24, 64, 96]))
    dq = bool(rng.integers(0, 2))
    group = int(rng.choice([256, 100])) if dq else 256
    return rng, M, out, inp, r, dq, group


@pytest.mark.parametrize("seed", range(10))
def test_large_tile_sweep(F, seed):
    """Shapes for the 256 x 256 register-dequant kernels: forward grids with
    a split tail pass, dX grids split over the weight rows."""
    import torch

    rng, M, out, inp, r, dq, group = _draw_large(seed)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    a = O.rne_bf16_bits((rng.standard_normal((r, inp)) * np.sqrt(2.0 / inp)).astype(np.float32))
    b = O.rne_bf16_bits((rng.standard_normal((out, r)) * 0.01).astype(np.float32))
    dh = O.rne_bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    s = 2.0
    print("case M=%d out=%d in=%d r=%d dq=%s group=%d" % (M, out, inp, r, dq, group), flush=True)
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq, dq_group=group), w.shape, dq_group=group)
    href, uref = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])


@pytest.mark.parametrize("seed", range(8))
def test_multi_adapter_sweep(F, seed):
    import torch

    rng, M, out, inp, r, dq, group = _draw(2000 + seed)
    n = int(rng.integers(1, 9))
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    ab = O.rne_bf16_bits((rng.standard_normal((n, r, inp)) * 0.05).astype(np.float32))
    bb = O.rne_bf16_bits((rng.standard_normal((n, out, r)) * 0.05).astype(np.float32))
    scales = (2.0 ** rng.integers(-2, 3, size=n)).astype(np.float32)
    ids = rng.integers(-1, n + 1, size=M).astype(np.int32)
    print("case M=%d out=%d in=%d r=%d n=%d dq=%s" % (M, out, inp, r, n, dq), flush=True)
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    h = F.qlora_linear_forward_multi(q, U.bf(x), U.bf(ab), U.bf(bb), torch.from_numpy(scales).to(U.dev()),
                                     torch.from_numpy(ids).to(U.dev()))
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq, dq_group=group), w.shape, dq_group=group)
    U.assert_close("h", U.bf16_to_f64(h), O.forward_multi(wb, x, ab, bb, scales.astype(np.float64), ids))
