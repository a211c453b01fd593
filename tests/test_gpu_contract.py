"""GPU checks of two contract points of the C ABI beyond the pages: a weight
block holding Inf or NaN (quantized to a NaN scale, so everything reading it
is NaN), and int8 scale codes outside [0, 127] from another producer (every
call decodes fl32(fl32(q/127) * c) for the signed code).  The expected values
come from the oracle on the same inputs."""

import sys

import numpy as np
import pytest

from oracle import nf4_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu] %s" % request.node.nodeid, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def F():
    from bit_nf4_quantized_04_amd import nf4qlora

    return nf4qlora


def _nan_close(name, got, ref):
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref), err_msg=name + ": NaN pattern")
    ok = ~np.isnan(ref)
    assert ok.any() and (~ok).any()
    U.assert_close(name, got[ok], ref[ok])


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("M", [1, 4, 16, 64, 300, 1100])
def test_non_finite_weights_through_the_layer(F, M, dq):
    """A weight with one NaN and one Inf element, through the forward and the
    backward at token counts that reach every product kernel (the single-token
    GEMV, the few-token kernels, the tiled GEMMs): an output reading a
    non-finite block is NaN, as in the oracle (s * T[c] with s NaN, for level
    0 too), and every other output matches the oracle."""
    import torch

    out, inp, r, s = 4096, 1024, 16, 2.0
    rng = np.random.default_rng(83 + M + dq)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    w[100, 70] = np.nan
    w[3000, 1000] = -np.inf
    ref = O.quantize(w, double_quant=dq)
    x = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    a = O.rne_bf16_bits((rng.standard_normal((r, inp)) * 0.05).astype(np.float32))
    b = O.rne_bf16_bits((rng.standard_normal((out, r)) * 0.01).astype(np.float32))
    dh = O.rne_bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    q = F.nf4_quantize(U.f32(w), double_quant=dq)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    torch.cuda.synchronize()
    wb = O.compute_weight(ref, w.shape)
    href, _ = O.forward(wb, x, a, b, s)
    g = O.backward(wb, x, dh, a, b, s)
    _nan_close("h", U.bf16_to_f64(h), href)
    if dq:  # a NaN group constant reaches every dX column
        assert np.isnan(g["dX"]).all() and np.isnan(U.bf16_to_f64(dX)).all()
    else:
        _nan_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])


@pytest.mark.parametrize("dq,block", [(False, 64), (True, 64), (True, 128)])
def test_non_finite_blocks(F, dq, block):
    import torch

    rng = np.random.default_rng(61 + dq + block)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    w[0, 5] = np.inf
    w[7, 300] = np.nan
    w[50, 511] = -np.inf
    q = F.nf4_quantize(U.f32(w), double_quant=dq, block_size=block)
    wd = F.nf4_dequantize(q)
    torch.cuda.synchronize()
    ref = O.quantize(w, double_quant=dq, block_size=block)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref["codes"])
    got_s = q.absmax.cpu().numpy()[:ref["absmax"].size]
    np.testing.assert_array_equal(np.isnan(got_s), np.isnan(ref["absmax"]))
    fin = ~np.isnan(ref["absmax"])
    np.testing.assert_array_equal(got_s[fin].view(np.uint32), ref["absmax"][fin].view(np.uint32))
    if dq:
        np.testing.assert_array_equal(q.scale_codes.cpu().numpy()[:ref["scale_codes"].size], ref["scale_codes"])
        gg = q.group_absmax.cpu().numpy()[:ref["group_absmax"].size]
        np.testing.assert_array_equal(np.isnan(gg), np.isnan(ref["group_absmax"]))
        fg = ~np.isnan(gg)
        np.testing.assert_array_equal(gg[fg].view(np.uint32), ref["group_absmax"][fg].view(np.uint32))
    wref = O.dequantize(ref, w.shape, block_size=block)
    got = wd.cpu().numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(wref))
    ok = ~np.isnan(wref)
    np.testing.assert_array_equal(got[ok].view(np.uint32), wref[ok].view(np.uint32))
    assert np.isnan(wref).any()


@pytest.mark.parametrize("M,out,inp", [(1, 512, 1024), (4, 256, 512), (16, 256, 512), (40, 320, 512),
                                       (600, 2048, 1024)])
def test_negative_scale_codes_decode_alike(F, M, out, inp):
    """A double-quantized weight whose int8 scale codes include negative
    values (made on the CPU from the oracle's storage): dequantize, the
    forward and the backward all use the signed decode, as the oracle does."""
    import torch

    rng = np.random.default_rng(71 + M)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    ref = O.quantize(w, double_quant=True)
    sc = ref["scale_codes"].copy()
    neg = rng.random(sc.size) < 0.3
    sc[neg] = -sc[neg]
    sc[::97] = -128
    ref["scale_codes"] = sc
    r, s = 16, 2.0
    x = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    a = O.rne_bf16_bits((rng.standard_normal((r, inp)) * 0.05).astype(np.float32))
    b = O.rne_bf16_bits((rng.standard_normal((out, r)) * 0.01).astype(np.float32))
    dh = O.rne_bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    q = U.weight_from_oracle(F, ref, out, inp, True)
    wd = F.nf4_dequantize(q)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    torch.cuda.synchronize()
    wref = O.dequantize(ref, w.shape)
    np.testing.assert_array_equal(wd.cpu().numpy().view(np.uint32), wref.view(np.uint32))
    assert (wref < 0).any() and O.decode_scales(sc, ref["group_absmax"]).min() < 0
    wb = O.compute_weight(ref, w.shape)
    href, _ = O.forward(wb, x, a, b, s)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])
