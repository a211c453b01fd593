"""GPU parity of the quantizer and dequantizer: bit-exact against the oracle."""

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


def _gpu_quant(F, w, dq, group=256):
    import torch

    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    torch.cuda.synchronize()
    return q


def _compare_q(q, ref, dq):
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(q.absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32))
    if dq:
        np.testing.assert_array_equal(q.scale_codes.cpu().numpy(), ref["scale_codes"])
        np.testing.assert_array_equal(q.group_absmax.cpu().numpy().view(np.uint32),
                                      ref["group_absmax"].view(np.uint32))


@pytest.mark.parametrize("shape,dq,group", [
    ((256, 256), False, 256),       # the tiny workload
    ((384, 512), True, 256),        # 3072 blocks: 12 full groups
    ((100, 192), True, 256),        # 300 blocks: a partial last group
    ((7, 64), True, 5),             # odd group size, partial last group
    ((1, 64), True, 256),           # a single block
    ((33, 320), True, 10**6),       # one global constant
])
def test_quantize_matches_oracle(F, shape, dq, group):
    rng = np.random.default_rng(hash(shape) % 2**32)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w.reshape(-1)[::997] *= 40  # outliers: coarse scales inside their DQ groups
    q = _gpu_quant(F, w, dq, group)
    _compare_q(q, O.quantize(w, double_quant=dq, dq_group=group), dq)


def _adversarial_blocks():
    t = O.NF4_LEVELS.astype(np.float64)
    mids = (t[:-1] + t[1:]) / 2
    rows = []
    # blocks of normalized values right at / next to every midpoint, scale 1
    for m in mids:
        f = np.float32(m)
        vals = [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2)),
                np.nextafter(np.nextafter(f, np.float32(2)), np.float32(2))]
        blk = np.zeros(64, dtype=np.float32)
        blk[:4] = vals
        blk[4] = 1.0  # absmax element
        blk[5:9] = [-v for v in vals]
        rows.append(blk)
    rows.append(np.zeros(64, dtype=np.float32))                       # all-zero block
    b = np.zeros(64, dtype=np.float32); b[17] = -3.5; rows.append(b)  # one nonzero, negative
    b = np.zeros(64, dtype=np.float32); b[0] = 2.0; b[63] = -2.0; rows.append(b)  # +s and -s
    b = np.full(64, -0.0, dtype=np.float32); b[9] = 1e-3; rows.append(b)  # negative zeros
    b = (np.arange(1, 65, dtype=np.float32) * np.float32(1e-45)); rows.append(b)  # subnormals
    b = (np.linspace(-1, 1, 64) * 3e38).astype(np.float32); rows.append(b)  # near float max
    b = (np.linspace(-1, 1, 64) * 1e-30).astype(np.float32); rows.append(b)  # tiny normal scale
    b = np.full(64, 0.25, dtype=np.float32); rows.append(b)           # constant block
    # midpoint sweep scaled: w = m * s for a non-trivial s (division then rounds)
    rng = np.random.default_rng(3)
    for s in rng.uniform(0.01, 5.0, 6).astype(np.float32):
        blk = (np.repeat(mids, 5)[:63] * s).astype(np.float32)
        rows.append(np.concatenate([blk, [s]]).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("dq", [False, True])
def test_quantize_adversarial_blocks(F, dq):
    w = _adversarial_blocks()
    q = _gpu_quant(F, w, dq)
    _compare_q(q, O.quantize(w, double_quant=dq), dq)


@pytest.mark.parametrize("c", [2, 3, 4])
def test_quantize_workload_full_size_sampled(F, c):
    """Full-size weights of the decode / 7B / 70B workloads quantized on the
    GPU; the oracle re-derives 48 sampled double-quant groups independently."""
    from bit_nf4_quantized_04_amd import workloads as wl

    w = wl.weight(c)
    q = _gpu_quant(F, w, True)
    flat = w.reshape(-1)
    ng = (flat.size // 64 + 255) // 256
    rng = np.random.default_rng(c)
    groups = np.unique(np.concatenate([[0, ng - 1], rng.integers(0, ng, 46)]))
    codes = q.codes.cpu().numpy()
    sc = q.scale_codes.cpu().numpy()
    ga = q.group_absmax.cpu().numpy()
    ab = q.absmax.cpu().numpy()
    for g in groups:
        lo, hi = g * 16384, min((g + 1) * 16384, flat.size)
        ref = O.quantize(flat[lo:hi], double_quant=True)
        np.testing.assert_array_equal(codes[lo // 2:hi // 2], ref["codes"])
        np.testing.assert_array_equal(sc[lo // 64:hi // 64], ref["scale_codes"])
        np.testing.assert_array_equal(ab[lo // 64:hi // 64], ref["absmax"])
        assert ga[g] == ref["group_absmax"][0]


@pytest.mark.parametrize("shape,dq,group", [((256, 256), False, 256), ((384, 512), True, 256),
                                            ((100, 192), True, 256), ((7, 64), True, 5)])
def test_dequantize_bit_exact(F, shape, dq, group):
    import torch

    rng = np.random.default_rng(11)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w.reshape(-1)[::131] *= 30
    ref = O.quantize(w, double_quant=dq, dq_group=group)
    # the oracle's quantized buffers are the GPU's input here
    qw = F.NF4Weight(torch.from_numpy(ref["codes"]).to(U.dev()),
                     torch.from_numpy(ref["absmax"]).to(U.dev()),
                     None if not dq else torch.from_numpy(ref["scale_codes"]).to(U.dev()),
                     None if not dq else torch.from_numpy(ref["group_absmax"]).to(U.dev()),
                     shape[0], shape[1], dq, group)
    w32 = F.nf4_dequantize(qw).cpu().numpy()
    wbf = F.nf4_dequantize_bf16(qw)
    torch.cuda.synchronize()
    want = O.dequantize(ref, shape, dq_group=group)
    np.testing.assert_array_equal(w32.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(U.bits_of(wbf), O.rne_bf16_bits(want))


def test_dequantize_workload_full_size(F):
    """Decode workload weight [4096, 4096]: GPU quantize -> GPU dequantize,
    compared in full with the oracle's dequantization of its own quantization."""
    from bit_nf4_quantized_04_amd import workloads as wl
    import torch

    w = wl.weight(2)
    q = _gpu_quant(F, w, True)
    got = F.nf4_dequantize(q).cpu().numpy()
    gotb = U.bits_of(F.nf4_dequantize_bf16(q))
    torch.cuda.synchronize()
    ref = U.oracle_quantize_chunked(w.reshape(-1), True)
    want = O.dequantize(ref, w.shape)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(gotb, O.rne_bf16_bits(want))


def test_repeat_determinism(F):
    from bit_nf4_quantized_04_amd import workloads as wl

    w = wl.weight(1)
    a = _gpu_quant(F, w, True)
    b = _gpu_quant(F, w, True)
    assert np.array_equal(a.codes.cpu().numpy(), b.codes.cpu().numpy())
    assert np.array_equal(a.scale_codes.cpu().numpy(), b.scale_codes.cpu().numpy())
