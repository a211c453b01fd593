"""GPU checks of the calibration library (include/nf4calib.h) whose figures
the benchmark quotes as measured ceilings: the plain read must touch every
byte it is asked to (the XOR of its per-workgroup words equals the XOR of
the whole buffer, computed on the host), and the two MFMA loops must run to
completion with finite, repeatable sums, their flop counts following the
header's formula."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu] %s" % request.node.nodeid, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def CAL():
    from bit_nf4_quantized_04_amd import calib

    return calib


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 7])
@pytest.mark.parametrize("workgroups", [0, 3])
def test_read_touches_every_word(CAL, nbytes, workgroups):
    import torch

    rng = np.random.default_rng(nbytes + workgroups)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    wgs = workgroups or CAL.default_workgroups(0)
    assert wgs > 0
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    CAL.read(buf, sink, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("dequant", [False, True])
def test_mfma_loops_finish_with_finite_repeatable_sums(CAL, dequant):
    import torch

    wgs = 8
    sink = torch.zeros(wgs * 8, dtype=torch.float32, device="cuda")
    fl = CAL.mfma_tile(20, sink, wgs, dequant)
    assert fl == wgs * 8 * 20 * 8 * 32 * 32 * 16 * 2
    torch.cuda.synchronize()
    first = sink.cpu().numpy().copy()
    assert np.isfinite(first).all() and (first != 0).any()
    CAL.mfma_tile(20, sink, wgs, dequant)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sink.cpu().numpy(), first)

    sink2 = torch.zeros(wgs, dtype=torch.float32, device="cuda")
    fl2 = CAL.mfma(20, sink2, wgs, 4)
    assert fl2 == wgs * 4 * 20 * 8 * 32 * 32 * 16 * 2
    torch.cuda.synchronize()
    assert np.isfinite(sink2.cpu().numpy()).all()
