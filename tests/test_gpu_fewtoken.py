"""GPU parity of the few-token decode forward (2 to 16 tokens) on the shapes
that reach its edge cases, each against the oracle: token counts below the
kernel's 4- and 16-token capacities, a row count that is not a multiple of
the 16-row tile, a row length whose 64-blocks do not fill the last 256-wide
block-step, no adapter and the largest rank the kernel takes, blocks of 64
with and without double quant, and a weight tall enough for the four-wave
workgroup shape."""

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


def _case(F, seed, M, out, inp, r, dq):
    import torch

    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    a = O.rne_bf16_bits((rng.standard_normal((max(r, 1), inp)) * np.sqrt(2.0 / inp)).astype(np.float32))[:r]
    b = O.rne_bf16_bits((rng.standard_normal((out, max(r, 1))) * 0.01).astype(np.float32))[:, :r]
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    s = 2.0
    print("case M=%d out=%d in=%d r=%d dq=%s" % (M, out, inp, r, dq), flush=True)
    q = F.nf4_quantize(U.f32(w), double_quant=dq)
    A = U.bf(a) if r else None
    B = U.bf(b) if r else None
    h = F.qlora_linear_forward(q, U.bf(x), A, B, s)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq), w.shape)
    href, _ = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("r", [0, 16, 64])
@pytest.mark.parametrize("M", [2, 5, 12, 16])
def test_few_tokens_ragged_rows_and_blocks(F, M, r, dq):
    # 250 rows: the last 16-row tile is partial; 17 blocks of 64: the last
    # block-step holds one block
    _case(F, 100 * M + r + int(dq), M, 250, 64 * 17, r, dq)


@pytest.mark.parametrize("M", [3, 16])
def test_few_tokens_tall_weight(F, M):
    # more than 512 row tiles: four waves per workgroup
    _case(F, 7 + M, M, 8208, 64 * 5, 64, True)
