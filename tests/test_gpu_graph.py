"""The layer calls captured in a HIP graph (torch.cuda.graph) and replayed:
the library launches only kernels on the caller's stream (no allocation, no
memset, no synchronization), so a captured call must give, on every replay,
the bits the same call gives eagerly.  Each replay is checked separately,
with the program's own eager work and a synchronization between replays."""

import sys

import numpy as np
import pytest

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


def _bits(rng, shape, std):
    from oracle import nf4_oracle as O

    return O.rne_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


@pytest.mark.parametrize("M,out,inp,r,dq", [
    (1, 4096, 2048, 64, True),     # decode: u kernel + fused GEMV
    (1, 1000, 1024, 16, False),    # decode, ragged rows
    (8, 2048, 1024, 32, True),     # few tokens
    (512, 2048, 1024, 64, True),   # tiled forward and backward
])
def test_layer_calls_replay_in_a_graph(F, M, out, inp, r, dq):
    import torch

    rng = np.random.default_rng(900 + M + r)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    q = F.nf4_quantize(U.f32(w), double_quant=dq)
    x, dh = U.bf(_bits(rng, (M, inp), 1.0)), U.bf(_bits(rng, (M, out), 1.0))
    a, b = U.bf(_bits(rng, (r, inp), np.sqrt(2.0 / inp))), U.bf(_bits(rng, (out, r), 0.01))
    dev = x.device
    wsf = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, out, inp, M, r), dtype=torch.uint8, device=dev)
    wsb = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD, out, inp, M, r), dtype=torch.uint8, device=dev)
    h = torch.empty((M, out), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((M, inp), dtype=torch.bfloat16, device=dev)
    da = torch.empty((r, inp), dtype=torch.float32, device=dev)
    db = torch.empty((out, r), dtype=torch.float32, device=dev)
    t = q.c_struct()
    lib = F._lib

    def step():
        st = F._stream()
        F._check(lib.qlora_linear_forward(F.C.byref(t), F._ptr(x), M, F._ptr(a), F._ptr(b), r, 2.0, F._ptr(h),
                                          F._ptr(u), F._ptr(wsf), wsf.numel(), st), "forward")
        F._check(lib.qlora_linear_backward(F.C.byref(t), F._ptr(x), F._ptr(dh), M, F._ptr(a), F._ptr(b), r, 2.0,
                                           F._ptr(u), F._ptr(dx), F._ptr(da), F._ptr(db), F._ptr(wsb),
                                           wsb.numel(), st), "backward")

    outs = (h, u, dx, da, db)
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:  # eager work between replays
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("h", "u", "dX", "dA", "dB"), outs, want):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), \
                "replay %d: %s differs from the eager call" % (rep, name)


def test_dropout_and_multi_adapter_calls_replay_in_a_graph(F):
    """The dropout forward + backward (the seed is an argument, so every
    replay draws the same mask) and the multi-adapter forward (token
    bucketing with workgroup-local atomics; the order inside a bucket does
    not change any token's output) replay bit for bit."""
    import torch

    rng = np.random.default_rng(4321)
    M, out, inp, r, n = 600, 2048, 1024, 16, 6
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    x, dh = U.bf(_bits(rng, (M, inp), 1.0)), U.bf(_bits(rng, (M, out), 1.0))
    a, b = U.bf(_bits(rng, (r, inp), np.sqrt(2.0 / inp))), U.bf(_bits(rng, (out, r), 0.01))
    ab, bb = U.bf(_bits(rng, (n, r, inp), np.sqrt(2.0 / inp))), U.bf(_bits(rng, (n, out, r), 0.01))
    dev = x.device
    ids = torch.from_numpy(rng.integers(0, n, M).astype(np.int32)).to(dev)
    scales = torch.full((n,), 2.0, dtype=torch.float32, device=dev)
    wsf = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD | F.QLORA_OP_DROPOUT, out, inp, M, r),
                      dtype=torch.uint8, device=dev)
    wsb = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD | F.QLORA_OP_DROPOUT, out, inp, M, r),
                      dtype=torch.uint8, device=dev)
    wsm = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD_MULTI, out, inp, M, r, n),
                      dtype=torch.uint8, device=dev)
    h = torch.empty((M, out), dtype=torch.bfloat16, device=dev)
    hm = torch.empty((M, out), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((M, inp), dtype=torch.bfloat16, device=dev)
    da = torch.empty((r, inp), dtype=torch.float32, device=dev)
    db = torch.empty((out, r), dtype=torch.float32, device=dev)
    t = q.c_struct()
    lib = F._lib
    d = F.qlora_dropout(0.1, 0, 77)

    def step():
        st = F._stream()
        F._check(lib.qlora_linear_forward_dropout(F.C.byref(t), F._ptr(x), M, F._ptr(a), F._ptr(b), r, 2.0,
                                                  F.C.byref(d), F._ptr(h), F._ptr(u), F._ptr(wsf), wsf.numel(),
                                                  st), "forward_dropout")
        F._check(lib.qlora_linear_backward_dropout(F.C.byref(t), F._ptr(x), F._ptr(dh), M, F._ptr(a), F._ptr(b),
                                                   r, 2.0, F.C.byref(d), F._ptr(u), F._ptr(dx), F._ptr(da),
                                                   F._ptr(db), F._ptr(wsb), wsb.numel(), st), "backward_dropout")
        F._check(lib.qlora_linear_forward_multi(F.C.byref(t), F._ptr(x), M, F._ptr(ab), F._ptr(bb), n, r,
                                                F._ptr(scales), F._ptr(ids), F._ptr(hm), F._ptr(wsm), wsm.numel(),
                                                st), "forward_multi")

    outs = (h, u, dx, da, db, hm)
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("h", "u", "dX", "dA", "dB", "h multi"), outs, want):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), \
                "replay %d: %s differs from the eager call" % (rep, name)
