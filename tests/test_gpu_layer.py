"""GPU parity of the QLoRA layer (forward, backward, multi-adapter) against the
oracle, elementwise within |err| <= 1e-2|ref| + 1e-3 rms(ref)."""

import sys

import ctypes as C

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


def _bits(rng, shape, std):
    return O.rne_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _case(seed, M, out, inp, r, dq=True):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = _bits(rng, (M, inp), 1.0)
    a = _bits(rng, (r, inp), np.sqrt(2.0 / inp))
    b = _bits(rng, (out, r), 0.01)
    dh = _bits(rng, (M, out), 1.0)
    return w, x, a, b, dh


SMALL = [  # (M, out, in, r): ragged M and out, several tiles, r from 1 to 64
    (5, 200, 320, 8),
    (1, 96, 128, 4),
    (17, 130, 256, 1),
    (130, 257, 192, 16),
    (3, 64, 64, 64),
    (260, 300, 448, 24),
    (300, 160, 192, 40),  # out % 16 == 0: the streamed rank-r backward products
]


@pytest.mark.parametrize("M,out,inp,r", SMALL)
@pytest.mark.parametrize("dq", [False, True])
def test_forward_small(F, M, out, inp, r, dq):
    import torch

    w, x, a, b, _ = _case(M * 7 + out, M, out, inp, r)
    s = 2.0
    q = F.nf4_quantize(U.f32(w), double_quant=dq)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq), w.shape)
    href, uref = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("u", u.cpu().numpy(), uref)


@pytest.mark.parametrize("M", [2, 4, 16])
@pytest.mark.parametrize("out", [4096, 8200])
def test_few_token_forward_both_workgroup_shapes(F, M, out):
    """The few-token forward kernel takes eight waves per workgroup below 512
    row tiles (4096 rows) and four at or above (8200 rows: 513 tiles, the last
    one ragged); both against the oracle."""
    import torch

    inp, r, s = 512, 16, 2.0
    w, x, a, b, _ = _case(M * 13 + out, M, out, inp, r)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    href, uref = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("u", u.cpu().numpy(), uref)


@pytest.mark.parametrize("M,out,inp,r", SMALL)
def test_backward_small(F, M, out, inp, r):
    import torch

    w, x, a, b, dh = _case(M * 13 + out, M, out, inp, r)
    s = 0.5
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    _, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    for uu in (u, None):  # saved u, and recomputed u
        dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=uu)
        torch.cuda.synchronize()
        wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
        g = O.backward(wb, x, dh, a, b, s)
        U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
        U.assert_close("dA", dA.cpu().numpy(), g["dA"])
        U.assert_close("dB", dB.cpu().numpy(), g["dB"])


# The few-token backward (M <= 16): one pass over the weight rows for dX and
# dU.  Ragged rows, several 1024-column slabs and rank-r slabs, r not a
# multiple of 4, absmax without double quant, a non-power-of-two double-quant
# group, and enough rows for many row chunks.
@pytest.mark.parametrize("M,out,inp,r,dq,group", [
    (1, 96, 128, 4, False, 256),
    (2, 100, 192, 3, True, 256),
    (16, 64, 1088, 65, True, 256),
    (7, 333, 1024, 16, False, 256),
    (1, 8192, 128, 64, True, 256),
    (3, 250, 640, 12, True, 100),
])
def test_backward_few_tokens(F, M, out, inp, r, dq, group):
    import torch

    w, x, a, b, dh = _case(M * 29 + out + r, M, out, inp, r)
    s = 2.0
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    _, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    _, dA2, dB2 = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u, want_dx=False)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq, dq_group=group), w.shape, dq_group=group)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])
    assert torch.equal(dA, dA2) and torch.equal(dB, dB2)


def test_zero_B_gives_base_output(F):
    """B = 0: the output is the base product alone (LoRA init in the pages)."""
    import torch

    w, x, a, b, _ = _case(5, 33, 160, 256, 8)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h0 = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(np.zeros_like(b)), 2.0)
    hb = F.qlora_linear_forward(q, U.bf(x), None, None, 2.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(U.bits_of(h0), U.bits_of(hb))
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    U.assert_close("h", U.bf16_to_f64(hb), O._bf(x) @ wb.T)


def _workload(c, M):
    from bit_nf4_quantized_04_amd import workloads as wl

    sh = wl.SHAPES[c]
    w = wl.weight(c)
    x = wl.activations(c, M)
    a, b = wl.adapters(c)
    return w, x, a, b, sh["alpha"] / sh["r"]


def test_tiny_workload_forward_backward(F):
    import torch
    from bit_nf4_quantized_04_amd import workloads as wl

    w, x, a, b, s = _workload(1, 4)
    dh = wl.upstream_grad(1, 4)
    q = F.nf4_quantize(U.f32(w), double_quant=False)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=False), w.shape)
    href, _ = O.forward(wb, x, a, b, s)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_workload_forward(F, M):
    import torch

    w, x, a, b, s = _workload(2, M)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s)
    torch.cuda.synchronize()
    ref = U.oracle_quantize_chunked(w.reshape(-1), True)
    wb = O.compute_weight(ref, w.shape)
    href, _ = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)


def test_7b_mlp_workload_forward_backward(F):
    """LLaMA-7B MLP shape 4096 -> 11008, 2048 tokens, r = 64: full compare."""
    import torch
    from bit_nf4_quantized_04_amd import workloads as wl

    w, x, a, b, s = _workload(3, 2048)
    dh = wl.upstream_grad(3, 2048)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    torch.cuda.synchronize()
    ref = U.oracle_quantize_chunked(w.reshape(-1), True)
    wb = O.compute_weight(ref, w.shape)
    href, _ = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])


def test_multi_adapter_small(F):
    import torch

    rng = np.random.default_rng(21)
    out, inp, r, n, M = 200, 256, 8, 7, 90
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = _bits(rng, (M, inp), 1.0)
    ab = _bits(rng, (n, r, inp), 0.05)
    bb = _bits(rng, (n, out, r), 0.05)
    scales = np.array([2.0, 0.5, 1.0, 4.0, 0.25, 2.0, 1.5], dtype=np.float32)
    ids = rng.integers(-2, n + 2, size=M).astype(np.int32)  # includes invalid ids
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h = F.qlora_linear_forward_multi(q, U.bf(x), U.bf(ab), U.bf(bb),
                                     torch.from_numpy(scales).to(U.dev()),
                                     torch.from_numpy(ids).to(U.dev()))
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    href = O.forward_multi(wb, x, ab, bb, scales.astype(np.float64), ids)
    U.assert_close("h", U.bf16_to_f64(h), href)


@pytest.mark.parametrize("M,out,inp,r,n", [
    (700, 4096, 512, 6, 5),   # split reduction, gather in the partial sum, scalar gather (r % 8)
    (500, 4096, 256, 16, 9),  # one split: the gather in the kernel's epilogue, 16-byte gather
])
def test_multi_adapter_large_tiles(F, M, out, inp, r, n):
    """The multi-adapter forward on the 256 x 256 register-dequant kernel:
    ragged M, invalid ids."""
    import torch

    rng = np.random.default_rng(23 + M)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = _bits(rng, (M, inp), 1.0)
    ab = _bits(rng, (n, r, inp), 0.05)
    bb = _bits(rng, (n, out, r), 0.05)
    scales = (2.0 ** rng.integers(-2, 3, size=n)).astype(np.float32)
    ids = rng.integers(-1, n + 1, size=M).astype(np.int32)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h = F.qlora_linear_forward_multi(q, U.bf(x), U.bf(ab), U.bf(bb),
                                     torch.from_numpy(scales).to(U.dev()),
                                     torch.from_numpy(ids).to(U.dev()))
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    href = O.forward_multi(wb, x, ab, bb, scales.astype(np.float64), ids)
    U.assert_close("h", U.bf16_to_f64(h), href)


@pytest.mark.parametrize("n,r", [(5000, 2), (3, 80)])
def test_multi_adapter_unbucketed(F, n, r):
    """More adapters than the token bucketing takes (4096), or r > 64: the
    per-token down-projection and gather."""
    import torch

    rng = np.random.default_rng(n + r)
    out, inp, M = 320, 256, 600
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = _bits(rng, (M, inp), 1.0)
    ab = _bits(rng, (n, r, inp), 0.05)
    bb = _bits(rng, (n, out, r), 0.05)
    scales = (2.0 ** rng.integers(-2, 3, size=n)).astype(np.float32)
    ids = rng.integers(-1, n + 1, size=M).astype(np.int32)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h = F.qlora_linear_forward_multi(q, U.bf(x), U.bf(ab), U.bf(bb),
                                     torch.from_numpy(scales).to(U.dev()),
                                     torch.from_numpy(ids).to(U.dev()))
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    href = O.forward_multi(wb, x, ab, bb, scales.astype(np.float64), ids)
    U.assert_close("h", U.bf16_to_f64(h), href)


def test_multi_adapter_workload(F):
    """64 adapters, r = 16, 2048 tokens with uniform ids on the 4096 x 4096 base."""
    import torch
    from bit_nf4_quantized_04_amd import workloads as wl

    c = 5
    sh = wl.SHAPES[c]
    w = wl.weight(c)
    x = wl.activations(c, 2048)
    ab, bb = wl.adapter_bank(c)
    ids = wl.adapter_ids(c, 2048, sh["n_adapters"])
    scales = np.full(sh["n_adapters"], sh["alpha"] / sh["r"], dtype=np.float32)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h = F.qlora_linear_forward_multi(q, U.bf(x), U.bf(ab), U.bf(bb),
                                     torch.from_numpy(scales).to(U.dev()),
                                     torch.from_numpy(ids).to(U.dev()))
    torch.cuda.synchronize()
    ref = U.oracle_quantize_chunked(w.reshape(-1), True)
    wb = O.compute_weight(ref, w.shape)
    href = O.forward_multi(wb, x, ab, bb, scales.astype(np.float64), ids)
    U.assert_close("h", U.bf16_to_f64(h), href)


# Shapes that take the large-tile (256 x 256) kernels: at least 512 output
# tiles, ragged in every dimension, and cheap for the oracle.
# (600, 4096, 1024, 8): 48 tiles of 256 x 256, the register-dequant kernel
# on a grid smaller than the GPU.
@pytest.mark.parametrize("M,out,inp,r", [(4000, 8200, 192, 16), (4096, 8192, 128, 0), (600, 4096, 1024, 8)])
def test_forward_large_tiles(F, M, out, inp, r):
    import torch

    w, x, a, b, _ = _case(M + out, M, out, inp, max(r, 1))
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    if r:
        h = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), 2.0)
    else:
        h = F.qlora_linear_forward(q, U.bf(x), None, None, 2.0)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    href = O._bf(x) @ wb.T
    if r:
        href, _ = O.forward(wb, x, a, b, 2.0)
    U.assert_close("h", U.bf16_to_f64(h), href)


# (1000, 1024, 2048, 24): 32 dX tiles, so the reduction over the weight rows
# is split eight ways (the rank-r steps in the last split), ragged M.
@pytest.mark.parametrize("M,out,inp,r", [(4000, 500, 8256, 16), (4096, 256, 8192, 64), (1000, 1024, 2048, 24)])
def test_backward_large_tiles(F, M, out, inp, r):
    import torch

    w, x, a, b, dh = _case(M + inp, M, out, inp, r)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), 0.5)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    g = O.backward(wb, x, dh, a, b, 0.5)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])


# The register-dequant kernels with absmax scales (no double quant) and with a
# double-quant group that is not a power of two (the fp32 block scales are
# decoded by division then).
@pytest.mark.parametrize("dq,group", [(False, 256), (True, 100)])
def test_large_tiles_scale_formats(F, dq, group):
    import torch

    M, out, inp, r = 600, 4096, 2048, 8  # 48 forward tiles; 24 dX tiles, split eight ways
    w, x, a, b, dh = _case(M + out + group, M, out, inp, r)
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), 2.0, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), 2.0, u=u)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq, dq_group=group), w.shape, dq_group=group)
    href, _ = O.forward(wb, x, a, b, 2.0)
    U.assert_close("h", U.bf16_to_f64(h), href)
    g = O.backward(wb, x, dh, a, b, 2.0)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])


# The adapter merged into the bf16 base weight: ragged rows and column tiles,
# r not a multiple of 8, r over one 64-row chunk, absmax scales, a
# non-power-of-two double-quant group.
@pytest.mark.parametrize("out,inp,r,dq,group", [
    (200, 320, 8, True, 256),
    (130, 192, 3, True, 256),
    (1000, 2048, 64, True, 256),
    (96, 1088, 70, False, 256),
    (250, 640, 12, True, 100),
])
def test_merge(F, out, inp, r, dq, group):
    import torch

    w, _, a, b, _ = _case(out * 3 + r, 1, out, inp, r)
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group)
    s = 2.0
    wm = F.qlora_merge(q, U.bf(a), U.bf(b), s)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=dq, dq_group=group), w.shape, dq_group=group)
    ref = O.bf16_bits_to_f32(O.merge(wb, a, b, s)).astype(np.float64)
    U.assert_close("merged", U.bf16_to_f64(wm), ref)
    # without the adapter the merge is the bit-exact bf16 dequantization
    wz = F.qlora_merge(q, U.bf(a), U.bf(np.zeros_like(b)), s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wz.view(torch.int16).cpu().numpy().view(np.uint16),
                                  O.rne_bf16_bits(O.dequantize(O.quantize(w, double_quant=dq, dq_group=group),
                                                               w.shape, dq_group=group)))


class _DevView:
    """A device address standing for a pinned host tensor (for the binding)."""

    def __init__(self, ptr, t):
        self.ptr, self.t = ptr, t

    def data_ptr(self):
        return self.ptr

    def numel(self):
        return self.t.numel()


@pytest.mark.parametrize("host_state", [False, True])
def test_adamw_steps(F, host_state):
    """Five AdamW steps on a ragged parameter vector against the oracle; the
    moments in device memory or in pinned host memory (paged optimizer
    state); the bf16 copy of the parameters."""
    import torch

    rng = np.random.default_rng(31 + host_state)
    n = 12345
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    hp32 = {k: float(np.float32(x)) for k, x in hp.items()}
    p0 = rng.standard_normal(n).astype(np.float32)
    p = torch.from_numpy(p0.copy()).to(U.dev())
    if host_state:
        m = torch.zeros(n, dtype=torch.float32).pin_memory()
        v = torch.zeros(n, dtype=torch.float32).pin_memory()
        # the kernel gets the device address of the pinned pages
        rt = F.HipEvents().rt
        rt.hipHostGetDevicePointer.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_uint]
        dev_ptrs = []
        for t in (m, v):
            dp = C.c_void_p()
            if rt.hipHostGetDevicePointer(C.byref(dp), C.c_void_p(t.data_ptr()), 0) != 0 or not dp.value:
                pytest.skip("pinned host memory is not mapped for the device")
            dev_ptrs.append(_DevView(dp.value, t))
        mk, vk = dev_ptrs
    else:
        m = torch.zeros(n, dtype=torch.float32, device=U.dev())
        v = torch.zeros(n, dtype=torch.float32, device=U.dev())
        mk, vk = m, v
    pb = torch.empty(n, dtype=torch.bfloat16, device=U.dev())
    rp, rm, rv = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 10.0 ** rng.integers(-4, 1)).astype(np.float32)
        F.qlora_adamw_step(p, torch.from_numpy(g).to(U.dev()), mk, vk, t, p_bf16=pb, **hp)
        torch.cuda.synchronize()
        # the oracle steps from the GPU's fp32 state, so errors do not compound
        # (with the hyperparameters as the call receives them: float32)
        rp, rm, rv = O.adamw_step(p_prev if t > 1 else rp, g, m_prev if t > 1 else rm,
                                  v_prev if t > 1 else rv, t, **hp32)
        gp, gm, gv = p.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy()
        # bounds from the fp32 arithmetic: a few roundings (2^-24 relative
        # each) of every term's magnitude
        pp = p_prev if t > 1 else p0.astype(np.float64)
        mp = m_prev if t > 1 else np.zeros(n)
        vp = v_prev if t > 1 else np.zeros(n)
        b1, b2, lr = hp32["beta1"], hp32["beta2"], hp32["lr"]
        u = 2.0 ** -24
        step_mag = lr * np.abs(rm / (1 - b1 ** t)) / (np.sqrt(rv / (1 - b2 ** t)) + hp32["eps"])
        assert np.all(np.abs(gm - rm) <= 4 * u * (b1 * np.abs(mp) + (1 - b1) * np.abs(g)))
        assert np.all(np.abs(gv - rv) <= 4 * u * (b2 * vp + (1 - b2) * g.astype(np.float64) ** 2))
        assert np.all(np.abs(gp - rp) <= 4 * u * np.abs(pp) + 16 * u * step_mag)
        np.testing.assert_array_equal(pb.view(torch.int16).cpu().numpy().view(np.uint16), O.rne_bf16_bits(gp))
        p_prev, m_prev, v_prev = gp.astype(np.float64), gm.astype(np.float64), gv.astype(np.float64)


# The merged 16-bit weight taken back to NF4 storage: nf4_quantize_bf16 of
# the merge output equals the oracle's quantizer on the same bf16 values
# (widened exactly to fp32), bit for bit, codes and scales.
@pytest.mark.parametrize("out,inp,r,dq,bs", [(300, 256, 16, True, 64), (512, 1024, 64, False, 64),
                                             (96, 320, 8, True, 128)])
def test_merged_weight_requantized(F, out, inp, r, dq, bs):
    import torch

    rng = np.random.default_rng(out + inp + r)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    a = O.rne_bf16_bits((rng.standard_normal((r, inp)) * np.sqrt(2.0 / inp)).astype(np.float32))
    b = O.rne_bf16_bits((rng.standard_normal((out, r)) * 0.01).astype(np.float32))
    q = F.nf4_quantize(U.f32(w), double_quant=dq, block_size=bs)
    wm = F.qlora_merge(q, U.bf(a), U.bf(b), 2.0)
    q2 = F.nf4_quantize(wm, double_quant=dq, block_size=bs)
    torch.cuda.synchronize()
    wm_f32 = O.bf16_bits_to_f32(wm.view(torch.int16).cpu().numpy().view(np.uint16))
    ref = O.quantize(wm_f32, double_quant=dq, block_size=bs)
    np.testing.assert_array_equal(q2.codes.cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(q2.absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32))
    if dq:
        np.testing.assert_array_equal(q2.scale_codes.cpu().numpy(), ref["scale_codes"])
        np.testing.assert_array_equal(q2.group_absmax.cpu().numpy().view(np.uint32),
                                      ref["group_absmax"].view(np.uint32))


# The largest accepted rank (256) through every layer call, on a few tokens
# (general path) and one token.
@pytest.mark.parametrize("M", [1, 40])
def test_largest_rank(F, M):
    import torch

    out, inp, r, s = 300, 512, 256, 0.25
    w, x, a, b, dh = _case(4242 + M, M, out, inp, r)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    hd, ud = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True, dropout=(0.1, 9))
    gd = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=ud, dropout=(0.1, 9))
    wm = F.qlora_merge(q, U.bf(a), U.bf(b), s)
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    href, uref = O.forward(wb, x, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("u", u.cpu().numpy(), uref)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])
    keep = O.dropout_keep(M, inp, 0.1, 9)
    xf, af, bf_, dhf = O._bf(x), O._bf(a), O._bf(b), O._bf(dh)
    hdr, udr = O.forward_dropout64(wb, xf, af, bf_, s, keep, 0.1)
    U.assert_close("h dropout", U.bf16_to_f64(hd), hdr)
    U.assert_close("u dropout", ud.cpu().numpy(), udr)
    gdr = O.backward_dropout64(wb, xf, dhf, af, bf_, s, keep, 0.1)
    U.assert_close("dX dropout", U.bf16_to_f64(gd[0]), gdr["dX"])
    U.assert_close("dA dropout", gd[1].cpu().numpy(), gdr["dA"])
    U.assert_close("dB dropout", gd[2].cpu().numpy(), gdr["dB"])
    U.assert_close("merged", U.bf16_to_f64(wm), O.bf16_bits_to_f32(O.merge(wb, a, b, s)).astype(np.float64))


# No tokens: the forward writes nothing, the backward gives zero dA and dB.
def test_no_tokens(F):
    import torch

    out, inp, r = 128, 256, 8
    w, x, a, b, dh = _case(77, 1, out, inp, r)
    q = F.nf4_quantize(U.f32(w), double_quant=True)
    x0 = torch.empty((0, inp), dtype=torch.bfloat16, device=U.dev())
    dh0 = torch.empty((0, out), dtype=torch.bfloat16, device=U.dev())
    h = F.qlora_linear_forward(q, x0, U.bf(a), U.bf(b), 2.0)
    assert tuple(h.shape) == (0, out)
    dX, dA, dB = F.qlora_linear_backward(q, x0, dh0, U.bf(a), U.bf(b), 2.0)
    torch.cuda.synchronize()
    assert tuple(dX.shape) == (0, inp)
    assert torch.count_nonzero(dA).item() == 0 and torch.count_nonzero(dB).item() == 0
