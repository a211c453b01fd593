"""GPU parity of the FP4 quant type (the E2M1 reading of the oracle): the
quantizer and dequantizer bit-exact, every float32 of [-1, 1] through the
code search, and the layer calls (forward, backward, multi-adapter, merge,
blocks of 128) within the stated tolerance, all against the oracle."""

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


def _bits(rng, shape, scale):
    return O.rne_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _compare_q(q, ref, dq):
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(q.absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32))
    if dq:
        np.testing.assert_array_equal(q.scale_codes.cpu().numpy(), ref["scale_codes"])
        np.testing.assert_array_equal(q.group_absmax.cpu().numpy().view(np.uint32),
                                      ref["group_absmax"].view(np.uint32))


def _special_blocks():
    lv = O.FP4_LEVELS[:8].astype(np.float64)
    rows = []
    for i in range(7):  # values at and next to every magnitude midpoint, both signs, absmax 1
        f = np.float32((lv[i] + lv[i + 1]) / 2)
        vals = [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
        blk = np.zeros(64, dtype=np.float32)
        blk[:3] = vals
        blk[3] = 1.0
        blk[4:7] = [-v for v in vals]
        rows.append(blk)
    rows.append(np.zeros(64, dtype=np.float32))                          # all-zero block
    b = np.full(64, -0.0, dtype=np.float32); b[9] = 1e-3; rows.append(b)  # negative zeros
    b = np.full(64, -1e-9, dtype=np.float32); b[0] = 1.0; rows.append(b)  # tiny negatives round to -0
    b = (np.arange(1, 65, dtype=np.float32) * np.float32(1e-45)); rows.append(b)  # subnormals
    b = (np.linspace(-1, 1, 64) * 3e38).astype(np.float32); rows.append(b)  # near float max
    b = np.ones(64, dtype=np.float32); b[5] = np.nan; rows.append(b)      # non-finite blocks
    b = np.ones(64, dtype=np.float32); b[60] = -np.inf; rows.append(b)
    return np.stack(rows)


@pytest.mark.parametrize("block,dq,group", [(64, False, 256), (64, True, 256), (128, True, 256), (64, True, 5)])
def test_fp4_quantize_and_dequantize_match_oracle(F, block, dq, group):
    import torch

    rng = np.random.default_rng(501 + block + dq)
    w = (rng.standard_normal((96, 1024)) * 0.02).astype(np.float32)
    w.reshape(-1)[::997] *= 40
    sp = _special_blocks().reshape(-1)
    w.reshape(-1)[:sp.size] = sp
    q = F.nf4_quantize(U.f32(w), double_quant=dq, dq_group=group, block_size=block, quant_type="fp4")
    wd = F.nf4_dequantize(q)
    wb = F.nf4_dequantize_bf16(q)
    torch.cuda.synchronize()
    ref = O.quantize(w, double_quant=dq, dq_group=group, block_size=block, quant_type="fp4")
    got_s = q.absmax.cpu().numpy()
    nan = np.isnan(ref["absmax"])
    np.testing.assert_array_equal(np.isnan(got_s), nan)
    ref2 = dict(ref)
    ref2["absmax"] = np.where(nan, np.float32(0), ref["absmax"])
    q.absmax[torch.from_numpy(nan).to(q.absmax.device)] = 0.0
    if dq:
        gnan = np.isnan(ref["group_absmax"])
        np.testing.assert_array_equal(np.isnan(q.group_absmax.cpu().numpy()), gnan)
        ref2["group_absmax"] = np.where(gnan, np.float32(0), ref["group_absmax"])
        q.group_absmax[torch.from_numpy(gnan).to(q.group_absmax.device)] = 0.0
    _compare_q(q, ref2, dq)
    wref = O.dequantize(ref, w.shape, block_size=block, dq_group=group)
    got = wd.cpu().numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(wref))
    ok = ~np.isnan(wref)
    np.testing.assert_array_equal(got[ok].view(np.uint32), wref[ok].view(np.uint32))
    gb = wb.view(torch.int16).cpu().numpy().view(np.uint16)
    rb = O.rne_bf16_bits(np.where(ok, wref, np.float32(0)))
    np.testing.assert_array_equal(gb[ok], rb[ok])


def test_fp4_every_float32_in_unit_interval_gets_its_code(F):
    """Every float32 in [-1, 1] through the FP4 quantizer, 63 per block beside
    an element 1.0 (absmax 1, so the normalized value is the value itself).
    Expected codes: the sign bit, and the number of exact magnitude midpoints
    of the oracle's table strictly below |v| (the CPU pins tie this to the
    exact arg-min and its tie rule)."""
    import torch

    t64 = O.FP4_LEVELS[:8].astype(np.float64)
    mids = (t64[:-1] + t64[1:]) / 2
    ranges = [(0x00000000, 0x3F800000), (0x80000000, 0xBF800000)]
    per = 63
    chunk_blocks = 1 << 21
    d = U.dev()
    checked = 0
    for lo, hi in ranges:
        n = hi - lo + 1
        for c0 in range(0, n, per * chunk_blocks):
            cnt = min(per * chunk_blocks, n - c0)
            nblk = (cnt + per - 1) // per
            pad = nblk * per - cnt
            bits = torch.arange(lo + c0, lo + c0 + cnt, dtype=torch.int64, device=d)
            bits = torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits)
            if pad:
                bits = torch.cat([bits, torch.zeros(pad, dtype=torch.int64, device=d)])
            vals = bits.to(torch.int32).view(torch.float32).view(nblk, per)
            wt = torch.cat([torch.ones(nblk, 1, dtype=torch.float32, device=d), vals], dim=1).contiguous()
            q = F.nf4_quantize(wt, double_quant=False, quant_type="fp4")
            torch.cuda.synchronize()
            codes = O.unpack_codes(q.codes[:nblk * 32].cpu().numpy()).reshape(nblk, 64)
            absmax = q.absmax[:nblk].cpu().numpy()
            del q, wt, vals, bits
            assert np.all(absmax == 1.0)
            assert np.all(codes[:, 0] == 7)
            hv = (np.arange(lo + c0, lo + c0 + cnt, dtype=np.uint64)).astype(np.uint32).view(np.float32)
            mag = np.searchsorted(mids, np.abs(hv.astype(np.float64)), side="left").astype(np.uint8)
            want = mag | (np.signbit(hv).astype(np.uint8) << 3)
            got = codes[:, 1:].reshape(-1)[:cnt]
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, "value %r: code %d, expected %d" % (hv[bad[0]], got[bad[0]], want[bad[0]])
            checked += cnt
        print("range %08x..%08x checked" % (lo, hi), flush=True)
    assert checked == 2 * (0x3F800000 + 1)


@pytest.mark.parametrize("M", [1, 4, 16, 64, 300, 1100])
@pytest.mark.parametrize("block", [64, 128])
def test_fp4_layer_forward_backward(F, M, block):
    """Forward and backward on an FP4 weight at token counts that reach every
    product kernel (single-token GEMV, few-token kernels, tiled GEMMs)."""
    import torch

    out, inp, r, s = 4096, 1024, 16, 2.0
    rng = np.random.default_rng(601 + M + block)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = _bits(rng, (M, inp), 1.0)
    a = _bits(rng, (r, inp), 0.05)
    b = _bits(rng, (out, r), 0.01)
    dh = _bits(rng, (M, out), 1.0)
    q = F.nf4_quantize(U.f32(w), double_quant=True, block_size=block, quant_type="fp4")
    h, u = F.qlora_linear_forward(q, U.bf(x), U.bf(a), U.bf(b), s, want_u=True)
    dX, dA, dB = F.qlora_linear_backward(q, U.bf(x), U.bf(dh), U.bf(a), U.bf(b), s, u=u)
    torch.cuda.synchronize()
    ref = O.quantize(w, double_quant=True, block_size=block, quant_type="fp4")
    wb = O.compute_weight(ref, w.shape, block_size=block)
    href, uref = O.forward(wb, x, a, b, s)
    g = O.backward(wb, x, dh, a, b, s)
    U.assert_close("h", U.bf16_to_f64(h), href)
    U.assert_close("u", u.cpu().numpy(), uref)
    U.assert_close("dX", U.bf16_to_f64(dX), g["dX"])
    U.assert_close("dA", dA.cpu().numpy(), g["dA"])
    U.assert_close("dB", dB.cpu().numpy(), g["dB"])
    # the FP4 weight is not the NF4 one: the two quant types give different outputs
    wn = O.compute_weight(O.quantize(w, double_quant=True, block_size=block), w.shape, block_size=block)
    assert not np.array_equal(wn, wb)


def test_fp4_multi_adapter(F):
    import torch

    rng = np.random.default_rng(611)
    out, inp, r, n, M = 4096, 512, 16, 9, 700
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    x = _bits(rng, (M, inp), 1.0)
    ab = _bits(rng, (n, r, inp), 0.05)
    bb = _bits(rng, (n, out, r), 0.05)
    scales = np.linspace(0.25, 4.0, n).astype(np.float32)
    ids = rng.integers(-1, n + 1, size=M).astype(np.int32)
    q = F.nf4_quantize(U.f32(w), double_quant=True, quant_type="fp4")
    h = F.qlora_linear_forward_multi(q, U.bf(x), U.bf(ab), U.bf(bb), torch.from_numpy(scales).to(U.dev()),
                                     torch.from_numpy(ids).to(U.dev()))
    torch.cuda.synchronize()
    wb = O.compute_weight(O.quantize(w, double_quant=True, quant_type="fp4"), w.shape)
    href = O.forward_multi(wb, x, ab, bb, scales.astype(np.float64), ids)
    U.assert_close("h", U.bf16_to_f64(h), href)


def test_fp4_merge_and_requantize(F):
    import torch

    rng = np.random.default_rng(621)
    out, inp, r, s = 1000, 2048, 64, 2.0
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    a = _bits(rng, (r, inp), 0.05)
    b = _bits(rng, (out, r), 0.01)
    q = F.nf4_quantize(U.f32(w), double_quant=True, quant_type="fp4")
    ref = O.quantize(w, double_quant=True, quant_type="fp4")
    wm = F.qlora_merge(q, U.bf(a), U.bf(b), s)
    wz = F.qlora_merge(q, U.bf(a), U.bf(np.zeros_like(b)), s)
    torch.cuda.synchronize()
    wb = O.compute_weight(ref, w.shape)
    U.assert_close("merged", U.bf16_to_f64(wm), O.bf16_bits_to_f32(O.merge(wb, a, b, s)).astype(np.float64))
    # without the adapter the merge is the bf16 dequantization, bit for bit,
    # except that a -0 weight (code 8) plus the zero product is +0, in the
    # oracle's exact sum as in the kernel's fp32 one
    got = wz.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, O.merge(wb, a, np.zeros_like(b), s))
    deq = O.rne_bf16_bits(O.dequantize(ref, w.shape))
    assert np.all((got == deq) | ((deq == 0x8000) & (got == 0)))
    # the merged bf16 weight back to FP4 storage: the codes of the oracle on its fp32 values
    q2 = F.nf4_quantize(wm, double_quant=True, quant_type="fp4")
    torch.cuda.synchronize()
    wm32 = O.bf16_bits_to_f32(wm.view(torch.int16).cpu().numpy().view(np.uint16))
    _compare_q(q2, O.quantize(wm32, double_quant=True, quant_type="fp4"), True)
