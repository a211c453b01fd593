"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test ties one oracle function to a value the pages print, a closed form,
a brute-force computation in exact rational arithmetic, or a library routine,
chosen so that a plausible slip (a wrong level, index, sign, rounding mode or
operand order) fails at least one of them.  CPU only.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_from_fraction(q: Fraction) -> np.float32:
    # Python's Fraction -> float is correctly rounded to binary64; a quotient of
    # two binary32 numbers then rounds innocuously to binary32 (53 >= 2*24 + 2).
    return np.float32(float(q))


def _exact_code(w: np.float32) -> int:
    """Exact arg-min over the 16 levels, ties to the lower index (Fractions)."""
    wf = Fraction(float(w))
    best, bestd = None, None
    for k, t in enumerate(O.NF4_LEVELS):
        d = abs(wf - Fraction(float(t)))
        if bestd is None or d < bestd:
            best, bestd = k, d
    return best


# --------------------------------------------------------------------- table
def test_levels_agree_with_second_page_table():
    """Two independent printings of the levels agree to four decimals."""
    rows = []
    with open(os.path.join(GOLDEN, "nf4_levels_4dp.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                idx, binary, val = line.split()
                rows.append((int(idx), binary, float(val)))
    assert [r[0] for r in rows] == list(range(16))
    assert [r[1] for r in rows] == [format(i, "04b") for i in range(16)]
    got = np.round(O.NF4_LEVELS.astype(np.float64), 4)
    np.testing.assert_array_equal(got, np.array([r[2] for r in rows]))


def test_levels_invariants():
    t = O.NF4_LEVELS
    assert t.dtype == np.float32 and t.shape == (16,)
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    assert t[0] == -1.0 and t[7] == 0.0 and t[15] == 1.0
    assert np.count_nonzero(t == 0) == 1


def test_levels_are_normal_quantiles():
    """The levels are normalized standard-normal quantiles with equal-mass
    bins on each side of zero (8 positive, 7 negative, plus 0).  The offset of
    the outermost probability is not on the pages, so it is fitted here."""
    from scipy.optimize import minimize_scalar
    from scipy.stats import norm

    def levels(delta):
        pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
        neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
        v = np.sort(np.concatenate([pos, [0.0], neg]))
        return v / np.max(np.abs(v))

    res = minimize_scalar(lambda d: np.max(np.abs(levels(d) - O.NF4_LEVELS)),
                          bounds=(0.9, 0.999), method="bounded",
                          options={"xatol": 1e-10})
    assert res.fun < 2e-6


# --------------------------------------------------------- worked example
def test_worked_example_from_the_pages():
    g = _load("worked_example.json")
    w = np.array(g["W"], dtype=np.float32)
    codes, s = O.quantize_first_level(w, block_size=w.size)
    assert s.shape == (1,) and s[0] == np.float32(g["absmax"])
    wn = O.normalize(w.reshape(1, -1), s)
    np.testing.assert_array_equal(np.round(wn[0].astype(np.float64), 4), g["normalized_4dp"])
    assert codes.tolist() == g["codes"]
    packed = O.pack_codes(codes)
    assert packed.tolist() == g["packed_bytes"]
    assert O.unpack_codes(packed).tolist() == g["codes"]
    stored = packed.nbytes + s.nbytes
    assert w.nbytes == g["fp32_bytes"] and stored == g["quantized_bytes"]
    assert round(100 * (1 - stored / w.nbytes), 1) == g["reduction_percent"]


# ---------------------------------------------------- code search, exact
def test_nearest_code_matches_exact_rational_argmin():
    rng = np.random.default_rng(1)
    vals = list(rng.uniform(-1, 1, 3000).astype(np.float32))
    mids = [(Fraction(float(O.NF4_LEVELS[k])) + Fraction(float(O.NF4_LEVELS[k + 1]))) / 2
            for k in range(15)]
    for m in mids:  # the midpoints and their float32 neighbours
        f = np.float32(float(m))
        for v in (f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))):
            vals.append(v)
    vals += [np.float32(v) for v in (-1.0, 1.0, 0.0, -0.0, 1e-45, -1e-45, 1e-38)]
    arr = np.array(vals, dtype=np.float32)
    got = O.nearest_code(arr)
    want = np.array([_exact_code(v) for v in arr])
    np.testing.assert_array_equal(got, want)


def test_exact_ties_go_to_the_lower_level():
    ties = 0
    for k in range(15):
        m = (Fraction(float(O.NF4_LEVELS[k])) + Fraction(float(O.NF4_LEVELS[k + 1]))) / 2
        f = np.float32(float(m))
        if Fraction(float(f)) == m:
            ties += 1
            assert O.nearest_code(np.array([f]))[0] == k
    assert ties == 6  # midpoints 2|3, 6|7, 7|8, 9|10, 11|12, 13|14 are float32 values


def test_nearest_code_sweep_around_every_midpoint():
    """Every float32 within 4096 ulps of each midpoint, plus a random sample,
    against the midpoint formulation: code = #{k : midpoint_k < w'}."""
    t64 = O.NF4_LEVELS.astype(np.float64)
    mids = (t64[:-1] + t64[1:]) / 2  # exact in binary64
    chunks = []
    for m in mids:
        c = np.array([m], dtype=np.float32).view(np.int32)[0]
        span = np.arange(-4096, 4097, dtype=np.int64)  # adjacent bit patterns = adjacent floats
        chunks.append((c + span).astype(np.int32).view(np.float32))
    rng = np.random.default_rng(7)
    chunks.append(rng.uniform(-1, 1, 1_000_000).astype(np.float32))
    w = np.concatenate(chunks)
    w = w[(w >= -1) & (w <= 1)]
    want = np.searchsorted(mids, w.astype(np.float64), side="left")
    np.testing.assert_array_equal(O.nearest_code(w), want.astype(np.uint8))


def test_normalize_is_a_correctly_rounded_division():
    rng = np.random.default_rng(3)
    blocks = (rng.standard_normal((50, 64)) * 0.02).astype(np.float32)
    s = O.block_absmax(blocks)
    wn = O.normalize(blocks, s)
    for b in range(0, 50, 7):
        for j in range(64):
            q = Fraction(float(blocks[b, j])) / Fraction(float(s[b]))
            assert wn[b, j] == _f32_from_fraction(q)


def test_absmax_element_maps_to_plus_or_minus_one():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    codes, s = O.quantize_first_level(w)
    codes = codes.reshape(-1, 64)
    blocks = w.reshape(-1, 64)
    idx = np.argmax(np.abs(blocks), axis=1)
    at = codes[np.arange(codes.shape[0]), idx]
    sign = np.sign(blocks[np.arange(blocks.shape[0]), idx])
    assert np.all(np.where(sign > 0, at == 15, at == 0))
    qt = O.quantize(w, double_quant=False)
    wd = O.dequantize(qt, w.shape).reshape(-1, 64)
    np.testing.assert_array_equal(np.abs(wd[np.arange(wd.shape[0]), idx]), s)


def test_zero_block_and_signed_zero():
    w = np.zeros((2, 64), dtype=np.float32)
    w[0, 5] = -0.0
    w[1, :] = np.float32(0.01)
    w[1, 3] = -0.0
    codes, s = O.quantize_first_level(w)
    assert s[0] == 0 and np.all(codes[:64] == 7)
    assert codes[64 + 3] == 7 and np.all(np.delete(codes[64:], 3) == 15)
    qt = O.quantize(w, double_quant=True)
    np.testing.assert_array_equal(O.dequantize(qt, w.shape)[0], 0)


# ----------------------------------------------------------- round trips
def test_table_values_round_trip():
    """A block of s*T[k] values quantizes back to codes k and scale s, and
    dequantizes to the same float32 values (no double quant)."""
    rng = np.random.default_rng(5)
    for s in rng.uniform(1e-4, 10, 40).astype(np.float32):
        perm = rng.permutation(64) % 16
        w = (s * O.NF4_LEVELS[perm]).astype(np.float32)
        w[0] = s  # make sure the absmax element is present
        perm[0] = 15
        codes, sc = O.quantize_first_level(w)
        assert sc[0] == s
        np.testing.assert_array_equal(codes, perm)
        qt = O.quantize(w, double_quant=False)
        np.testing.assert_array_equal(O.dequantize(qt, w.shape), w)


@pytest.mark.parametrize("dq", [False, True])
def test_quantize_dequantize_quantize_is_stable(dq):
    rng = np.random.default_rng(11 + dq)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3, 7] = 0.9  # an outlier makes coarse scales in its DQ group
    qt = O.quantize(w, double_quant=dq)
    w1 = O.dequantize(qt, w.shape)
    qt2 = O.quantize(w1, double_quant=dq)
    np.testing.assert_array_equal(qt2["codes"], qt["codes"])
    if dq:
        np.testing.assert_array_equal(qt2["scale_codes"], qt["scale_codes"])
        np.testing.assert_array_equal(qt2["group_absmax"], qt["group_absmax"])
    np.testing.assert_array_equal(O.dequantize(qt2, w.shape), w1)


# ------------------------------------------------------ double quantization
def test_double_quant_properties():
    rng = np.random.default_rng(6)
    s = np.abs(rng.standard_normal(256 * 5 + 37)).astype(np.float32)
    s[100] = 0
    q, c = O.double_quantize_scales(s, 256)
    assert q.dtype == np.int8 and c.shape == (6,)
    assert np.all(q >= 0) and np.all(q <= 127)
    for g in range(6):
        sl = s[g * 256:(g + 1) * 256]
        assert c[g] == sl.max()
        assert q[g * 256 + int(np.argmax(sl))] == 127
        qg = q[g * 256:(g + 1) * 256].astype(np.int64)
        order = np.argsort(sl, kind="stable")
        assert np.all(np.diff(qg[order]) >= 0)  # monotone in the scale
    assert q[100] == 0
    dec = O.decode_scales(q, c, 256)
    gi = np.arange(s.size) // 256
    # an 8-bit absmax quantizer with 127 positive steps errs by at most half a step
    assert np.all(np.abs(dec.astype(np.float64) - s) <= c[gi].astype(np.float64) / 254 * (1 + 1e-6))


def test_double_quant_two_page_formulas_agree():
    """The n4n.ai listing divides by the absmax then multiplies by 127; the
    hashnode page forms 127/absmax first.  Both describe the same quantizer:
    they agree except on rare rounding boundaries."""
    rng = np.random.default_rng(8)
    s = np.abs(rng.standard_normal(200_000) * 0.02).astype(np.float32)
    q, c = O.double_quantize_scales(s, s.size)
    alt = np.rint((np.float32(127) / c[0]) * s).astype(np.int64)
    assert np.mean(alt != q) < 1e-4


def test_double_quant_single_global_constant():
    """group >= number of blocks reproduces the n4n.ai listing's one constant."""
    s = np.array([0.5, 0.25, 1.0, 0.125], dtype=np.float32)
    q, c = O.double_quantize_scales(s, 1024)
    assert c.tolist() == [1.0]
    assert q.tolist() == [64, 32, 127, 16]  # 63.5 -> 64, 31.75 -> 32, 15.875 -> 16


def test_double_quant_rounds_half_to_even():
    """torch's round() (the n4n.ai listing) sends exact halves to the even
    integer.  These float32 scales (bit patterns) give s/c*127 = k + 0.5
    exactly in float32 with c = 1, for even k."""
    bits = np.array([998310404, 1017201285, 1024533061, 1028760391], dtype=np.uint32)
    s = np.concatenate([bits.view(np.float32), np.array([1.0], dtype=np.float32)])
    assert ((s[:4] / s[4]) * np.float32(127)).astype(np.float32).tolist() == [0.5, 2.5, 4.5, 6.5]
    q, _ = O.double_quantize_scales(s, 256)
    assert q.tolist() == [0, 2, 4, 6, 127]


def _round_f32_exact(x: Fraction) -> Fraction:
    """The binary32 value nearest to the exact rational x (ties to even),
    subnormals included, as an exact Fraction.  Written from the definition:
    the spacing of binary32 values in [2^e, 2^(e+1)) is 2^(e-23), and below
    2^-126 it is 2^-149."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def _rint_half_even(x: Fraction) -> int:
    lo = x.numerator // x.denominator
    rem = x - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo


def test_exact_float32_rounding_helper():
    """The helper above against float32 values whose neighbours are known."""
    for v in (1.0, 0.1, 3.0e-39, 1.0e-45, 0.338, 127.0 / 3.0):
        f = np.float32(v)
        assert _round_f32_exact(Fraction(float(f))) == Fraction(float(f))
        up = np.nextafter(f, np.float32(np.inf))
        mid = (Fraction(float(f)) + Fraction(float(up))) / 2
        even = f if (int(np.array([f]).view(np.uint32)[0]) % 2 == 0) else up
        assert _round_f32_exact(mid) == Fraction(float(even))
        assert _round_f32_exact(mid - Fraction(1, 2 ** 200)) == Fraction(float(f))
        assert _round_f32_exact(mid + Fraction(1, 2 ** 200)) == Fraction(float(up))


@pytest.mark.parametrize("grouped", [True, False])
def test_double_quant_matches_the_page_listing_in_torch(grouped):
    """"QLoRA explained", "Double quantization": the scales are divided by
    their absmax, multiplied by 127, rounded (torch's round, half to even) and
    cast to int8, all in torch float32.  That listing, run as printed on
    torch's CPU tensors, against the oracle on 2^22 block scales whose
    constants are far from 1: in groups of 256 ("From LoRA to QLoRA",
    "Pillar 2"), and as the listing's single global constant."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    n = 1 << 22
    ng = n // 256
    # block absmax values as the first level makes them (the absmax of 64
    # normal weights is about 2.5 sigma), sigma spread over many binades
    sigma = 2.0 ** rng.uniform(-14.0, 3.0, ng)
    s = (np.abs(rng.standard_normal((ng, 256))) * sigma[:, None]).astype(np.float32).reshape(-1)
    st = torch.from_numpy(s.copy())
    if grouped:
        st = st.view(ng, 256)
        scale_absmax = st.abs().amax(dim=1, keepdim=True)
        q_page = (st / scale_absmax * 127).round().to(torch.int8).reshape(-1).numpy()
        c_page = scale_absmax.reshape(-1).numpy()
        q, c = O.double_quantize_scales(s, 256)
    else:
        scale_absmax = st.abs().max()
        q_page = (st / scale_absmax * 127).round().to(torch.int8).numpy()
        c_page = np.array([scale_absmax.item()], dtype=np.float32)
        q, c = O.double_quantize_scales(s, n)
    assert not np.any(c == 1.0)
    np.testing.assert_array_equal(c, c_page)
    np.testing.assert_array_equal(q, q_page)


def _dq_pairs_where_the_page_orders_differ(n_wanted=5):
    """Scale / constant pairs (c != 1) on which dividing first ("QLoRA
    explained") and forming 127/c first ("From LoRA to QLoRA", "Vanilla
    Uniform Quantization") give different codes."""
    rng = np.random.default_rng(42)
    c = (rng.uniform(1.0, 2.0, 4_000_000) * 2.0 ** rng.integers(-12, 3, 4_000_000)).astype(np.float32)
    s = (c * rng.uniform(0.0, 1.0, c.size)).astype(np.float32)
    div_first = np.rint(((s / c).astype(np.float32) * np.float32(127)).astype(np.float32))
    recip_first = np.rint(((np.float32(127) / c).astype(np.float32) * s).astype(np.float32))
    idx = np.nonzero(div_first != recip_first)[0]
    assert idx.size >= n_wanted
    return s, c, idx[:n_wanted]


def test_double_quant_order_by_exact_arithmetic():
    """q = rint(fl32(fl32(s/c) * 127)) evaluated in exact rational arithmetic
    with correctly rounded float32 steps, at constants c != 1: on random pairs
    and on pairs where the other page's order (127/c first) disagrees, so a
    swapped order fails here."""
    s, c, diff = _dq_pairs_where_the_page_orders_differ()
    rng = np.random.default_rng(43)
    pick = np.concatenate([diff, rng.choice(s.size, 400, replace=False)])
    ss, cc = s[pick], c[pick]
    # one group of two blocks per pair: the constant is c itself (s <= c)
    inter = np.empty(2 * pick.size, dtype=np.float32)
    inter[0::2], inter[1::2] = ss, cc
    q, cg = O.double_quantize_scales(inter, 2)
    np.testing.assert_array_equal(cg, cc)
    assert np.all(q[1::2] == 127)
    for i in range(pick.size):
        ratio = _round_f32_exact(Fraction(float(ss[i])) / Fraction(float(cc[i])))
        want = _rint_half_even(_round_f32_exact(ratio * 127))
        assert int(q[2 * i]) == want, (ss[i], cc[i])
    for i in range(diff.size):  # the other order really differs here
        recip = _round_f32_exact(Fraction(127) / Fraction(float(cc[i])))
        other = _rint_half_even(_round_f32_exact(recip * Fraction(float(ss[i]))))
        assert other != int(q[2 * i])


def test_double_quant_partial_last_group_exact():
    """A partial last group takes the maximum of its own blocks only."""
    rng = np.random.default_rng(44)
    s = (np.abs(rng.standard_normal(256 + 37)) * 0.013).astype(np.float32)
    q, c = O.double_quantize_scales(s, 256)
    assert c.shape == (2,) and c[1] == s[256:].max() and c[0] == s[:256].max()
    for b in list(range(0, 256, 17)) + list(range(256, 293)):
        cg = c[b // 256]
        ratio = _round_f32_exact(Fraction(float(s[b])) / Fraction(float(cg)))
        assert int(q[b]) == _rint_half_even(_round_f32_exact(ratio * 127))


def test_decode_scales_by_exact_arithmetic():
    """The scale decode (the step-by-step inverse of the double quant; the
    pages print no inverse) is s~ = fl32(fl32(q/127) * c): every code 0..127
    against 1,200 constants spread over 2^-126 .. 2^40 (subnormal results
    included), in exact rational arithmetic.  Plausible other orders of the
    same decode give different bits on this set, so each fails here."""
    rng = np.random.default_rng(45)
    nc = 1200
    cs = (rng.uniform(1.0, 2.0, nc) * 2.0 ** rng.integers(-126, 41, nc)).astype(np.float32)
    cs[:4] = np.array([1.0, 0.338, 1.0e-38, 3.0e38 / 127.0], dtype=np.float32)
    q = np.tile(np.arange(128, dtype=np.int8), nc)
    got = O.decode_scales(q, cs, 128).reshape(nc, 128)
    frac = [_round_f32_exact(Fraction(k, 127)) for k in range(128)]
    want = np.empty((nc, 128), dtype=np.float32)
    for i in range(nc):
        cf = Fraction(float(cs[i]))
        for k in range(128):
            want[i, k] = np.float32(float(_round_f32_exact(frac[k] * cf)))
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    # q = 127 gives the constant back exactly (the group's largest scale)
    np.testing.assert_array_equal(got[:, 127], cs)
    qf = np.arange(128, dtype=np.float32)[None, :]
    c2 = cs[:, None]
    others = {
        "q*c first": ((qf * c2).astype(np.float32) / np.float32(127)).astype(np.float32),
        "c/127 first": (qf * (c2 / np.float32(127)).astype(np.float32)).astype(np.float32),
    }
    for name, alt in others.items():
        assert np.any(alt.view(np.uint32) != want.view(np.uint32)), name


# -------------------------------------------- blocks of 128 (the pages allow 64 or 128)
def test_block128_codes_by_exact_argmin():
    """Blocks of 128 contiguous elements of the row-major flattening ("QLoRA
    explained", "The quantization backbone"; "From LoRA to QLoRA",
    "Block-Wise (Chunking) Quantization"): each block's absmax divides its
    own 128 elements, checked against exact rational arithmetic."""
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((3, 128)) * 0.03).astype(np.float32)
    codes, sc = O.quantize_first_level(w, 128)
    assert codes.shape == (384,) and sc.shape == (3,)
    codes = codes.reshape(3, 128)
    for b in range(3):
        blk = w[b]
        m = np.float32(np.max(np.abs(blk)))
        assert sc[b] == m
        for j in range(128):
            wn = _f32_from_fraction(Fraction(float(blk[j])) / Fraction(float(m)))
            assert codes[b, j] == _exact_code(wn)


def test_block128_equals_block64_when_halves_share_the_absmax():
    """If both 64-element halves of every 128-block hold the block's absmax,
    quantizing in blocks of 128 or of 64 gives the same codes, scales that
    repeat pairwise, and (with second-level groups covering the same
    elements) the same scale codes and group constants."""
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    blocks = w.reshape(-1, 128)
    m = np.max(np.abs(blocks), axis=1)
    blocks[:, 5] = m
    blocks[:, 64 + 9] = -m
    w = blocks.reshape(w.shape)
    a = O.quantize(w, double_quant=False, block_size=128)
    b = O.quantize(w, double_quant=False, block_size=64)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(np.repeat(a["absmax"], 2), b["absmax"])
    a = O.quantize(w, double_quant=True, block_size=128, dq_group=8)
    b = O.quantize(w, double_quant=True, block_size=64, dq_group=16)
    np.testing.assert_array_equal(np.repeat(a["scale_codes"], 2), b["scale_codes"])
    np.testing.assert_array_equal(a["group_absmax"], b["group_absmax"])
    np.testing.assert_array_equal(O.dequantize(a, w.shape, block_size=128, dq_group=8),
                                  O.dequantize(b, w.shape, block_size=64, dq_group=16))


def test_block128_storage_closed_form():
    """4 bits per code plus one fp32 scale per 128 weights (0.25 bit), or one
    int8 scale per 128 weights and one fp32 constant per 256 blocks."""
    n = 128 * 256 * 10
    cb, sb, gb = O.storage_bytes(n, double_quant=False, block_size=128)
    assert (cb, sb, gb) == (n // 2, 4 * n // 128, 0)
    cb, sb, gb = O.storage_bytes(n, double_quant=True, block_size=128)
    assert (cb, sb, gb) == (n // 2, n // 128, 4 * 10)
    assert 8 * (sb + gb) / n == 8 / 128 + 32 / (128 * 256)


# ------------------------------------------------- adapter-input dropout
def test_philox_known_answers():
    """The counter-based generator behind the dropout mask reproduces the
    known-answer vectors published with it."""
    g = _load("philox_kat.json")
    for v in g["vectors"]:
        ctr = [int(h, 16) for h in v["ctr"]]
        key = [int(h, 16) for h in v["key"]]
        got = O.philox4x32_10([ctr], [key])[0]
        assert ["%08x" % int(w) for w in got] == v["out"]


def test_dropout_threshold_and_keep_rate():
    assert O.dropout_threshold(0.0) == 0 and O.dropout_threshold(0.5) == 2 ** 31
    assert np.all(O.dropout_keep(3, 64, 0.0, 123))
    for p in (0.05, 0.5):
        keep = O.dropout_keep(512, 1024, p, 7)
        n = keep.size
        sigma = math.sqrt(p * (1 - p) / n)
        assert abs(keep.mean() - (1 - p)) < 6 * sigma
    a = O.dropout_keep(8, 128, 0.3, 1)
    assert np.array_equal(a, O.dropout_keep(8, 128, 0.3, 1))        # deterministic in the seed
    assert not np.array_equal(a, O.dropout_keep(8, 128, 0.3, 2))    # and depends on it
    assert np.array_equal(a[:4], O.dropout_keep(4, 128, 0.3, 1))     # element (m, k) depends on m*in + k only
    assert np.array_equal(a.reshape(-1)[:10], O.dropout_keep(1, 10, 0.3, 1)[0])  # also for a ragged tail


def test_dropout_element_uses_one_word_of_its_counter():
    """Element e of the flattened input is decided by output word e mod 4 of
    the generator at counter floor(e/4): checked one element at a time,
    against single calls of the generator, with a 64-bit seed."""
    seed, p = (5 << 32) | 77, 0.4
    thr = O.dropout_threshold(p)
    keep = O.dropout_keep(6, 64, p, seed).reshape(-1)
    for e in (0, 1, 2, 3, 4, 7, 63, 64, 201, 383):
        w = O.philox4x32_10([[e // 4, 0, 0, 0]], [[77, 5]])[0]
        assert keep[e] == (int(w[e % 4]) >= thr)


def test_dropout_p0_is_the_plain_layer():
    rng = np.random.default_rng(31)
    M, out, inp, r = 5, 24, 64, 4
    wb = rng.standard_normal((out, inp))
    x, dh = rng.standard_normal((M, inp)), rng.standard_normal((M, out))
    a, b = rng.standard_normal((r, inp)), rng.standard_normal((out, r))
    keep = O.dropout_keep(M, inp, 0.0, 5)
    h0, u0 = O.forward64(wb, x, a, b, 2.0)
    h1, u1 = O.forward_dropout64(wb, x, a, b, 2.0, keep, 0.0)
    np.testing.assert_array_equal(h0, h1)
    np.testing.assert_array_equal(u0, u1)
    g0 = O.backward64(wb, x, dh, a, b, 2.0)
    g1 = O.backward_dropout64(wb, x, dh, a, b, 2.0, keep, 0.0)
    for k in ("dX", "dA", "dB", "dU"):
        np.testing.assert_array_equal(g0[k], g1[k])


def test_dropout_backward_matches_finite_differences():
    """With the mask fixed the layer is linear in x, A and B, so central
    differences are exact up to rounding."""
    rng = np.random.default_rng(32)
    M, out, inp, r, p, s = 3, 7, 64, 3, 0.3, 2.0
    wb = rng.standard_normal((out, inp))
    x, dh = rng.standard_normal((M, inp)), rng.standard_normal((M, out))
    a, b = rng.standard_normal((r, inp)), rng.standard_normal((out, r))
    keep = O.dropout_keep(M, inp, p, 11)
    assert 0 < keep.sum() < keep.size
    g = O.backward_dropout64(wb, x, dh, a, b, s, keep, p)
    loss = lambda xx, aa, bb: float(np.sum(dh * O.forward_dropout64(wb, xx, aa, bb, s, keep, p)[0]))
    eps = 1e-3
    for name, arr, fn in (("dX", x, lambda v: loss(v, a, b)), ("dA", a, lambda v: loss(x, v, b)),
                          ("dB", b, lambda v: loss(x, a, v))):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            e = np.zeros_like(arr)
            e[idx] = eps
            num[idx] = (fn(arr + e) - fn(arr - e)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-7, atol=1e-7)


def test_storage_accounting_matches_the_pages():
    g = _load("accounting.json")["double_quant"]
    n = 64 * 256 * 100
    cb, sb, gb = O.storage_bytes(n, double_quant=False)
    over_plain = 8 * sb / n
    cb2, sb2, gb2 = O.storage_bytes(n, double_quant=True)
    over_dq = 8 * (sb2 + gb2) / n
    assert cb == cb2 == n // 2
    assert over_plain == g["overhead_bits_fp32_scales"]
    assert round(over_dq, 3) == g["overhead_bits_dq"]
    assert round(over_plain - over_dq, 3) == g["saving_bits"]


def test_lora_parameter_count_matches_the_pages():
    g = _load("accounting.json")["lora_params"]
    per = g["r"] * (g["d"] + g["k"])  # A is r x d, B is k x r
    assert per == g["per_matrix"]
    assert per * g["matrices_per_layer"] == g["per_layer"]
    total = per * g["matrices_per_layer"] * g["layers"]
    assert round(total / 1e6, 1) == g["total_millions"]
    assert round(total * 2 / 1e6, 1) == g["fp16_megabytes"]


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    a = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    edge = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F817FFF, 0x00000001,
                     0x80008000, 0x7F7FFFFF, 0x00400000, 0x80000000, 0],
                    dtype=np.uint32).view(np.float32)
    a = np.concatenate([a, edge])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.rne_bf16_bits(a), want)
    np.testing.assert_array_equal(O.bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


# ----------------------------------------------------------- layer: forward
def _small_layer(seed=0, M=3, inp=128, out=64, r=4):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    qt = O.quantize(w, double_quant=True)
    wb = O.compute_weight(qt, w.shape)
    x = O.rne_bf16(rng.standard_normal((M, inp)).astype(np.float32)).astype(np.float64)
    a = O.rne_bf16((rng.standard_normal((r, inp)) * 0.1).astype(np.float32)).astype(np.float64)
    b = O.rne_bf16((rng.standard_normal((out, r)) * 0.01).astype(np.float32)).astype(np.float64)
    return wb, x, a, b


def test_forward_against_exact_summation():
    wb, x, a, b = _small_layer()
    s = 2.0
    h, u = O.forward64(wb, x, a, b, s)
    for m in range(x.shape[0]):
        uu = [math.fsum(x[m, k] * a[j, k] for k in range(x.shape[1])) for j in range(a.shape[0])]
        for o in range(0, wb.shape[0], 5):
            base = math.fsum(x[m, k] * wb[o, k] for k in range(x.shape[1]))
            lora = math.fsum(uu[j] * b[o, j] for j in range(a.shape[0]))
            ref = base + s * lora
            assert abs(h[m, o] - ref) <= 1e-12 * max(1.0, abs(ref))
        np.testing.assert_allclose(u[m], uu, rtol=1e-12, atol=1e-14)


def test_zero_B_gives_the_base_output_exactly():
    wb, x, a, b = _small_layer(1)
    h, _ = O.forward64(wb, x, a, np.zeros_like(b), 2.0)
    np.testing.assert_array_equal(h, x @ wb.T)


def test_merge_identity():
    """x (Wb + s B A)^T equals the unmerged forward (deployment merge)."""
    wb, x, a, b = _small_layer(2)
    s = 0.25
    h, _ = O.forward64(wb, x, a, b, s)
    merged = wb + s * (b @ a)
    np.testing.assert_allclose(x @ merged.T, h, rtol=1e-12, atol=1e-14)


def _nearest_bf16_bits_exact(q) -> int:
    """Brute force: the bf16 value nearest to the rational q (ties to an even
    mantissa), found by comparing exact distances to the bf16 grid points
    around it."""
    import struct
    from fractions import Fraction

    f = float(q)
    hi16 = struct.unpack("<I", struct.pack("<f", f))[0] >> 16
    best = None
    for cand in range(max(hi16 - 2, 0), hi16 + 3):
        if (cand & 0x7F80) == 0x7F80:
            continue
        val = Fraction(struct.unpack("<f", struct.pack("<I", cand << 16))[0])
        key = (abs(val - q), cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_merge_by_exact_rational_arithmetic():
    """The merged bf16 weight against exact rational sums, rounded by brute
    force (mixed signs, so the bit-pattern neighbours cover both sides)."""
    from fractions import Fraction

    rng = np.random.default_rng(21)
    out, inp, r = 5, 64, 3
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    wb = O.compute_weight(O.quantize(w, double_quant=True), w.shape)
    a = O.rne_bf16_bits((rng.standard_normal((r, inp)) * 0.1).astype(np.float32))
    b = O.rne_bf16_bits((rng.standard_normal((out, r)) * 0.1).astype(np.float32))
    s = 0.5
    got = O.merge(wb, a, b, s)
    af, bf = O._bf(a), O._bf(b)
    for o in range(out):
        for i in range(inp):
            q = Fraction(wb[o, i]) + Fraction(s) * sum(Fraction(bf[o, j]) * Fraction(af[j, i]) for j in range(r))
            if q < 0:
                want = _nearest_bf16_bits_exact(-q) | 0x8000
            else:
                want = _nearest_bf16_bits_exact(q)
            assert int(got[o, i]) == want, (o, i, hex(int(got[o, i])), hex(want))


def test_merge_without_adapter_is_the_dequantized_weight():
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    qt = O.quantize(w, double_quant=True)
    wb = O.compute_weight(qt, w.shape)
    a = O.rne_bf16_bits(rng.standard_normal((4, 128)).astype(np.float32))
    b = O.rne_bf16_bits(rng.standard_normal((8, 4)).astype(np.float32))
    want = O.dequantize_bf16_bits(qt, w.shape)
    np.testing.assert_array_equal(O.merge(wb, a, np.zeros_like(b), 2.0), want)
    np.testing.assert_array_equal(O.merge(wb, a, b, 0.0), want)


def test_merged_weight_reproduces_the_forward():
    """x Wm^T with the merged bf16 weight equals the unmerged forward up to the
    rounding of the merged weight: each merged entry is within half a bf16
    ulp (2^-8 of its magnitude) of Wb + s B A, so the output error is at most
    |x| (2^-8 |Wb + s B A|)^T."""
    wb, x, a, b = _small_layer(6, M=4)
    s = 2.0
    ab, bb = O.rne_bf16_bits(a.astype(np.float32)), O.rne_bf16_bits(b.astype(np.float32))
    wm = O.bf16_bits_to_f32(O.merge(wb, ab, bb, s)).astype(np.float64)
    exact = wb + s * (O._bf(bb) @ O._bf(ab))
    assert np.all(np.abs(wm - exact) <= 2.0 ** -8 * np.abs(exact))
    h, _ = O.forward64(wb, x, a, b, s)
    bound = np.abs(x) @ (2.0 ** -8 * np.abs(exact)).T
    assert np.all(np.abs(x @ wm.T - h) <= bound + 1e-12)
    assert np.abs(x @ wm.T - h).max() > 0  # the rounding is visible, the bound is not vacuous


def test_single_token_is_a_matrix_vector_product():
    wb, x, a, b = _small_layer(3, M=1)
    h, u = O.forward64(wb, x, a, b, 2.0)
    ref = np.array([np.dot(wb[o], x[0]) + 2.0 * np.dot(b[o], a @ x[0]) for o in range(wb.shape[0])])
    np.testing.assert_allclose(h[0], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------- layer: backward
def test_backward_matches_finite_differences():
    """h is linear in x, A and B, so a central difference of L = <dH, h> is
    exact up to rounding for any step; compare every gradient entry."""
    wb, x, a, b = _small_layer(4, M=2, inp=64, out=16, r=3)
    s = 2.0
    rng = np.random.default_rng(12)
    dh = rng.standard_normal((2, 16))
    g = O.backward64(wb, x, dh, a, b, s)

    def loss(xx, aa, bb):
        return float(np.sum(dh * O.forward64(wb, xx, aa, bb, s)[0]))

    for name, arr in (("dX", x), ("dA", a), ("dB", b)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += 0.5
            m = arr.copy(); m[idx] -= 0.5
            args = {"dX": (p, a, b), "dA": (x, p, b), "dB": (x, a, p)}[name]
            argm = {"dX": (m, a, b), "dA": (x, m, b), "dB": (x, a, m)}[name]
            num[idx] = loss(*args) - loss(*argm)
        np.testing.assert_allclose(g[name], num, rtol=1e-9, atol=1e-11)


def test_backward_has_no_weight_gradient_and_du_is_consistent():
    wb, x, a, b = _small_layer(5)
    rng = np.random.default_rng(13)
    dh = rng.standard_normal((x.shape[0], wb.shape[0]))
    g = O.backward64(wb, x, dh, a, b, 0.5)
    assert set(g) == {"dX", "dA", "dB", "dU"}
    # dU is the gradient w.r.t. u = x A^T; chain rule through u gives dA and the LoRA part of dX
    np.testing.assert_allclose(g["dA"], g["dU"].T @ x, rtol=1e-12)
    np.testing.assert_allclose(g["dX"] - dh @ wb, g["dU"] @ a, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------- multi-adapter
def test_multi_adapter_reduces_to_single_adapter():
    rng = np.random.default_rng(14)
    out, inp, r, n, M = 32, 64, 4, 5, 40
    w = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    qt = O.quantize(w, double_quant=True)
    wb = O.compute_weight(qt, w.shape)
    xb = O.rne_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    ab = O.rne_bf16_bits((rng.standard_normal((n, r, inp)) * 0.05).astype(np.float32))
    bb = O.rne_bf16_bits((rng.standard_normal((n, out, r)) * 0.05).astype(np.float32))
    scales = np.array([2.0, 0.5, 1.0, 4.0, 8.0])
    ids = rng.integers(-1, n + 1, size=M)  # includes out-of-range ids
    h = O.forward_multi(wb, xb, ab, bb, scales, ids)
    for i in range(n):
        sel = ids == i
        if sel.any():
            hi, _ = O.forward(wb, xb[sel], ab[i], bb[i], scales[i])
            np.testing.assert_allclose(h[sel], hi, rtol=1e-12, atol=1e-14)
    bad = (ids < 0) | (ids >= n)
    assert bad.any()
    np.testing.assert_allclose(h[bad], O._bf(xb[bad]) @ wb.T, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- AdamW step
def test_adamw_matches_torch():
    """The library routine as the pin: torch.optim.AdamW (float64, CPU) over
    several steps with weight decay."""
    import torch

    rng = np.random.default_rng(30)
    n = 257
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 1e-2 for _ in range(5)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    tp = torch.nn.Parameter(torch.tensor(p0.copy(), dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = O.adamw_step(p, g, m, v, t, **hp)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
    st = opt.state[tp]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13)


def test_adamw_closed_forms():
    """With a constant gradient the bias-corrected moments are exactly g and
    g^2 at every step, so each step moves p by lr*g/(|g| + eps) (plus the
    decay); the first step from zero moments is the same closed form."""
    g = np.array([0.5, -2.0, 1e-3, 0.0])
    lr, eps, wd = 1e-2, 1e-8, 0.1
    p = np.array([1.0, -1.0, 0.25, 3.0])
    m = v = np.zeros(4)
    want = p.copy()
    for t in range(1, 6):
        p, m, v = O.adamw_step(p, g, m, v, t, lr, 0.9, 0.999, eps, wd)
        want = want * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
        np.testing.assert_allclose(p, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, g * (1 - 0.9 ** 5), rtol=1e-12)
    np.testing.assert_allclose(v, g * g * (1 - 0.999 ** 5), rtol=1e-12)


def test_tolerance_helper():
    ref = np.array([1.0, -2.0, 0.0, 3.0])
    ok, worst = O.tolerance_ok(ref * (1 + 5e-3), ref)
    assert ok and worst < 1
    ok, _ = O.tolerance_ok(ref + np.array([0, 0, 0.01, 0]), ref)
    assert not ok


def test_header_dropout_contract_matches_the_oracle():
    """The dropout mask as the public header states it (word e mod 4 of the
    generator at counter floor(e/4), kept iff the word is >= ceil(p 2^32)),
    and the header's own example (seed 0, p = 0.5, elements 0..7), against
    the oracle's mask."""
    hdr = open(os.path.join(os.path.dirname(GOLDEN), "..", "include", "nf4qlora.h")).read()
    flat = " ".join(" ".join(ln.strip().lstrip("/*").strip() for ln in hdr.splitlines()).split())
    assert "counter (lo, hi of floor(e/4), 0, 0)" in flat
    assert "element e is kept iff word w_(e mod 4) is >= ceil(p * 2^32)" in flat
    assert "e = m*in + k" in flat
    keep = O.dropout_keep(1, 8, 0.5, 0)[0]
    w0 = O.philox4x32_10([[0, 0, 0, 0]], [[0, 0]])[0]
    w1 = O.philox4x32_10([[1, 0, 0, 0]], [[0, 0]])[0]
    want = [int(v) >= 2 ** 31 for v in list(w0) + list(w1)]
    assert keep.tolist() == want


def test_non_finite_blocks_dequantize_to_nan():
    """A block holding Inf or NaN has no absmax scale: it is stored with
    scale NaN and level 0 everywhere (so all of it dequantizes to NaN); the
    other blocks are untouched, and with double quant the NaN scale's group
    gets constant NaN and codes 0 (all its weights NaN), the other groups
    what they get without it."""
    rng = np.random.default_rng(51)
    w = (rng.standard_normal((4, 64 * 8)) * 0.02).astype(np.float32)
    clean = O.quantize(w, double_quant=False)
    bad = w.copy()
    bad[0, 3] = np.inf
    bad[2, 64 * 5 + 9] = np.nan
    bad[3, 70] = -np.inf
    codes, s = O.quantize_first_level(bad)
    nb = [3 // 64, (2 * 512 + 64 * 5 + 9) // 64, (3 * 512 + 70) // 64]
    for b in range(s.size):
        if b in nb:
            assert np.isnan(s[b]) and np.all(codes[64 * b:64 * b + 64] == 7)
        else:
            assert s[b] == clean["absmax"][b]
            np.testing.assert_array_equal(codes[64 * b:64 * b + 64],
                                          O.unpack_codes(clean["codes"])[64 * b:64 * b + 64])
    d = O.dequantize(O.quantize(bad, double_quant=False), bad.shape).reshape(-1, 64)
    assert np.all(np.isnan(d[nb])) and not np.any(np.isnan(np.delete(d, nb, axis=0)))
    q, c = O.double_quantize_scales(s, 8)  # groups of 8 blocks = one matrix row each
    qc, cc = O.double_quantize_scales(clean["absmax"], 8)
    assert np.isnan(c[0]) and np.isnan(c[2]) and np.isnan(c[3]) and c[1] == cc[1]
    assert np.all(q[0:8] == 0) and np.all(q[16:32] == 0)
    np.testing.assert_array_equal(q[8:16], qc[8:16])
    dd = O.dequantize(O.quantize(bad, double_quant=True, dq_group=8), bad.shape, dq_group=8)
    assert np.all(np.isnan(dd[[0, 2, 3]])) and not np.any(np.isnan(dd[1]))


# ---------------------------------------------------------------- FP4 (E2M1)
# The published E2M1 element values (OCP Microscaling Formats v1.0, the FP4
# table): positive codes 0..7, negative codes 8..15 in the same order.
E2M1_PUBLISHED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp4_levels_are_the_published_e2m1_values_over_six():
    for c in range(16):
        v = E2M1_PUBLISHED[c & 7] * (-1.0 if c & 8 else 1.0)
        assert O.e2m1_value(c) == v
        want = _f32_from_fraction(Fraction(v).limit_denominator(2) / 6)
        assert O.FP4_LEVELS[c] == want, c
        assert np.signbit(O.FP4_LEVELS[c]) == bool(c & 8)
    assert O.FP4_LEVELS[7] == 1.0 and O.FP4_LEVELS[15] == -1.0
    assert np.all(np.diff(O.FP4_LEVELS[:8]) > 0)


def _exact_fp4_code(w: np.float32) -> int:
    """Exact rational arg-min of |w| over the 8 magnitudes, ties to the even
    code, sign bit of w."""
    m = abs(Fraction(float(w)))
    d = [abs(m - Fraction(float(t))) for t in O.FP4_LEVELS[:8]]
    best = min(d)
    cands = [k for k in range(8) if d[k] == best]
    k = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
    return k + (8 if np.signbit(w) else 0)


def test_fp4_code_matches_exact_rational_argmin():
    rng = np.random.default_rng(401)
    w = rng.uniform(-1, 1, 3000).astype(np.float32)
    lv = O.FP4_LEVELS[:8].astype(np.float64)
    mids = []
    for i in range(7):  # around every midpoint, a few ulps each side
        mid = np.float32((lv[i] + lv[i + 1]) / 2)
        for k in range(-3, 4):
            v = mid
            for _ in range(abs(k)):
                v = np.nextafter(v, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
            mids += [v, -v]
    w = np.concatenate([w, np.array(mids, dtype=np.float32), O.FP4_LEVELS, np.float32([0.0, -0.0, 1e-30, -1e-30])])
    got = O.nearest_code_fp4(w)
    want = np.array([_exact_fp4_code(v) for v in w], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_fp4_exact_ties_go_to_the_even_code():
    # of the seven midpoints only the one between 0 and fl32(1/12) is a
    # float32 value; there the even code is also the lower one (0)
    lv = O.FP4_LEVELS[:8]
    hit = 0
    for i in range(7):
        mid = (Fraction(float(lv[i])) + Fraction(float(lv[i + 1]))) / 2
        f = np.float32(float(mid))
        if Fraction(float(f)) != mid:
            continue  # not a float32: no float32 input can tie there
        hit += 1
        even = i if i % 2 == 0 else i + 1
        assert O.nearest_code_fp4(np.float32([f]))[0] == even
        assert O.nearest_code_fp4(np.float32([-f]))[0] == even + 8
    assert hit == 1


def test_fp4_signed_zero_and_zero_block():
    w = np.zeros(64, dtype=np.float32)
    w[3] = -0.0
    codes, s = O.quantize_first_level(w, quant_type="fp4")
    assert s[0] == 0 and np.all(codes == 0)  # all-zero block: +0 everywhere
    w = np.full(64, 1e-9, dtype=np.float32)
    w[0], w[1] = 1.0, -1e-9
    codes, s = O.quantize_first_level(w, quant_type="fp4")
    assert codes[0] == 7 and codes[2] == 0 and codes[1] == 8  # -tiny rounds to -0


def test_fp4_grid_values_round_trip():
    # a block holding s * level for every code (s a power of two, so every
    # product and quotient is exact) quantizes to those codes and back
    for s in (np.float32(1.0), np.float32(0.25), np.float32(2.0 ** -20)):
        codes = np.array([c for c in range(16) if c != 8] * 5)[:64]
        w = (O.FP4_LEVELS[codes] * s).astype(np.float32)
        q = O.quantize(w, double_quant=False, quant_type="fp4")
        np.testing.assert_array_equal(O.unpack_codes(q["codes"]), codes)
        np.testing.assert_array_equal(O.dequantize(q, w.shape), w)


def test_fp4_error_bound_and_differs_from_nf4():
    rng = np.random.default_rng(402)
    w = (rng.standard_normal(64 * 200) * 0.02).astype(np.float32)
    q = O.quantize(w, double_quant=False, quant_type="fp4")
    d = O.dequantize(q, w.shape)
    s = np.repeat(q["absmax"], 64)
    # the largest gap between neighbouring levels is 1/3 (between 2/3 and 1);
    # one fl32 rounding of w/s and one of s*T add at most a few ulps of s
    assert np.all(np.abs(d - w) <= s * (1.0 / 6) * (1 + 1e-6) + 4 * np.spacing(s))
    qn = O.quantize(w, double_quant=False)
    assert not np.array_equal(q["codes"], qn["codes"])
    np.testing.assert_array_equal(q["absmax"], qn["absmax"])


def test_fp4_non_finite_block_dequantizes_to_nan():
    w = np.ones(128, dtype=np.float32) * 0.5
    w[70] = np.inf
    q = O.quantize(w, double_quant=False, quant_type="fp4")
    assert np.all(O.unpack_codes(q["codes"])[64:] == 0) and np.isnan(q["absmax"][1])
    d = O.dequantize(q, w.shape)
    assert np.all(np.isnan(d[64:])) and np.all(d[:64] == 0.5)
