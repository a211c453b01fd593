"""CPU oracle for the NF4 QLoRA linear layer (test infrastructure only).

This module is the plain, slow definition that the HIP library is checked
against.  It is *test infrastructure*: only the test-suite, the smoke check and
the benchmark's CPU-baseline leg may import it.  It shares no code, table or
constant with the GPU library; the only thing both sides consume is the seeded
input generator, which holds none of the method's arithmetic.

Sources (cited by page title and section):

* "QLoRA Finetuner" (mrtz.app), section "2. Block-by-Block NormalFloat4 (NF4)
  Quantization": 64-element blocks, absmax scale per block, division by the
  scale, nearest of 16 NF4 levels, dequantization as scale times level; section
  "1. Low-Rank Adaptation (LoRA)": the forward h = W0 x + (alpha/r) B(A x).
* "QLoRA explained: fine-tuning in 4-bit precision" (n4n.ai), section "Common
  misconceptions" (the 16 NF4 levels), section "Double quantization" (int8
  quantization of the block scales by their absmax, times 127, rounded),
  section "The LoRA adapter path" (tensor layout x @ W^T, (x @ A^T) @ B^T *
  scale, dequantized weight cast to bfloat16, gradients only into A and B).
* "Parameter-Efficient Fine-Tuning: From LoRA to QLoRA" (hashnode), section
  "Pillar 1: 4-bit NormalFloat (NF4) Quantization" (level table, worked
  example, nibble packing with the first element in the high nibble) and
  section "Pillar 2: Double Quantization (DQ)" (8-bit scales, groups of 256).
* Same page, section "The Real-World Bottleneck: Multi-Tenant AI at Scale":
  one resident base with a per-request adapter chosen by client id.
* "How Fine-Tuning LLMs with LoRA and QLoRA Works" (instagit), FAQ on merging
  adapters into the base weights (W + (alpha/r) B A), and "QLoRA explained",
  section "Merging and deploying" (a standalone 16-bit model): ``merge``.
* "QLoRA Finetuner", section "1. Low-Rank Adaptation (LoRA)", and the
  adapter-branch diagram of the same page: dropout on the input of the
  adapter branch only, h = W0 x + (alpha/r) B(A(dropout(x))); "QLoRA
  explained" sets lora_dropout = 0.05.  The pages give no random number
  generator: ``philox4x32_10`` is the published counter-based generator of
  Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
  3" (SC 2011), and ``dropout_keep`` the reading stated there (each
  counter's four output words serve four consecutive elements).
* "QLoRA Specification for EMEP Fine-Tuning" ("GPU Orchestration": adapters
  and optimizer state in full precision), "QLoRA explained" ("Paged
  optimizers": the Adam moments of the LoRA parameters paged to host memory):
  ``adamw_step``.

Precision: every step the method states in float32 is computed with NumPy
float32 elementwise operations (each one IEEE round-to-nearest-even).  All
products and sums of the linear algebra are computed in float64 from the exact
bf16/fp32 input values.  The code search is an exact arg-min (see
``nearest_code``).  Readings of points the pages leave open are marked
"READING" in the docstrings.

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
the pages print, closed forms, brute force or library routines.  The double
quant is pinned to the page's own listing run in torch float32 and, operation
order included, to exact rational arithmetic at constants other than 1.  The
decode of the double-quantized scale (``decode_scales``) has no worked value on
the pages (they print no inverse); its reading is pinned by exact rational
evaluation over every code and by the round-trip identities.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# The 16 NF4 levels, as printed (decimal) in "QLoRA explained", section "Common
# misconceptions"; the same table to four decimals is in "Parameter-Efficient
# Fine-Tuning: From LoRA to QLoRA", section "Pillar 1", "NF4 Level Lookup
# Table".  Index 0..15 is the 4-bit code.
# ---------------------------------------------------------------------------
NF4_LEVELS = np.array(
    [
        -1.0,
        -0.6961928009986877,
        -0.5250730514526367,
        -0.39491748809814453,
        -0.28444138169288635,
        -0.18477343022823334,
        -0.09105003625154495,
        0.0,
        0.07958029955625534,
        0.16093020141124725,
        0.24611230194568634,
        0.33791524171829224,
        0.44070982933044434,
        0.5626170039176941,
        0.7229568362236023,
        1.0,
    ],
    dtype=np.float32,
)

# ---------------------------------------------------------------------------
# FP4, the other 4-bit quant type ("QLoRA Specification for EMEP Fine-Tuning",
# "Hyperparameters": nf4 or fp4).  The pages say only that FP4 is an
# IEEE-style exponent/mantissa format ("QLoRA explained", "Common
# misconceptions").  READING: the 4-bit float with one sign, two exponent
# (bias 1) and one mantissa bit, no infinities or NaN -- the E2M1 element type
# of the OCP Microscaling Formats specification (v1.0) -- with the code being
# its bit pattern; its values are divided by their maximum, 6, so that the
# block's absmax maps to +-1 exactly as with NF4.
# ---------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """Value of the E2M1 bit pattern ``code`` (0..15): sign bit 3, exponent
    bits 2..1, mantissa bit 0; exponent field 0 is subnormal (m * 2**-1),
    otherwise 2**(e - 1) * (1 + m / 2)."""
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m * 0.5)
    return sign * mag


# fl32(value / 6): one float32 division of exact operands
FP4_LEVELS = np.array([np.float32(e2m1_value(c)) / np.float32(6) for c in range(16)], dtype=np.float32)

QUANT_TYPES = ("nf4", "fp4")


def levels(quant_type: str = "nf4") -> np.ndarray:
    if quant_type == "nf4":
        return NF4_LEVELS
    if quant_type == "fp4":
        return FP4_LEVELS
    raise ValueError("quant type %r" % (quant_type,))


BLOCK_SIZE = 64  # "QLoRA Finetuner", section 2: static blocks of 64 elements
DQ_GROUP = 256  # "From LoRA to QLoRA", Pillar 2: second pass block size 256


def _as_f32(a):
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("expected float32 input, got %s" % a.dtype)
    return a


# ---------------------------------------------------------------------------
# bf16 rounding (the compute dtype): "QLoRA explained", "The LoRA adapter
# path" casts the dequantized weight to bfloat16; "QLoRA Specification for
# EMEP Fine-Tuning", "Hyperparameters", names bfloat16 the compute dtype.
# ---------------------------------------------------------------------------
def rne_bf16_bits(f32) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest, ties to even.

    Written from the definition: keep the top 16 bits of the binary32 pattern,
    rounding on the 16 dropped bits.  Only finite inputs are meaningful here.
    """
    a = _as_f32(f32)
    u = a.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    top = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((top & 1) == 1))
    return ((top + up.astype(np.uint64)) & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bfloat16 bit pattern -> the float32 of the same value (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def rne_bf16(f32) -> np.ndarray:
    """float32 -> float32 holding the bf16-rounded value."""
    return bf16_bits_to_f32(rne_bf16_bits(f32))


# ---------------------------------------------------------------------------
# Quantization, first level ("QLoRA Finetuner", section 2; "From LoRA to QLoRA",
# "Block-Wise (Chunking) Quantization" and the worked example).
# ---------------------------------------------------------------------------
def split_blocks(w, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Flatten row-major and cut into contiguous blocks of ``block_size``.

    READING: a tensor whose size is not a multiple of the block size is
    rejected (the page's reshape into (n_blocks, block_size) admits no partial
    block).
    """
    a = _as_f32(w).reshape(-1)
    if a.size % block_size:
        raise ValueError("element count %d is not a multiple of %d" % (a.size, block_size))
    return a.reshape(-1, block_size)


def block_absmax(blocks) -> np.ndarray:
    """s_i = max_j |w_ij| per block (exact; a maximum does not round)."""
    return np.max(np.abs(_as_f32(blocks)), axis=1)


def normalize(blocks, absmax) -> np.ndarray:
    """w'_ij = w_ij / s_i as one float32 division.

    READING: a block whose absmax is 0 holds only zeros; its normalized values
    are defined as 0 (the division 0/0 is not taken).
    """
    b = _as_f32(blocks)
    s = _as_f32(absmax)
    safe = np.where(s == 0, np.float32(1), s).astype(np.float32)
    out = (b / safe[:, None]).astype(np.float32)
    out[s == 0, :] = np.float32(0)
    return out


def nearest_code(wn) -> np.ndarray:
    """Index of the NF4 level nearest to each normalized value.

    Distances |w' - T[k]| are formed in float64.  For float32 w' in [-1, 1]
    that difference is exact whenever it can decide the minimum (both terms
    are within a factor 2**29 of each other near every midpoint; far from the
    midpoints the winner is unambiguous), so this is the exact arg-min.

    READING: the pages do not say how an exact tie between two levels is
    broken; the tie goes to the lower index (first minimum).
    """
    w = _as_f32(wn).astype(np.float64)
    d = np.abs(w[..., None] - NF4_LEVELS.astype(np.float64))
    return np.argmin(d, axis=-1).astype(np.uint8)


def nearest_code_fp4(wn) -> np.ndarray:
    """FP4 code of each normalized value: the sign bit of w' and the nearest
    of the eight magnitudes FP4_LEVELS[0..7] to |w'|.

    As in ``nearest_code`` the distances are exact where they decide.
    READING: IEEE-style conversion keeps the sign (a zero or a value that
    rounds to zero keeps the sign of w') and breaks an exact tie to the even
    code (mantissa bit 0), as IEEE round-to-nearest-even does.
    """
    w = _as_f32(wn)
    mag = np.abs(w.astype(np.float64))
    lv = FP4_LEVELS[:8].astype(np.float64)
    d = np.abs(mag[..., None] - lv)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among the tied candidates (at most two, adjacent) take the even one
    even = cand & ((np.arange(8) & 1) == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    neg = np.signbit(w)
    return (code + 8 * neg).astype(np.uint8)


def pack_codes(codes) -> np.ndarray:
    """Two 4-bit codes per byte, element 2i in the high nibble
    ("From LoRA to QLoRA", worked example, "Byte Packing")."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        raise ValueError("odd number of codes")
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0xF
    return out


def zero_code(quant_type: str = "nf4") -> int:
    """The code of level 0.0: 7 for NF4, 0 (+0) for FP4."""
    return 7 if quant_type == "nf4" else 0


def quantize_first_level(w, block_size: int = BLOCK_SIZE, quant_type: str = "nf4"):
    """Blockwise 4-bit quantization: returns (codes[unpacked], absmax[fp32]).

    READING (the pages assume finite weights): a block that holds Inf or NaN
    has no absmax scale; it is stored with scale NaN and the code of level 0
    (7 for NF4, 0 for FP4) for every element, so all of it dequantizes to NaN.
    An all-zero block gets that code too.
    """
    levels(quant_type)
    blocks = split_blocks(w, block_size)
    bad = ~np.all(np.isfinite(blocks), axis=1)
    clean = np.where(bad[:, None], np.float32(0), blocks).astype(np.float32)
    s = block_absmax(clean)
    wn = normalize(clean, s)
    codes = nearest_code(wn) if quant_type == "nf4" else nearest_code_fp4(wn)
    codes[s == 0, :] = zero_code(quant_type)  # all-zero block: every normalized value is 0 -> level 0.0
    s[bad] = np.float32(np.nan)
    return codes.reshape(-1), s


# ---------------------------------------------------------------------------
# Double quantization ("QLoRA explained", section "Double quantization";
# "From LoRA to QLoRA", section "Pillar 2").
# ---------------------------------------------------------------------------
def double_quantize_scales(absmax, group: int = DQ_GROUP):
    """Quantize the fp32 block scales to int8, one fp32 constant per group.

    q_b = round_half_even( fl32( fl32(s_b / c_g) * 127 ) ),  c_g = max s_b.

    READINGS: group size 256 as on "From LoRA to QLoRA" (the n4n.ai listing
    uses one global constant, i.e. group >= number of blocks); the order
    divide-then-multiply of the n4n.ai listing; the last group may be partial;
    a group whose constant is 0 gets codes 0; a group holding a NaN scale (a
    block that held Inf or NaN) gets constant NaN and codes 0, so every
    weight of the group dequantizes to NaN.
    """
    s = _as_f32(absmax).reshape(-1)
    nb = s.size
    ng = (nb + group - 1) // group
    c = np.zeros(ng, dtype=np.float32)
    q = np.zeros(nb, dtype=np.int8)
    for g in range(ng):
        sl = s[g * group:(g + 1) * group]
        if np.any(np.isnan(sl)):
            c[g] = np.float32(np.nan)
            continue
        cg = np.max(sl) if sl.size else np.float32(0)  # scales are >= 0
        c[g] = cg
        if cg == 0:
            continue
        ratio = (sl / cg).astype(np.float32)
        scaled = (ratio * np.float32(127)).astype(np.float32)
        q[g * group:(g + 1) * group] = np.rint(scaled).astype(np.int8)
    return q, c


def decode_scales(q, c, group: int = DQ_GROUP) -> np.ndarray:
    """s~_b = fl32( fl32(q_b / 127) * c_g ).

    READING: the pages give no inverse of the scale quantization (no worked
    value exists); this is the step-by-step reverse of
    ``double_quantize_scales``, two correctly rounded float32 steps.  Pinned
    by exact rational evaluation of those two steps for every code 0..127 and
    constants over the whole float32 range, and by round-trip identities.
    """
    qf = np.asarray(q, dtype=np.int8).astype(np.float32)
    cc = _as_f32(c)
    gidx = np.arange(qf.size) // group
    frac = (qf / np.float32(127)).astype(np.float32)
    return (frac * cc[gidx]).astype(np.float32)


def quantize(w, double_quant: bool, block_size: int = BLOCK_SIZE, dq_group: int = DQ_GROUP,
             quant_type: str = "nf4"):
    """The full storage format: dict(codes=packed u8, absmax, scale_codes,
    group_absmax, quant_type)."""
    codes, s = quantize_first_level(w, block_size, quant_type)
    out = {"codes": pack_codes(codes), "absmax": s, "scale_codes": None, "group_absmax": None,
           "quant_type": quant_type}
    if double_quant:
        q, c = double_quantize_scales(s, dq_group)
        out["scale_codes"] = q
        out["group_absmax"] = c
    return out


def block_scales(qt, block_size: int = BLOCK_SIZE, dq_group: int = DQ_GROUP) -> np.ndarray:
    """Per-block scale used by dequantization: s_b, or its DQ decode."""
    if qt.get("scale_codes") is not None:
        return decode_scales(qt["scale_codes"], qt["group_absmax"], dq_group)
    return _as_f32(qt["absmax"])


def dequantize(qt, shape, block_size: int = BLOCK_SIZE, dq_group: int = DQ_GROUP) -> np.ndarray:
    """w~ = fl32(scale_b * T[code])  ("QLoRA Finetuner", section 2, last item),
    T the level table of the weight's quant type (NF4 unless stated)."""
    codes = unpack_codes(qt["codes"])
    sc = block_scales(qt, block_size, dq_group)
    per_elem = np.repeat(sc, block_size)
    w = (per_elem * levels(qt.get("quant_type", "nf4"))[codes]).astype(np.float32)
    return w.reshape(shape)


def dequantize_bf16_bits(qt, shape, **kw) -> np.ndarray:
    return rne_bf16_bits(dequantize(qt, shape, **kw))


def compute_weight(qt, shape, **kw) -> np.ndarray:
    """Wb = bf16(w~) as float64: the weight every product of the layer uses."""
    return bf16_bits_to_f32(dequantize_bf16_bits(qt, shape, **kw)).astype(np.float64)


# ---------------------------------------------------------------------------
# The layer ("QLoRA Finetuner", section 1; "QLoRA explained", "The LoRA adapter
# path").  Layout: W [out, in], x [M, in], A [r, in], B [out, r], h [M, out].
# Inputs x, A, B, dH are bf16 bit patterns (uint16); everything is float64.
# ---------------------------------------------------------------------------
def _bf(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def lora_down(x_bits, a_bits) -> np.ndarray:
    """u = x A^T  [M, r]."""
    return _bf(x_bits) @ _bf(a_bits).T


def forward64(wb, x, a, b, scale: float):
    """h = x Wb^T + scale * (x A^T) B^T on float64 arrays.  Returns (h, u).

    Dropout on the adapter branch is the identity (p = 0).
    """
    x = np.asarray(x, dtype=np.float64)
    u = x @ np.asarray(a, dtype=np.float64).T
    h = x @ np.asarray(wb, dtype=np.float64).T + float(scale) * (u @ np.asarray(b, dtype=np.float64).T)
    return h, u


def forward(wb, x_bits, a_bits, b_bits, scale: float):
    """The layer forward on bf16 inputs (bit patterns); float64 result (h, u)."""
    return forward64(wb, _bf(x_bits), _bf(a_bits), _bf(b_bits), scale)


def backward64(wb, x, dh, a, b, scale: float):
    """Gradients of h = x Wb^T + s (x A^T) B^T for upstream dH (float64 arrays).

    The dequantized weight is a constant ("QLoRA explained", "The LoRA adapter
    path": no gradient into the 4-bit storage), so there is no dW.  Plain
    calculus on the forward gives, with u = x A^T:
        dU = s dH B,   dB = s dH^T u,   dA = dU^T x,   dX = dH Wb + dU A.
    Returns dict(dX, dA, dB, dU) in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s = float(scale)
    u = x @ a.T
    du = s * (dh @ b)
    db = s * (dh.T @ u)
    da = du.T @ x
    dx = dh @ np.asarray(wb, dtype=np.float64) + du @ a
    return {"dX": dx, "dA": da, "dB": db, "dU": du}


def backward(wb, x_bits, dh_bits, a_bits, b_bits, scale: float):
    """The layer backward on bf16 inputs (bit patterns); float64 results."""
    return backward64(wb, _bf(x_bits), _bf(dh_bits), _bf(a_bits), _bf(b_bits), scale)


# ---------------------------------------------------------------------------
# LoRA dropout on the adapter input ("QLoRA Finetuner", section 1 and its
# adapter-branch diagram).  READING (the pages name dropout and its rate
# only): inverted dropout, an element kept with probability 1 - p and the kept
# ones scaled by 1/(1 - p); element e = m*in + k of x [M, in] takes output
# word e mod 4 of Philox-4x32-10 at counter (lo, hi of floor(e/4), 0, 0) and
# key (lo, hi of the 64-bit seed): kept iff that word >= ceil(p 2^32).  (All
# four words of a counter are used, one per element.)
# ---------------------------------------------------------------------------
_PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers (Salmon et al. 2011)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key schedule increments (golden ratio, sqrt 3 - 1)


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox-4x32 with 10 rounds on arrays of counters [n, 4] and keys [n, 2]
    (uint32): each round multiplies words 0 and 2 by the two multipliers into
    64-bit products, and the new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
    hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key advances by the two increments
    between rounds."""
    c = np.array(ctr, dtype=np.uint64).reshape(-1, 4)
    k = np.array(key, dtype=np.uint64).reshape(-1, 2)
    mask = np.uint64(0xFFFFFFFF)
    for rnd in range(10):
        if rnd:
            k = (k + np.array(_PHILOX_W, dtype=np.uint64)) & mask
        p0 = c[:, 0] * np.uint64(_PHILOX_M[0])
        p1 = c[:, 2] * np.uint64(_PHILOX_M[1])
        c = np.stack([(p1 >> np.uint64(32)) ^ c[:, 1] ^ k[:, 0], p1 & mask,
                      (p0 >> np.uint64(32)) ^ c[:, 3] ^ k[:, 1], p0 & mask], axis=1)
    return c.astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """ceil(p 2^32) for p in [0, 1): the smallest output word that is dropped."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout rate must lie in [0, 1)")
    return int(math.ceil(float(p) * 4294967296.0))


def dropout_keep(M: int, inp: int, p: float, seed: int) -> np.ndarray:
    """Boolean keep mask [M, inp] of the adapter-input dropout."""
    n = M * inp
    idx = np.arange((n + 3) // 4, dtype=np.uint64)   # counters
    ctr = np.zeros((idx.size, 4), dtype=np.uint64)
    ctr[:, 0] = idx & np.uint64(0xFFFFFFFF)
    ctr[:, 1] = idx >> np.uint64(32)
    key = np.empty((idx.size, 2), dtype=np.uint64)
    key[:, 0] = seed & 0xFFFFFFFF
    key[:, 1] = (seed >> 32) & 0xFFFFFFFF
    words = philox4x32_10(ctr, key).reshape(-1)[:n].astype(np.uint64)   # word e mod 4 of counter e // 4
    return (words >= np.uint64(dropout_threshold(p))).reshape(M, inp)


def forward_dropout64(wb, x, a, b, scale: float, keep, p: float):
    """h = x Wb^T + s (dropout(x) A^T) B^T with dropout(x) = keep * x / (1 - p)
    (float64).  Returns (h, u) with u = dropout(x) A^T."""
    x = np.asarray(x, dtype=np.float64)
    xd = np.where(keep, x, 0.0) / (1.0 - p)
    u = xd @ np.asarray(a, dtype=np.float64).T
    h = x @ np.asarray(wb, dtype=np.float64).T + float(scale) * (u @ np.asarray(b, dtype=np.float64).T)
    return h, u


def backward_dropout64(wb, x, dh, a, b, scale: float, keep, p: float):
    """Gradients of the dropout forward for upstream dH (float64): with
    xd = dropout(x) and u = xd A^T, dU = s dH B, dB = s dH^T u, dA = dU^T xd,
    dX = dH Wb + keep * (dU A) / (1 - p)."""
    x = np.asarray(x, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s = float(scale)
    xd = np.where(keep, x, 0.0) / (1.0 - p)
    u = xd @ a.T
    du = s * (dh @ b)
    db = s * (dh.T @ u)
    da = du.T @ xd
    dx = dh @ np.asarray(wb, dtype=np.float64) + np.where(keep, du @ a, 0.0) / (1.0 - p)
    return {"dX": dx, "dA": da, "dB": db, "dU": du}


def merge(wb, a_bits, b_bits, scale: float) -> np.ndarray:
    """The merged 16-bit weight W_new = Wb + (alpha/r) B A as bf16 bit patterns.

    "How Fine-Tuning LLMs with LoRA and QLoRA Works", FAQ on merging adapters
    back into the base weights (W + (alpha/r) B A); "QLoRA explained",
    "Merging and deploying" (a standalone 16-bit model).  READING: W is the
    layer's dequantized bf16 weight Wb; the sum is exact (float64 here) and
    rounded once to bf16.  Re-quantizing the merged weight is not done.
    """
    m = np.asarray(wb, dtype=np.float64) + float(scale) * (_bf(b_bits) @ _bf(a_bits))
    return _rne_bf16_bits_f64(m)


def _rne_bf16_bits_f64(v) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even, in one step.

    A float64 value is rounded directly to a multiple of its bf16 quantum
    (rounding it to float32 first could round twice): with v = m 2^e,
    0.5 <= |m| < 1, the quantum is 2^(e-8) for normal bf16 values and
    2^-133 below the normal range.  Finite inputs within the bf16 range.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = (np.round(v / quantum) * quantum).astype(np.float32)  # exact: a bf16 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def forward_multi(wb, x_bits, a_bank_bits, b_bank_bits, scales, ids):
    """Per-token adapter: h_t = x_t Wb^T + s_id (x_t A_id^T) B_id^T.

    ("From LoRA to QLoRA", "The Real-World Bottleneck": one resident base,
    adapter chosen per request.)  READING: a token whose id is outside
    [0, n_adapters) gets the base output only.
    """
    x = _bf(x_bits)
    a = _bf(a_bank_bits)  # [n, r, in]
    b = _bf(b_bank_bits)  # [n, out, r]
    ids = np.asarray(ids, dtype=np.int64)
    h = x @ np.asarray(wb, dtype=np.float64).T
    n = a.shape[0]
    for t in range(x.shape[0]):
        i = ids[t]
        if 0 <= i < n:
            h[t] += float(scales[i]) * (b[i] @ (a[i] @ x[t]))
    return h


# ---------------------------------------------------------------------------
# Storage accounting ("From LoRA to QLoRA", worked example memory footprint and
# Pillar 2 bits-per-parameter).
# ---------------------------------------------------------------------------
def adamw_step(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float):
    """One AdamW step on the adapter parameters, in float64.  Returns (p, m, v).

    The pages train only the adapters with AdamW and keep the adapters and
    their optimizer state (the Adam moments) in full precision, the moments
    possibly paged to host memory ("QLoRA Specification for EMEP
    Fine-Tuning", "GPU Orchestration"; "QLoRA explained", "Paged
    optimizers"; "QLoRA Finetuner", the AdamW example).  READING: the update
    rule is not printed; it is the published AdamW (decoupled weight decay,
    bias-corrected moments), step counted from 1:
        p <- p - lr*wd*p
        m <- beta1*m + (1-beta1)*g,   v <- beta2*v + (1-beta2)*g^2
        p <- p - lr * (m / (1-beta1^t)) / (sqrt(v / (1-beta2^t)) + eps)
    The 8-bit variant of the states is not taken (its encoding is not on the
    pages).
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    t = int(step)
    p = p - lr * weight_decay * p
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


def storage_bytes(numel: int, double_quant: bool, block_size: int = BLOCK_SIZE,
                  dq_group: int = DQ_GROUP):
    """(code bytes, first-level scale bytes stored, second-level bytes)."""
    nb = numel // block_size
    code_b = numel // 2
    if double_quant:
        return code_b, nb * 1, ((nb + dq_group - 1) // dq_group) * 4
    return code_b, nb * 4, 0


def tolerance_ok(got, ref, rel: float = 1e-2, floor: float = 1e-3):
    """|got - ref| <= rel*|ref| + floor*rms(ref), elementwise; returns (ok, worst ratio)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    bound = rel * np.abs(r) + floor * rms
    err = np.abs(g - r)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(err <= bound)), worst
