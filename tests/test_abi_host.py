"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function include/nf4qlora.h declares, and rejects bad arguments before any
launch.  Calls that would launch a kernel are not made here."""

import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4qlora.h")
LIB = os.path.join(ROOT, "bit_nf4_quantized_04_amd", "libnf4qlora.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libnf4qlora.so not built")


@pytest.fixture(scope="module")
def F():
    from bit_nf4_quantized_04_amd import nf4qlora

    return nf4qlora


CALIB_HEADER = os.path.join(ROOT, "include", "nf4calib.h")
CALIB_LIB = os.path.join(ROOT, "bit_nf4_quantized_04_amd", "libnf4calib.so")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_headers_are_the_two_libraries():
    """Every header under include/ belongs to one of the two libraries."""
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["nf4calib.h", "nf4qlora.h"]


def test_every_declared_function_is_exported(F):
    names = declared_functions()
    assert len(names) == 20, names
    lib = C.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(F.EXPORTS)


@pytest.mark.skipif(not os.path.exists(CALIB_LIB), reason="libnf4calib.so not built")
def test_calibration_library_exports_and_argument_errors():
    from bit_nf4_quantized_04_amd import calib

    names = declared_functions(CALIB_HEADER)
    assert set(names) == set(calib.EXPORTS)
    lib = C.CDLL(CALIB_LIB)
    for n in names:
        assert hasattr(lib, n), n
    L = calib._lib
    assert L.nf4calib_read(None, 64, FAKE, 0, None) == 1
    assert L.nf4calib_read(C.c_void_p(0x100004), 64, FAKE, 0, None) == 1  # misaligned
    assert L.nf4calib_read(FAKE, 65, FAKE, 0, None) == 1                  # not whole 16-byte pieces
    assert L.nf4calib_read(FAKE, 64, None, 0, None) == 1
    assert L.nf4calib_mfma(0, 4, 4, FAKE, None) == 1
    assert L.nf4calib_mfma(10, 4, 9, FAKE, None) == 1
    assert L.nf4calib_mfma(10, 4, 4, None, None) == 1
    assert L.nf4calib_mfma_tile(0, 4, 0, FAKE, None) == 1
    assert L.nf4calib_mfma_tile(10, 4, 2, FAKE, None) == 1
    assert L.nf4calib_mfma_tile(10, 4, 1, None, None) == 1


def test_profile_hook_arguments(F):
    lib = F._lib
    assert lib.nf4_profile_events(FAKE, None, 0) == F.NF4_EINVAL
    assert lib.nf4_profile_events(FAKE, FAKE, 2) == F.NF4_EINVAL
    assert lib.nf4_profile_events(None, None, 0) == F.NF4_OK


def test_version_table_and_strings(F):
    from oracle import nf4_oracle as O

    assert F.nf4_version() == 2
    np.testing.assert_array_equal(F.nf4_table(), O.NF4_LEVELS)
    for code in range(7):
        assert F.nf4_strerror(code) and "unknown" not in F.nf4_strerror(code)
    assert "unknown" in F.nf4_strerror(99)


def test_storage_sizes_match_the_pages(F):
    # Worked example ("From LoRA to QLoRA", Pillar 1): 6 weights, one block,
    # 3 code bytes + 4 scale bytes = 7 bytes.
    assert F.nf4_storage_sizes(2, 3, double_quant=False, block_size=6) == (3, 4, 0)
    # Pillar 2: 0.5 bits/param of fp32 scales -> about 0.127 with int8 scales in groups of 256.
    rows, cols = 4096, 4096
    cb, sb, gb = F.nf4_storage_sizes(rows, cols, double_quant=False)
    assert 8 * sb / (rows * cols) == 0.5
    cb2, sb2, gb2 = F.nf4_storage_sizes(rows, cols, double_quant=True)
    assert cb == cb2 == rows * cols // 2
    assert round(8 * (sb2 + gb2) / (rows * cols), 3) == 0.127


def _cfg(F, bs=64, dq=1, g=256):
    return F.nf4_config(bs, dq, g)


FAKE = C.c_void_p(0x100000)  # aligned, never dereferenced: every call below fails validation first


@pytest.mark.parametrize("entry", ["nf4_quantize", "nf4_quantize_bf16"])
def test_quantize_argument_errors(F, entry):
    """Both quantizer entry points (fp32 and bf16 input) validate alike."""
    lib = F._lib
    cfg = _cfg(F)
    fn = getattr(lib, entry)
    q = lambda W, r, c, cf, codes, ab, sc, ga: fn(W, r, c, cf, codes, ab, sc, ga, None)
    assert q(None, 64, 64, C.byref(cfg), FAKE, FAKE, FAKE, FAKE) == F.NF4_EINVAL
    assert q(FAKE, 64, 64, None, FAKE, FAKE, FAKE, FAKE) == F.NF4_EINVAL
    assert q(FAKE, -1, 64, C.byref(cfg), FAKE, FAKE, FAKE, FAKE) == F.NF4_EINVAL
    assert q(FAKE, 3, 5, C.byref(cfg), FAKE, FAKE, FAKE, FAKE) == F.NF4_ESHAPE
    bad = _cfg(F, bs=96)
    assert q(FAKE, 64, 64, C.byref(bad), FAKE, FAKE, FAKE, FAKE) == F.NF4_EUNSUPPORTED
    b128 = _cfg(F, bs=128)
    assert q(FAKE, 3, 64, C.byref(b128), FAKE, FAKE, FAKE, FAKE) == F.NF4_ESHAPE  # 192 elements: a partial block
    bad = _cfg(F, g=0)
    assert q(FAKE, 64, 64, C.byref(bad), FAKE, FAKE, FAKE, FAKE) == F.NF4_EUNSUPPORTED
    for qt in (2, -1):
        bad = F.nf4_config(64, 1, 256, qt)
        assert q(FAKE, 64, 64, C.byref(bad), FAKE, FAKE, FAKE, FAKE) == F.NF4_EUNSUPPORTED
    assert q(FAKE, 64, 64, C.byref(cfg), FAKE, FAKE, None, FAKE) == F.NF4_EINVAL  # DQ needs its outputs
    assert q(C.c_void_p(0x100004), 64, 64, C.byref(cfg), FAKE, FAKE, FAKE, FAKE) == F.NF4_EINVAL
    assert q(None, 0, 64, C.byref(cfg), None, None, None, None) == F.NF4_OK  # empty: no-op


def _tensor(F, rows=128, cols=256, dq=1, bs=64, g=256, codes=FAKE):
    return F.nf4_tensor(codes, FAKE, FAKE, FAKE, rows, cols, F.nf4_config(bs, dq, g))


def test_quant_type_of_a_tensor_is_validated(F):
    lib = F._lib
    for qt in (2, 7, -1):
        t = F.nf4_tensor(FAKE, FAKE, FAKE, FAKE, 128, 256, F.nf4_config(64, 1, 256, qt))
        assert lib.nf4_dequantize(C.byref(t), FAKE, None) == F.NF4_EUNSUPPORTED
        assert lib.qlora_linear_forward(C.byref(t), FAKE, 1, FAKE, FAKE, 16, 1.0, FAKE, None, FAKE, 1 << 30,
                                        None) == F.NF4_EUNSUPPORTED


def test_level_tables(F):
    """nf4_levels: the NF4 table (as nf4_table) and the FP4 levels, the
    published E2M1 values (OCP Microscaling v1.0: 0, 0.5, 1, 1.5, 2, 3, 4, 6
    and their negatives, code bit 3 the sign) divided by 6 in float32."""
    np.testing.assert_array_equal(F.nf4_levels("nf4"), F.nf4_table())
    fp4 = F.nf4_levels("fp4")
    mags = np.float32([0, 0.5, 1, 1.5, 2, 3, 4, 6]) / np.float32(6)
    want = np.concatenate([mags, -mags]).astype(np.float32)
    np.testing.assert_array_equal(fp4.view(np.uint32), want.view(np.uint32))
    assert F._lib.nf4_levels(2) is None or not bool(F._lib.nf4_levels(2))


def test_layer_argument_errors(F):
    lib = F._lib
    t = _tensor(F)
    fwd = lambda tt, x, M, A, B, r, s, h, ws, wsb: lib.qlora_linear_forward(
        C.byref(tt), x, M, A, B, r, s, h, None, ws, wsb, None)
    assert fwd(t, FAKE, -1, FAKE, FAKE, 4, 2.0, FAKE, FAKE, 1 << 30) == F.NF4_EINVAL
    assert fwd(t, FAKE, 4, FAKE, FAKE, 300, 2.0, FAKE, FAKE, 1 << 30) == F.NF4_EINVAL
    assert fwd(t, FAKE, 4, FAKE, FAKE, 4, float("nan"), FAKE, FAKE, 1 << 30) == F.NF4_EINVAL
    assert fwd(t, None, 4, FAKE, FAKE, 4, 2.0, FAKE, FAKE, 1 << 30) == F.NF4_EINVAL
    assert fwd(_tensor(F, cols=96), FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, FAKE, 1 << 30) == F.NF4_ESHAPE
    assert fwd(_tensor(F, bs=32), FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, FAKE, 1 << 30) == F.NF4_EUNSUPPORTED
    assert fwd(_tensor(F, codes=None), FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, FAKE, 1 << 30) == F.NF4_EINVAL
    need = F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 128, 256, 4, 4)
    assert need > 0
    assert fwd(t, FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, FAKE, need - 1) == F.NF4_EWORKSPACE
    assert fwd(t, FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, None, need) == F.NF4_EWORKSPACE
    assert fwd(t, FAKE, 0, FAKE, FAKE, 4, 2.0, FAKE, None, 0) == F.NF4_OK  # M == 0: no-op
    bwd = lambda tt, M, r, dA, wsb: lib.qlora_linear_backward(
        C.byref(tt), FAKE, FAKE, M, FAKE, FAKE, r, 2.0, None, FAKE, dA, FAKE, FAKE, wsb, None)
    assert bwd(t, 4, 0, FAKE, 1 << 30) == F.NF4_EINVAL  # backward needs r >= 1
    assert bwd(t, 4, 4, None, 1 << 30) == F.NF4_EINVAL
    nb = F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD, 128, 256, 4, 4)
    assert bwd(t, 4, 4, FAKE, nb - 1) == F.NF4_EWORKSPACE
    multi = lambda n, r, ids: lib.qlora_linear_forward_multi(
        C.byref(t), FAKE, 4, FAKE, FAKE, n, r, FAKE, ids, FAKE, FAKE, 1 << 30, None)
    assert multi(0, 4, FAKE) == F.NF4_EINVAL
    assert multi(3, 4, None) == F.NF4_EINVAL
    mb = F.qlora_workspace_bytes(F.QLORA_OP_FORWARD_MULTI, 128, 256, 4, 4, 3)
    assert lib.qlora_linear_forward_multi(C.byref(t), FAKE, 4, FAKE, FAKE, 3, 4, FAKE, FAKE, FAKE,
                                          FAKE, mb - 1, None) == F.NF4_EWORKSPACE


def test_dequantize_argument_errors(F):
    lib = F._lib
    assert lib.nf4_dequantize(None, FAKE, None) == F.NF4_EINVAL
    t = _tensor(F, rows=3, cols=5)
    assert lib.nf4_dequantize(C.byref(t), FAKE, None) == F.NF4_ESHAPE
    t = _tensor(F, rows=2, cols=96)  # 192 elements: a multiple of 64 is enough for dequantize
    assert lib.nf4_dequantize(C.byref(t), None, None) == F.NF4_EINVAL
    t = F.nf4_tensor(FAKE, None, None, None, 2, 64, F.nf4_config(64, 0, 256))
    assert lib.nf4_dequantize_bf16(C.byref(t), FAKE, None) == F.NF4_EINVAL  # no-DQ needs absmax


def test_block128_layer_calls(F):
    """A 128-element-block weight: the layer calls keep one fp32 scale per
    64-element half-block at the front of the workspace, so the workspace
    query with the flag is larger by exactly that (rounded to 256 bytes), and
    a call given only the 64-block size is refused."""
    lib = F._lib
    for op in (F.QLORA_OP_FORWARD, F.QLORA_OP_BACKWARD):
        base = F.qlora_workspace_bytes(op, 128, 256, 600, 8)
        flagged = F.qlora_workspace_bytes(op | F.QLORA_OP_BLOCK128, 128, 256, 600, 8)
        assert flagged == base + (128 * 256 // 16 + 255) // 256 * 256
    base = F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 128, 256, 1, 0)
    assert F.qlora_workspace_bytes(F.QLORA_OP_FORWARD | F.QLORA_OP_BLOCK128, 128, 256, 1, 0) == base + 2048
    t = _tensor(F, bs=128)
    fwd = lambda ws, wsb: lib.qlora_linear_forward(C.byref(t), FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, None, ws, wsb, None)
    assert fwd(FAKE, 1024) == F.NF4_EWORKSPACE  # the expansion alone needs 2048 bytes
    assert fwd(None, 1 << 20) == F.NF4_EWORKSPACE
    # a linear call on 128-blocks that straddle rows is fine (cols % 64 == 0),
    # a tensor that is not a whole number of blocks is not
    t2 = _tensor(F, rows=3, cols=64, bs=128)
    assert lib.qlora_linear_forward(C.byref(t2), FAKE, 4, FAKE, FAKE, 4, 2.0, FAKE, None, FAKE, 1 << 20, None) == F.NF4_ESHAPE


def test_dropout_argument_errors(F):
    """A dropout rate outside [0, 1) or no settings at all is refused before
    anything is launched; the dropout workspace holds xd (M*in bf16) and, in
    the backward, the fp32 dH Wb (M*in fp32) and the keep bits (M*in/8 bytes)."""
    lib = F._lib
    t = _tensor(F)
    fwd = lambda d: lib.qlora_linear_forward_dropout(C.byref(t), FAKE, 4, FAKE, FAKE, 4, 2.0, d, FAKE, None,
                                                     FAKE, 1 << 30, None)
    bwd = lambda d: lib.qlora_linear_backward_dropout(C.byref(t), FAKE, FAKE, 4, FAKE, FAKE, 4, 2.0, d, None,
                                                      FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    for p in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        d = F.qlora_dropout(p, 0, 1)
        assert fwd(C.byref(d)) == F.NF4_EINVAL
        assert bwd(C.byref(d)) == F.NF4_EINVAL
    assert fwd(None) == F.NF4_EINVAL and bwd(None) == F.NF4_EINVAL
    for op, extra in ((F.QLORA_OP_FORWARD, 600 * 256 * 2), (F.QLORA_OP_BACKWARD, 600 * 256 * (6 + 1 / 8))):
        base = F.qlora_workspace_bytes(op, 128, 256, 600, 8)
        assert F.qlora_workspace_bytes(op | F.QLORA_OP_DROPOUT, 128, 256, 600, 8) == base + extra
        both = F.qlora_workspace_bytes(op | F.QLORA_OP_DROPOUT | F.QLORA_OP_BLOCK128, 128, 256, 600, 8)
        assert both == base + extra + 128 * 256 // 16


def test_noalloc_forward_refuses_oversized_calls(F):
    """The allocation-free forward checks its need against its fixed scratch
    before anything is launched: a shape whose workspace query exceeds
    QLORA_NOALLOC_SCRATCH_BYTES is refused with NF4_ETOOLARGE, bad arguments
    as the plain forward, and M = 0 is a no-op."""
    lib = F._lib
    big = _tensor(F, rows=4096, cols=4096)
    need = F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 4096, 4096, 2048, 16)
    assert need > F.QLORA_NOALLOC_SCRATCH_BYTES
    call = lambda tt, M, r, s=2.0, x=FAKE: lib.qlora_linear_forward_noalloc(C.byref(tt), x, M, FAKE, FAKE, r, s,
                                                                           FAKE, None, None)
    assert call(big, 2048, 16) == F.NF4_ETOOLARGE
    assert "scratch" in F.nf4_strerror(F.NF4_ETOOLARGE)
    assert call(big, -1, 16) == F.NF4_EINVAL
    assert call(big, 4, 300) == F.NF4_EINVAL
    assert call(big, 4, 16, float("nan")) == F.NF4_EINVAL
    assert call(_tensor(F, cols=96), 4, 16) == F.NF4_ESHAPE
    assert call(big, 0, 16) == F.NF4_OK
    for (o, i, M, r) in ((28672, 8192, 1, 64), (28672, 8192, 16, 64), (28672, 8192, 4096, 64), (11008, 4096, 2048, 64)):
        assert F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, o, i, M, r) <= F.QLORA_NOALLOC_SCRATCH_BYTES


def test_workspace_sizes_are_monotone(F):
    a = F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 4096, 4096, 16, 16)
    b = F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 4096, 4096, 2048, 16)
    assert 0 < a < b
    assert F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 4096, 4096, 16, 0) == 0
    assert F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD, 4096, 4096, 16, 16) > a
    assert F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, 4096, 4096, 16, 999) == 0


def test_adamw_and_merge_argument_errors(F):
    lib = F._lib
    ad = lambda p, n, step, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8: lib.qlora_adamw_step(
        p, FAKE, FAKE, FAKE, None, n, step, lr, b1, b2, eps, 0.0, None)
    assert ad(FAKE, -1, 1) == F.NF4_EINVAL
    assert ad(FAKE, 10, 0) == F.NF4_EINVAL  # steps count from 1
    assert ad(FAKE, 10, 1, b1=1.0) == F.NF4_EINVAL
    assert ad(FAKE, 10, 1, eps=0.0) == F.NF4_EINVAL
    assert ad(FAKE, 10, 1, lr=float("inf")) == F.NF4_EINVAL
    assert ad(None, 10, 1) == F.NF4_EINVAL
    assert ad(None, 0, 1) == F.NF4_OK  # n == 0: no-op, nothing touched
    t = _tensor(F)
    mg = lambda tt, r, out: lib.qlora_merge(C.byref(tt), FAKE, FAKE, r, 2.0, out, None)
    assert mg(t, 0, FAKE) == F.NF4_EINVAL
    assert mg(t, 257, FAKE) == F.NF4_EINVAL
    assert mg(t, 4, None) == F.NF4_EINVAL
    assert mg(_tensor(F, codes=None), 4, FAKE) == F.NF4_EINVAL



def test_workspace_queries_without_tokens(F):
    """M = 0 is a valid call (a no-op forward, zero dA and dB): every
    workspace query answers it, for the split plans of both adapter-product
    schemes (r <= 64 with rows % 16 == 0, and r > 64) and long reductions."""
    for rows, cols, r in ((128, 256, 8), (28672, 8192, 64), (300, 512, 256), (4096, 4096, 100)):
        for op in (F.QLORA_OP_FORWARD, F.QLORA_OP_BACKWARD, F.QLORA_OP_FORWARD_MULTI,
                   F.QLORA_OP_BACKWARD | F.QLORA_OP_DROPOUT, F.QLORA_OP_FORWARD | F.QLORA_OP_BLOCK128):
            assert F.qlora_workspace_bytes(op, rows, cols, 0, r, 4) >= 0


def test_level_table_from_many_threads(F):
    """nf4_table() is safe to call from several threads at once (its table is
    initialised once) and every caller sees the 16 levels."""
    import threading

    from oracle import nf4_oracle as O

    lib = C.CDLL(LIB)
    lib.nf4_table.restype = C.POINTER(C.c_float)
    seen, errs = [], []

    def run():
        try:
            for _ in range(200):
                p = lib.nf4_table()
                seen.append(np.ctypeslib.as_array(p, shape=(16,)).copy())
        except Exception as e:  # pragma: no cover
            errs.append(e)

    th = [threading.Thread(target=run) for _ in range(8)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs and len(seen) == 1600
    for v in seen:
        np.testing.assert_array_equal(v, O.NF4_LEVELS)


@pytest.mark.parametrize("src,defines", [
    ("gemm_rd.hip", ["-DNF4_FWD_WAVES=4", "-DNF4_DX_WAVES=4"]),  # the four-wave GEMM forms
    ("skinny.hip", ["-DNF4_GEMV_NV=2"]),  # decode lookups partly from register byte planes
])
def test_build_options_compile(tmp_path, src, defines):
    """The kernels' build options other than the defaults still compile for
    gfx950 (device code only, at -O1 to keep this check short: the templates
    are instantiated and their static checks run; the default forms are what
    build() links)."""
    from bit_nf4_quantized_04_amd import build as B

    if not os.path.exists(B.HIPCC):
        pytest.skip("no hipcc")
    import subprocess

    flags = ["-O1" if f == "-O3" else f for f in B.FLAGS]
    cmd = [B.HIPCC, *flags, "--cuda-device-only", *defines, "-c", os.path.join(B.CSRC, src),
           "-o", str(tmp_path / "k.o")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    assert not [l for l in res.stderr.splitlines() if "error" in l]
