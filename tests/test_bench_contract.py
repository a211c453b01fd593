"""CPU checks of the benchmark's contract: the metric name is the one the
measurement is quoted on, the algorithmic work it divides by matches the
closed forms of the workloads (bytes of the fused decode product: 4-bit
codes, one int8 scale code per 64-block, one fp32 constant per group of 256
blocks, x, A, B and h in bf16; flops of the training pass: 2 M out in for
each of the two dequantized products plus the rank-r products), and a
request for several GPUs is refused before anything touches a GPU."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _groups(out, inp):
    return (out * inp // 64 + 255) // 256


def test_metric_is_the_quoted_one():
    with open(os.path.join(ROOT, "BASELINE.json")) as f:
        assert bench.METRIC == json.load(f)["metric"]


@pytest.mark.parametrize("out,inp,M,r,expect", [
    (28672, 8192, 1, 64, 125_960_192),  # the 70B projection at one token
    (4096, 4096, 1, 16, 8_933_376),     # the 4096 x 4096 decode at 1, 4 and 16 tokens
    (4096, 4096, 4, 16, 8_982_528),
    (4096, 4096, 16, 16, 9_179_136),
])
def test_decode_bytes(out, inp, M, r, expect):
    got = bench.decode_bytes(out, inp, M, r, _groups(out, inp))
    assert got == expect
    closed = (out * inp // 2 + out * inp // 64 + 4 * _groups(out, inp) + 2 * M * inp + 2 * r * (inp + out)
              + 2 * M * out)
    assert got == closed
    # a little over half a byte per weight
    assert 0.5 < got / (out * inp) < 0.56


def test_kernel_bytes_leave_out_what_other_kernels_read():
    out, inp, r = 28672, 8192, 64
    g = _groups(out, inp)
    # the fused product does not read A (the u kernel does) but reads u
    assert bench.gemv_kernel_bytes(out, inp, 1, r, g) == bench.decode_bytes(out, inp, 1, r, g) - 2 * r * inp + 4 * r
    # the few-token dX pass reads dH instead of x and writes no h
    assert bench.dx_gemv_kernel_bytes(out, inp, 1, r, g) == out * inp // 2 + out * inp // 64 + 4 * g + 2 * out + 2 * r * out


@pytest.mark.parametrize("out,inp,M,r,fwd,bwd", [
    (11008, 4096, 2048, 64, 188_643_016_704, 192_602_439_680),      # 7B MLP shape
    (28672, 8192, 4096, 64, 1_943_472_701_440, 1_962_800_054_272),  # 70B MLP shape
])
def test_train_flops(out, inp, M, r, fwd, bwd):
    f, b = bench.train_flops(out, inp, M, r)
    assert (f, b) == (fwd, bwd)
    # the dense products dominate: the rank-r terms are a few per cent here
    assert 2 * M * out * inp / f > 0.97 and 2 * M * out * inp / b > 0.95


def test_several_gpus_refused_without_a_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout.strip() == ""
