"""Benchmark of the NF4 QLoRA linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only PASS]

Workload of the JSON line: the 70B MLP projection 8192 -> 28672 (W0 [28672,
8192], 99.9% N(0, 0.015^2) entries and 0.1% 0.1 * Student-t(3) outliers), NF4
blocks of 64 with int8 double quantization in groups of 256, r = 64, alpha =
128, synthetic seeded inputs.  One step is one pass of the layer's hot path:
  * decode: the fused dequant-GEMV forward at M = 1 (u = x A^T, then
    h = x Wb^T + s u B^T), rotating over 5 resident copies of the quantized
    weight (630 MB > the 256 MB last-level cache) so every call streams W from HBM;
  * training: forward (u and h) and backward (dX, dA, dB) at M = 4096.
`value` is the decode throughput in algorithmic GB/s (the headline metric's
first figure); the training pass is reported as bf16 TFLOP/s in the same line,
beside the other workloads (the 4096 x 4096 decode at M = 1, 4, 16, the 7B
training pass, the multi-adapter forward) and the measured ceilings of this
GPU (a plain read of the same bytes, an MFMA loop).  Inputs are resident in
HBM before the timed region starts.  Each latency-bound section (the decode
steps) first runs its step untimed for 100 ms, then its W warmup steps, then
the K timed steps.  Rank 0 prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NF4 QLoRA linear: GB/s at M=1, bf16 TFLOP/s at M=4096, % of roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
SETTLE_MS = 100.0
KERNEL_MS_WHAT = ("mean over the timed steps of HIP events on the library's stream, from the end of the kernel "
                  "launched just before it in the same call to its own end (so it includes the dispatch gap "
                  "before it and cannot exceed the step)")
ONLY = ("decode", "decode_bwd", "train", "train_fwd", "train_bwd", "train7", "train7_fwd", "train7_bwd",
        "multi", "decode_c2", "read", "mfma", "structure", "vendor", "copy")


def decode_bytes(out, inp, M, r, ngroups, with_A=True, block=64):
    """Algorithmic HBM bytes of one decode forward (double quant, blocks of
    `block` elements: one int8 scale code per block)."""
    b = out * inp // 2 + out * inp // block + 4 * ngroups + 2 * M * inp + 2 * M * out
    b += 2 * r * out + (2 * r * inp if with_A else 0)
    return b


def gemv_kernel_bytes(out, inp, M, r, ngroups):
    """Algorithmic bytes of the fused dequant product kernel alone: codes,
    scale codes, group constants, x, B, u and h (A is read by the u kernel)."""
    return (out * inp // 2 + out * inp // 64 + 4 * ngroups + 2 * M * inp + 2 * r * out
            + 4 * M * r + 2 * M * out)


def dx_gemv_kernel_bytes(out, inp, M, r, ngroups):
    """Algorithmic bytes of the few-token dX kernel (one pass over the weight
    rows for dX and dU): codes, scale codes, group constants, dH and B."""
    return out * inp // 2 + out * inp // 64 + 4 * ngroups + 2 * M * out + 2 * r * out


def train_flops(out, inp, M, r):
    fwd = 2 * M * out * inp + 2 * M * r * (inp + out)
    bwd = 2 * M * out * inp + 4 * M * out * r + 4 * M * r * inp
    return fwd, bwd


def measured_traffic(kernel):
    """HBM bytes per launch (read + write) of `kernel` from the committed
    counter summary, or None when the library's sources have changed since the
    counters were taken (the summary records a hash of them)."""
    import hashlib

    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_nf4_quantized_04_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("source_sha256_16") != h.hexdigest()[:16] or not k:
        return None
    return int(round(k["read_bytes"] + k["write_bytes"]))


# ----------------------------------------------------------------- CPU oracle
def progress(msg):
    """One line on stderr when a section of the run has finished."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def _cores():
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return aff, int(blas)


def _run_for(budget_s, fn):
    """Call fn(i) until about budget_s seconds of it have run; returns (calls,
    seconds, sum of what fn returned)."""
    n, spent, acc = 0, 0.0, 0
    while spent < budget_s or n == 0:
        t0 = time.perf_counter()
        acc += fn(n)
        spent += time.perf_counter() - t0
        n += 1
    return n, spent, acc


def cpu_decode(O, wl, c, M, budget_s, rows_per=None):
    """The oracle doing the decode forward of workload c at M tokens on row
    samples of the workload weight (quantized once, untimed); GB/s of the same
    algorithmic bytes as the GPU line."""
    sh = wl.SHAPES[c]
    out, inp, r = sh["out"], sh["inp"], sh["r"]
    w = wl.weight(c)
    x = wl.activations(c, M)
    a, b = wl.adapters(c)
    scale = sh["alpha"] / r
    if rows_per is None:
        rows_per = out
    rng = np.random.default_rng(0)
    starts = sorted(set(int(s) * rows_per for s in rng.choice(out // rows_per, size=min(4, out // rows_per),
                                                              replace=False)))
    prepared = [(g0, O.quantize(np.ascontiguousarray(w[g0:g0 + rows_per]), double_quant=True)) for g0 in starts]
    ng = (rows_per * inp // 64 + 255) // 256
    nbytes = decode_bytes(rows_per, inp, M, r, ng)

    def one(i):
        g0, qt = prepared[i % len(prepared)]
        wb = O.compute_weight(qt, (rows_per, inp))
        O.forward(wb, x, a, b[g0:g0 + rows_per], scale)
        return nbytes

    n, spent, done = _run_for(budget_s, one)
    return done / spent / 1e9, n, spent, rows_per


def cpu_train(O, wl, c, rows_per, budget_s):
    """The oracle's dequantize + forward + backward (float64 BLAS) of workload
    c on row samples of the weight (all tokens, all input features);
    algorithmic GFLOP/s of the same formula as the GPU line."""
    sh = wl.SHAPES[c]
    out, inp, r = sh["out"], sh["inp"], sh["r"]
    M = max(sh["M"])
    w = wl.weight(c)
    x = wl.activations(c, M)
    dh = wl.upstream_grad(c, M)
    a, b = wl.adapters(c)
    scale = sh["alpha"] / r
    rng = np.random.default_rng(0)
    starts = [int(s) * rows_per for s in rng.choice(out // rows_per, size=2, replace=False)]
    prepared = [(g0, O.quantize(np.ascontiguousarray(w[g0:g0 + rows_per]), double_quant=True)) for g0 in starts]
    fl = sum(train_flops(rows_per, inp, M, r))

    def one(i):
        g0, qt = prepared[i % len(prepared)]
        wb = O.compute_weight(qt, (rows_per, inp))
        O.forward(wb, x, a, b[g0:g0 + rows_per], scale)
        O.backward(wb, x, np.ascontiguousarray(dh[:, g0:g0 + rows_per]), a, b[g0:g0 + rows_per], scale)
        return fl

    n, spent, done = _run_for(budget_s, one)
    return done / spent / 1e9, n, spent, M


def cpu_multi(O, wl, rows_per, budget_s):
    c = 5
    sh = wl.SHAPES[c]
    out, inp, r, n_ad = sh["out"], sh["inp"], sh["r"], sh["n_adapters"]
    M = max(sh["M"])
    w = wl.weight(c)
    x = wl.activations(c, M)
    ab, bb = wl.adapter_bank(c)
    ids = wl.adapter_ids(c, M, n_ad)
    scales = np.full(n_ad, sh["alpha"] / r)
    qt = O.quantize(np.ascontiguousarray(w[:rows_per]), double_quant=True)
    fl = 2 * M * rows_per * inp + 2 * M * r * (inp + rows_per)

    def one(i):
        wb = O.compute_weight(qt, (rows_per, inp))
        O.forward_multi(wb, x, ab, np.ascontiguousarray(bb[:, :rows_per]), scales, ids)
        return fl

    n, spent, done = _run_for(budget_s, one)
    return done / spent / 1e9, n, spent, M


def cpu_baselines(budget_s=8.0):
    """The oracle as it stands, timed on this host's cores, on bounded samples
    of each workload.  Returns (the headline object, the others)."""
    from bit_nf4_quantized_04_amd import workloads as wl
    from oracle import nf4_oracle as O

    aff, blas = _cores()
    note = "oracle as committed: dequantize in float32 NumPy elementwise (1 thread), products in float64 BLAS (%d threads)" % blas
    gbs, n, spent, rows = cpu_decode(O, wl, 4, 1, budget_s, rows_per=16384 * 64 // 8192)
    head = {
        "value": round(gbs, 3), "unit": "GB/s", "cores": aff, "blas_threads": blas, "kind": "oracle",
        "sample": "70B decode M=1: %d calls on %d-row slices (64 double-quant groups) of the workload weight, "
                  "%.1f s of CPU work; %s" % (n, rows, spent, note),
    }
    others = {}
    for M in (1, 4, 16):
        gbs, n, spent, rows = cpu_decode(O, wl, 2, M, budget_s / 4)
        others["decode_4096_M%d" % M] = {"value": round(gbs, 3), "unit": "GB/s",
                                         "sample": "%d calls on the whole 4096 x 4096 weight, %.1f s" % (n, spent)}
    g, n, spent, M = cpu_train(O, wl, 4, 64, budget_s)
    others["train_70b_M4096"] = {"value": round(g / 1e3, 4), "unit": "TFLOP/s",
                                 "sample": "%d forward+backward calls, M=%d, on 64-row slices of the 28672 x 8192 "
                                           "weight, %.1f s" % (n, M, spent)}
    g, n, spent, M = cpu_train(O, wl, 3, 256, budget_s / 2)
    others["train_7b_M2048"] = {"value": round(g / 1e3, 4), "unit": "TFLOP/s",
                                "sample": "%d forward+backward calls, M=%d, on 256-row slices of the 11008 x 4096 "
                                          "weight, %.1f s" % (n, M, spent)}
    g, n, spent, M = cpu_multi(O, wl, 512, budget_s / 2)
    others["multi_adapter_M2048"] = {"value": round(g / 1e3, 4), "unit": "TFLOP/s",
                                     "sample": "%d multi-adapter forward calls (per-token loop), M=%d, on a 512-row "
                                               "slice of the 4096 x 4096 weight, %.1f s" % (n, M, spent)}
    for v in others.values():
        v.update({"cores": aff, "blas_threads": blas, "kind": "oracle"})
    return head, others


# ------------------------------------------------------------------ GPU side
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=5)
    ap.add_argument("--only", choices=ONLY, default=None,
                    help="run one pass only, for profilers (prints its time, no JSON line); 'copy' is a "
                         "plain 512 MiB device copy (the calibration of HBM byte counters), 'read' and "
                         "'mfma' the ceiling kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: sharding the layer over several GPUs is "
              "not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_nf4_quantized_04_amd import calib as CAL
    from bit_nf4_quantized_04_amd import nf4qlora as F
    from bit_nf4_quantized_04_amd import workloads as wl

    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    hev = F.HipEvents()

    def timed(step, K, W, hook=None):
        """Mean ms per step over K steps (HIP events on the current stream);
        with hook = 0 or 1 also the dominant kernel's duration of every call
        (the library's event hook in that mode)."""
        for i in range(W):
            step(i)
        torch.cuda.synchronize()
        pairs = [(hev.create(), hev.create()) for _ in range(K)] if hook is not None else []
        t0, t1 = hev.create(), hev.create()
        hev.record(t0)
        for i in range(K):
            if hook is not None:
                F.nf4_profile_events(*pairs[i], mode=hook)
            step(i)
        hev.record(t1)
        torch.cuda.synchronize()
        F.nf4_profile_events(None, None)
        total = hev.elapsed_ms(t0, t1) / K
        kern = [hev.elapsed_ms(a, b) for a, b in pairs]
        for e in [t0, t1] + [e for p in pairs for e in p]:
            hev.destroy(e)
        return total, kern

    def settle(step, ms=SETTLE_MS):
        """Untimed run of `step` for `ms` milliseconds before a latency-bound
        section, so that its W warmup steps start at settled clocks."""
        t0 = time.perf_counter()
        i = 0
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(16):
                step(i)
                i += 1
            torch.cuda.synchronize()

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def ws(op, out, inp, M, r, n_ad=0):
        return torch.empty(max(F.qlora_workspace_bytes(op, out, inp, M, r, n_ad), 256), dtype=torch.uint8,
                           device=dev)

    def copies_of(q0, n):
        qs = [q0]
        for _ in range(n - 1):
            qs.append(F.NF4Weight(q0.codes.clone(), q0.absmax.clone(), q0.scale_codes.clone(),
                                  q0.group_absmax.clone(), q0.rows, q0.cols, True))
        return qs

    def run_only(step):
        settle(step)
        t, _ = timed(step, K, W)
        print("%s pass: %.4f ms/step over %d steps" % (args.only, t, K), flush=True)

    # ------------------------------------------------ ceilings of this GPU
    sink_u = torch.zeros(max(CAL.default_workgroups(0), 1), dtype=torch.int32, device=dev)

    def read_rate(nbytes, n_bufs, steps):
        bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(i) for i in range(n_bufs)]
        t, _ = timed(lambda i: CAL.read(bufs[i % n_bufs], sink_u), steps, 3)
        del bufs
        return nbytes / (t * 1e-3) / 1e9, t

    def mfma_rate():
        best = None
        for wgs_per_cu, waves in ((1, 8), (2, 4), (2, 8)):
            wgs = CAL.default_workgroups(1) // 4 * wgs_per_cu
            sink_f = torch.zeros(wgs, dtype=torch.float32, device=dev)
            iters = 4000
            fl = CAL.mfma(iters, sink_f, wgs, waves)
            t, _ = timed(lambda i: CAL.mfma(iters, sink_f, wgs, waves), 5, 2)
            rate = fl / (t * 1e-3) / 1e12
            if best is None or rate > best[0]:
                best = (rate, wgs, waves, t)
        return best

    def tile_rate(dequant):
        # the fused GEMM's inner loop without memory traffic (one workgroup of
        # eight waves per CU, one LDS fragment per MFMA, with or without the
        # dequantizing lookups): the ceiling of that structure on this GPU
        wgs = CAL.default_workgroups(1) // 4
        sink_t = torch.zeros(wgs * 8, dtype=torch.float32, device=dev)
        iters = 4000
        fl = CAL.mfma_tile(iters, sink_t, wgs, dequant)
        t, _ = timed(lambda i: CAL.mfma_tile(iters, sink_t, wgs, dequant), 5, 2)
        return fl / (t * 1e-3) / 1e12

    def vendor_gemm(M, n_out, n_in):
        # context only: the vendor library's plain bf16 product (torch.mm on
        # hipBLASLt) at the same shapes, on a bf16 weight that needs no
        # dequantization, forward (x W^T) and dX (dH W)
        g = torch.Generator(device=dev).manual_seed(7)
        xv = torch.randn(M, n_in, device=dev, dtype=torch.bfloat16, generator=g)
        wv = (torch.randn(n_out, n_in, device=dev, dtype=torch.bfloat16, generator=g) * 0.02)
        dv = torch.randn(M, n_out, device=dev, dtype=torch.bfloat16, generator=g)
        fl = 2.0 * M * n_out * n_in
        tf_, _ = timed(lambda i: torch.nn.functional.linear(xv, wv), 10, 3)
        td_, _ = timed(lambda i: torch.mm(dv, wv), 10, 3)
        del xv, wv, dv
        return {"forward_ms": round(tf_, 4), "forward_TFLOPs": round(fl / (tf_ * 1e-3) / 1e12, 1),
                "dx_ms": round(td_, 4), "dx_TFLOPs": round(fl / (td_ * 1e-3) / 1e12, 1)}

    if args.only == "structure":
        print("gemm structure: %.1f TFLOP/s bare, %.1f TFLOP/s with the dequantizing lookups"
              % (tile_rate(False), tile_rate(True)), flush=True)
        return
    if args.only == "vendor":
        print("vendor bf16 GEMM, M=4096 28672x8192: %s" % json.dumps(vendor_gemm(4096, 28672, 8192)), flush=True)
        return
    if args.only == "copy":
        src = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        t, _ = timed(lambda i: dst.copy_(src), K, W)
        print("copy pass: %d bytes read + %d written per launch, %.4f ms/launch (%.1f GB/s)"
              % (512 << 20, 512 << 20, t, 2 * (512 << 20) / (t * 1e-3) / 1e9), flush=True)
        return
    if args.only == "read":
        g, t = read_rate(124_911_872 // 16 * 16, 5, K)
        print("read pass: %.4f ms/launch, %.1f GB/s" % (t, g), flush=True)
        return
    if args.only == "mfma":
        rate, wgs, waves, t = mfma_rate()
        print("mfma pass: %.1f TFLOP/s (%d workgroups x %d waves, %.4f ms)" % (rate, wgs, waves, t), flush=True)
        return

    # ------------------------------------------------ 70B projection (workload 4)
    c = 4
    sh = wl.SHAPES[c]
    out, inp, r = sh["out"], sh["inp"], sh["r"]
    scale = sh["alpha"] / r
    Mtrain = max(sh["M"])
    ngroups = (out * inp // 64 + 255) // 256
    w = wl.weight(c)
    wt = torch.from_numpy(w).to(dev)
    qs = copies_of(F.nf4_quantize(wt, double_quant=True), args.copies)
    del wt, w
    a_bits, b_bits = wl.adapters(c)
    A, B = bf(a_bits), bf(b_bits)
    x1 = bf(wl.activations(c, 1))
    dH1 = bf(wl.upstream_grad(c, 1))
    ws_f1 = ws(F.QLORA_OP_FORWARD, out, inp, 1, r)
    ws_b1 = ws(F.QLORA_OP_BACKWARD, out, inp, 1, r)
    h1 = torch.empty((1, out), dtype=torch.bfloat16, device=dev)
    _, u1 = F.qlora_linear_forward(qs[0], x1, A, B, scale, want_u=True, ws=ws_f1, out=h1)

    def decode_step(i):
        F.qlora_linear_forward(qs[i % len(qs)], x1, A, B, scale, ws=ws_f1, out=h1)

    def decode_bwd_step(i):
        F.qlora_linear_backward(qs[i % len(qs)], x1, dH1, A, B, scale, u=u1, ws=ws_b1)

    if args.only in ("decode", "decode_bwd"):
        run_only(decode_step if args.only == "decode" else decode_bwd_step)
        return

    xt = bf(wl.activations(c, Mtrain))
    dH = bf(wl.upstream_grad(c, Mtrain))
    ws_ft = ws(F.QLORA_OP_FORWARD, out, inp, Mtrain, r)
    ws_bt = ws(F.QLORA_OP_BACKWARD, out, inp, Mtrain, r)
    ht = torch.empty((Mtrain, out), dtype=torch.bfloat16, device=dev)
    _, ut = F.qlora_linear_forward(qs[0], xt, A, B, scale, want_u=True, ws=ws_ft, out=ht)

    def train_step(i):
        _, u = F.qlora_linear_forward(qs[0], xt, A, B, scale, want_u=True, ws=ws_ft, out=ht)
        F.qlora_linear_backward(qs[0], xt, dH, A, B, scale, u=u, ws=ws_bt)

    def train_fwd(i):
        F.qlora_linear_forward(qs[0], xt, A, B, scale, ws=ws_ft, out=ht)

    def train_bwd(i):
        F.qlora_linear_backward(qs[0], xt, dH, A, B, scale, u=ut, ws=ws_bt)

    if args.only in ("train", "train_fwd", "train_bwd"):
        run_only({"train": train_step, "train_fwd": train_fwd, "train_bwd": train_bwd}[args.only])
        return

    # ------------------------------------------------ 7B MLP training (workload 3)
    c7 = 3
    sh7 = wl.SHAPES[c7]
    M7, r7, s7 = max(sh7["M"]), sh7["r"], sh7["alpha"] / sh7["r"]
    q7 = F.nf4_quantize(torch.from_numpy(wl.weight(c7)).to(dev), double_quant=True)
    a7, b7 = wl.adapters(c7)
    A7, B7 = bf(a7), bf(b7)
    x7, dH7 = bf(wl.activations(c7, M7)), bf(wl.upstream_grad(c7, M7))
    wsf7 = ws(F.QLORA_OP_FORWARD, sh7["out"], sh7["inp"], M7, r7)
    wsb7 = ws(F.QLORA_OP_BACKWARD, sh7["out"], sh7["inp"], M7, r7)
    h7 = torch.empty((M7, sh7["out"]), dtype=torch.bfloat16, device=dev)
    _, u7 = F.qlora_linear_forward(q7, x7, A7, B7, s7, want_u=True, ws=wsf7, out=h7)

    def train7_step(i):
        _, u = F.qlora_linear_forward(q7, x7, A7, B7, s7, want_u=True, ws=wsf7, out=h7)
        F.qlora_linear_backward(q7, x7, dH7, A7, B7, s7, u=u, ws=wsb7)

    def train7_fwd(i):
        F.qlora_linear_forward(q7, x7, A7, B7, s7, ws=wsf7, out=h7)

    def train7_bwd(i):
        F.qlora_linear_backward(q7, x7, dH7, A7, B7, s7, u=u7, ws=wsb7)

    if args.only in ("train7", "train7_fwd", "train7_bwd"):
        run_only({"train7": train7_step, "train7_fwd": train7_fwd, "train7_bwd": train7_bwd}[args.only])
        return

    # ------------------------------------------------ multi-adapter (workload 5)
    cm = 5
    shm = wl.SHAPES[cm]
    Mm = max(shm["M"])
    qm = F.nf4_quantize(torch.from_numpy(wl.weight(cm)).to(dev), double_quant=True)
    abm, bbm = wl.adapter_bank(cm)
    xm, Abm, Bbm = bf(wl.activations(cm, Mm)), bf(abm), bf(bbm)
    idsm = torch.from_numpy(wl.adapter_ids(cm, Mm, shm["n_adapters"])).to(dev)
    scm = torch.full((shm["n_adapters"],), shm["alpha"] / shm["r"], dtype=torch.float32, device=dev)
    hm = torch.empty((Mm, shm["out"]), dtype=torch.bfloat16, device=dev)
    wsm = ws(F.QLORA_OP_FORWARD_MULTI, shm["out"], shm["inp"], Mm, shm["r"], shm["n_adapters"])

    def multi_step(i):
        F.qlora_linear_forward_multi(qm, xm, Abm, Bbm, scm, idsm, ws=wsm, out=hm)

    if args.only == "multi":
        run_only(multi_step)
        return

    # ------------------------------------------------ 4096 x 4096 decode (workload 2)
    c2 = 2
    sh2 = wl.SHAPES[c2]
    q2 = copies_of(F.nf4_quantize(torch.from_numpy(wl.weight(c2)).to(dev), double_quant=True), 64)
    a2, b2 = wl.adapters(c2)
    A2, B2 = bf(a2), bf(b2)
    s2 = sh2["alpha"] / sh2["r"]
    dec2 = {}
    for M2 in sh2["M"]:
        x2 = bf(wl.activations(c2, M2))
        ws2 = ws(F.QLORA_OP_FORWARD, sh2["out"], sh2["inp"], M2, sh2["r"])
        h2 = torch.empty((M2, sh2["out"]), dtype=torch.bfloat16, device=dev)
        dec2[M2] = (lambda i, x2=x2, ws2=ws2, h2=h2:
                    F.qlora_linear_forward(q2[i % len(q2)], x2, A2, B2, s2, ws=ws2, out=h2))
    if args.only == "decode_c2":
        for M2, step in dec2.items():
            t, _ = timed(step, K, W)
            print("decode_c2 M=%d pass: %.4f ms/step over %d steps" % (M2, t, K), flush=True)
        return

    # ------------------------------------------------ timings
    settle(decode_step)
    t_dec, _ = timed(decode_step, K, W)
    _, k_dec = timed(decode_step, K, 1, hook=1)
    settle(decode_bwd_step)
    t_dbw, _ = timed(decode_bwd_step, K, W)
    _, k_dbw = timed(decode_bwd_step, K, 1, hook=1)
    progress("decode (70B, M=1) timed")
    t_tr, _ = timed(train_step, max(K // 2, 3), max(W // 2, 1))
    _, fwd_k = timed(train_fwd, max(K // 2, 3), 1, hook=0)
    _, bwd_k = timed(train_bwd, max(K // 2, 3), 1, hook=0)
    progress("training pass (70B, M=4096) timed")
    t_7b, _ = timed(train7_step, K, W)
    _, fwd7_k = timed(train7_fwd, K, 1, hook=0)
    _, bwd7_k = timed(train7_bwd, K, 1, hook=0)
    progress("training pass (7B, M=2048) timed")
    t_mu, _ = timed(multi_step, K, W)
    _, mu_k = timed(multi_step, K, 1, hook=0)
    progress("multi-adapter forward timed")
    t_c2 = {}
    for M2, step in dec2.items():
        settle(step)
        t_c2[M2] = timed(step, K, W)[0]
    # the same calls without the host's per-call cost: one call per weight
    # copy captured in a HIP graph, the graph replayed
    t_c2g = {}
    for M2, step in dec2.items():
        step(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(len(q2)):
                step(i)
        for _ in range(max(W // 4, 2)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(K // 8, 4)
        e0, e1 = hev.create(), hev.create()
        hev.record(e0)
        for _ in range(reps):
            g.replay()
        hev.record(e1)
        torch.cuda.synchronize()
        t_c2g[M2] = hev.elapsed_ms(e0, e1) / (reps * len(q2))
        hev.destroy(e0)
        hev.destroy(e1)
        del g
    del q2
    progress("4096 x 4096 decode timed")

    # the measured ceilings: a plain read of the GEMV kernel's bytes (rotated
    # over 5 buffers like the weight copies), of 1 GiB, and the MFMA loop
    kb = gemv_kernel_bytes(out, inp, 1, r, ngroups)
    read_kb, _ = read_rate(kb // 16 * 16, 5, K)
    read_1g, _ = read_rate(1 << 30, 2, max(K // 2, 3))
    mfma_meas, mfma_wgs, mfma_waves, _ = mfma_rate()
    tile_bare, tile_deq = tile_rate(False), tile_rate(True)
    vendor_70b = vendor_gemm(Mtrain, out, inp)
    vendor_7b = vendor_gemm(M7, sh7["out"], sh7["inp"])
    progress("ceilings measured")

    # ------------------------------------------------ the line
    dec_bytes = decode_bytes(out, inp, 1, r, ngroups)
    value = dec_bytes / (t_dec * 1e-3) / 1e9
    k_ms = float(np.mean(k_dec))
    achieved = kb / (k_ms * 1e-3) / 1e9
    kbw = dx_gemv_kernel_bytes(out, inp, 1, r, ngroups)
    kbw_ms = float(np.mean(k_dbw))
    ffwd, fbwd = train_flops(out, inp, Mtrain, r)
    tflops = (ffwd + fbwd) / (t_tr * 1e-3) / 1e12
    gemm_flops = 2 * Mtrain * out * (inp + r)
    dx_flops = 2 * Mtrain * out * inp + 2 * Mtrain * r * inp
    kf_ms, kd_ms = float(np.mean(fwd_k)), float(np.mean(bwd_k))
    f7 = sum(train_flops(sh7["out"], sh7["inp"], M7, r7))
    f7_fwd = 2 * M7 * sh7["out"] * (sh7["inp"] + r7)
    f7_dx = 2 * M7 * sh7["out"] * sh7["inp"] + 2 * M7 * r7 * sh7["inp"]
    k7f, k7d = float(np.mean(fwd7_k)), float(np.mean(bwd7_k))
    mu_flops = 2 * Mm * shm["out"] * shm["inp"] + 2 * Mm * shm["r"] * (shm["inp"] + shm["out"])
    mu_base = 2 * Mm * shm["out"] * shm["inp"]
    k_mu = float(np.mean(mu_k))
    ng2 = (sh2["out"] * sh2["inp"] // 64 + 255) // 256

    def tf(fl, ms):
        return fl / (ms * 1e-3) / 1e12

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "settle_ms": SETTLE_MS,
        "ms_per_step": round(t_dec, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random W0 of the workload's distribution, no trained weights)",
        "config": {
            "workload": "70B MLP 8192->28672 NF4 (block 64) + int8 double quant (group 256), "
                        "r=64 alpha=128; decode M=1 fwd, training M=4096 fwd+bwd",
            "out": out, "in": inp, "r": r, "alpha": sh["alpha"], "M_decode": 1, "M_train": Mtrain,
            "weight_copies_rotated": len(qs),
        },
        "decode_ms": round(t_dec, 5),
        "decode_GBps": round(value, 2),
        "decode_bwd_ms": round(t_dbw, 5),
        "train_ms_fwd_bwd": round(t_tr, 4),
        "train_TFLOPs": round(tflops, 2),
        "train_frac_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("k_gemv1"),
            "kernel": "k_gemv1 (fused dequant product, M=1)", "kernel_ms": round(k_ms, 5),
            "kernel_ms_what": KERNEL_MS_WHAT,
            "algorithmic_bytes_per_launch": kb,
            "peak_measured": round(read_kb, 1),
            "peak_measured_what": "plain read of the same bytes from HBM (5 rotated buffers)",
            "frac_measured": round(achieved / read_kb, 4),
        },
        "ceilings_measured": {
            "read_GBps_kernel_bytes": round(read_kb, 1),
            "read_GBps_1GiB": round(read_1g, 1),
            "mfma_bf16_TFLOPs": round(mfma_meas, 1),
            "mfma_loop": "%d workgroups x %d waves, 8 independent v_mfma_f32_32x32x16_bf16 per wave"
                         % (mfma_wgs, mfma_waves),
            "gemm_structure_TFLOPs": round(tile_bare, 1),
            "gemm_structure_dequant_TFLOPs": round(tile_deq, 1),
            "gemm_structure": "the fused GEMM's inner loop without memory traffic: 8 waves per CU, each a 256x32 "
                              "slab, one 16-byte LDS A-fragment read per MFMA; _dequant adds the byte-plane lookup "
                              "of one B operand per 8 MFMAs",
            "vendor_bf16_gemm_70b_M4096": vendor_70b,
            "vendor_bf16_gemm_7b_M2048": vendor_7b,
            "vendor_bf16_gemm": "context only: torch.mm / linear (hipBLASLt) on plain bf16 operands of the same "
                                "shapes, no dequantization",
        },
        "roofline_train": {
            "bound": "mfma", "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "peak_measured": round(mfma_meas, 1),
            "forward_kernel_ms": round(kf_ms, 4),
            "forward_achieved": round(tf(gemm_flops, kf_ms), 2),
            "forward_frac": round(tf(gemm_flops, kf_ms) / MFMA_BF16_PEAK_TFLOPS, 4),
            "forward_frac_measured": round(tf(gemm_flops, kf_ms) / mfma_meas, 4),
            "forward_frac_structure": round(tf(gemm_flops, kf_ms) / tile_deq, 4),
            "dx_kernel_ms": round(kd_ms, 4),
            "dx_achieved": round(tf(dx_flops, kd_ms), 2),
            "dx_frac": round(tf(dx_flops, kd_ms) / MFMA_BF16_PEAK_TFLOPS, 4),
            "dx_frac_measured": round(tf(dx_flops, kd_ms) / mfma_meas, 4),
            "traffic_forward": measured_traffic("k_fwd_rd"),
            "traffic_dx": measured_traffic("k_dx_rd"),
        },
        "roofline_decode_bwd": {
            "bound": "hbm", "kernel": "k_dxv (dX and dU pass over the weight rows, M=1)",
            "kernel_ms": round(kbw_ms, 5), "kernel_ms_what": KERNEL_MS_WHAT,
            "algorithmic_bytes_per_launch": kbw,
            "achieved": round(kbw / (kbw_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kbw / (kbw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "frac_measured": round(kbw / (kbw_ms * 1e-3) / 1e9 / read_kb, 4),
            "traffic": measured_traffic("k_dxv"),
        },
        "decode_4096": {
            "workload": "4096x4096 NF4 + double quant, r=16 alpha=32, forward, 64 rotated weight copies",
            **{"M%d" % M2: {"ms": round(t, 5),
                            "GBps": round(decode_bytes(4096, 4096, M2, sh2["r"], ng2) / (t * 1e-3) / 1e9, 2),
                            "frac_hbm_peak": round(decode_bytes(4096, 4096, M2, sh2["r"], ng2) / (t * 1e-3) / 1e9
                                                   / HBM_PEAK_GBS, 4)}
               for M2, t in t_c2.items()},
            "graph": {
                "what": "the same calls, one per weight copy, captured in one HIP graph and replayed (no host cost "
                        "per call)",
                **{"M%d" % M2: {"ms": round(t, 5),
                                "GBps": round(decode_bytes(4096, 4096, M2, sh2["r"], ng2) / (t * 1e-3) / 1e9, 2),
                                "frac_hbm_peak": round(decode_bytes(4096, 4096, M2, sh2["r"], ng2) / (t * 1e-3)
                                                       / 1e9 / HBM_PEAK_GBS, 4)}
                   for M2, t in t_c2g.items()}},
        },
        "train_7b": {
            "workload": "7B MLP %d->%d NF4 + double quant, r=%d, M=%d, forward + backward" % (
                sh7["inp"], sh7["out"], r7, M7),
            "ms": round(t_7b, 4), "TFLOPs": round(tf(f7, t_7b), 2),
            "frac_mfma_peak": round(tf(f7, t_7b) / MFMA_BF16_PEAK_TFLOPS, 4),
            "forward_kernel_ms": round(k7f, 4),
            "forward_frac": round(tf(f7_fwd, k7f) / MFMA_BF16_PEAK_TFLOPS, 4),
            "dx_kernel_ms": round(k7d, 4),
            "dx_frac": round(tf(f7_dx, k7d) / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "multi_adapter": {
            "workload": "%d adapters r=%d on %d->%d NF4 base, %d tokens" % (
                shm["n_adapters"], shm["r"], shm["inp"], shm["out"], Mm),
            "ms": round(t_mu, 4), "TFLOPs": round(tf(mu_flops, t_mu), 2),
            "frac_mfma_peak": round(tf(mu_flops, t_mu) / MFMA_BF16_PEAK_TFLOPS, 4),
            "base_kernel_ms": round(k_mu, 4),
            "base_kernel_frac": round(tf(mu_base, k_mu) / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "cpu_baseline": None,
    }
    if k_ms > t_dec:
        print("warning: the GEMV's event-measured time %.5f ms exceeds the step's %.5f ms" % (k_ms, t_dec),
              file=sys.stderr)
    extra_timings(line, args, timed, torch, F, wl, dev, bf, ws, copies_of, qs, A, B, x1, scale, sh, out, inp, r,
                  ngroups, Mtrain, xt, dH, ht, t_tr, ffwd, fbwd, q7, x7, dH7, A7, B7, s7, sh7, M7, r7, h7, f7, t_7b, settle)
    progress("merge, AdamW, blocks of 128, FP4 and dropout timed")
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["cpu_baseline_other"] = cpu_baselines()
        progress("oracle baselines timed")
    print(json.dumps(line), flush=True)


def extra_timings(line, args, timed, torch, F, wl, dev, bf, ws, copies_of, qs, A, B, x1, scale, sh, out, inp, r,
                  ngroups, Mtrain, xt, dH, ht, t_tr, ffwd, fbwd, q7, x7, dH7, A7, B7, s7, sh7, M7, r7, h7, f7, t_7b,
                  settle):
    """The rows beyond the hot path: merge, AdamW, blocks of 128, FP4, dropout."""
    K, W = args.steps, args.warmup
    wm = torch.empty((out, inp), dtype=torch.bfloat16, device=dev)
    t_mg, _ = timed(lambda i: F.qlora_merge(qs[i % len(qs)], A, B, scale, out=wm), K, W)
    del wm
    n_ad = r * (inp + out)
    pa = torch.randn(n_ad, device=dev)
    ga = torch.randn(n_ad, device=dev) * 1e-3
    ma, va = torch.zeros(n_ad, device=dev), torch.zeros(n_ad, device=dev)
    pab = torch.empty(n_ad, dtype=torch.bfloat16, device=dev)
    t_ad, _ = timed(lambda i: F.qlora_adamw_step(pa, ga, ma, va, i + 1, 1e-4, 0.9, 0.999, 1e-8, 0.01, p_bf16=pab),
                    K, W)
    ad_bytes = 30 * n_ad  # p, m, v read and written, g read, the bf16 copy written
    # blocks of 128: the decode step and the 7B training pass
    wt = torch.from_numpy(wl.weight(4)).to(dev)
    q0 = F.nf4_quantize(wt, double_quant=True, block_size=128)
    del wt
    q128 = [q0] + [F.NF4Weight(q0.codes.clone(), q0.absmax.clone(), q0.scale_codes.clone(), q0.group_absmax.clone(),
                               out, inp, True, 256, 128) for _ in range(2)]
    h1 = torch.empty((1, out), dtype=torch.bfloat16, device=dev)
    ws_d128 = ws(F.QLORA_OP_FORWARD | F.QLORA_OP_BLOCK128, out, inp, 1, r)
    d128_step = (lambda i: F.qlora_linear_forward(q128[i % len(q128)], x1, A, B, scale, ws=ws_d128, out=h1))
    settle(d128_step)
    t_d128, _ = timed(d128_step, K, W)
    del q128, q0
    # FP4 codes (the other quant type): the decode step and the 7B training pass
    wt = torch.from_numpy(wl.weight(4)).to(dev)
    q0 = F.nf4_quantize(wt, double_quant=True, quant_type="fp4")
    del wt
    qf4 = [q0] + [F.NF4Weight(q0.codes.clone(), q0.absmax.clone(), q0.scale_codes.clone(), q0.group_absmax.clone(),
                              out, inp, True, 256, 64, "fp4") for _ in range(len(qs) - 1)]
    ws_f1 = ws(F.QLORA_OP_FORWARD, out, inp, 1, r)
    f4_step = (lambda i: F.qlora_linear_forward(qf4[i % len(qf4)], x1, A, B, scale, ws=ws_f1, out=h1))
    settle(f4_step)
    t_f4, _ = timed(f4_step, K, W)
    del qf4, q0
    q7f = F.nf4_quantize(torch.from_numpy(wl.weight(3)).to(dev), double_quant=True, quant_type="fp4")
    wsf7f = ws(F.QLORA_OP_FORWARD, sh7["out"], sh7["inp"], M7, r7)
    wsb7f = ws(F.QLORA_OP_BACKWARD, sh7["out"], sh7["inp"], M7, r7)

    def train7_fp4_step(i):
        _, u = F.qlora_linear_forward(q7f, x7, A7, B7, s7, want_u=True, ws=wsf7f, out=h7)
        F.qlora_linear_backward(q7f, x7, dH7, A7, B7, s7, u=u, ws=wsb7f)

    t_7bf4, _ = timed(train7_fp4_step, K, W)
    del q7f, wsf7f, wsb7f
    q7b = F.nf4_quantize(torch.from_numpy(wl.weight(3)).to(dev), double_quant=True, block_size=128)
    wsf7b = ws(F.QLORA_OP_FORWARD | F.QLORA_OP_BLOCK128, sh7["out"], sh7["inp"], M7, r7)
    wsb7b = ws(F.QLORA_OP_BACKWARD | F.QLORA_OP_BLOCK128, sh7["out"], sh7["inp"], M7, r7)

    def train7_128_step(i):
        _, u = F.qlora_linear_forward(q7b, x7, A7, B7, s7, want_u=True, ws=wsf7b, out=h7)
        F.qlora_linear_backward(q7b, x7, dH7, A7, B7, s7, u=u, ws=wsb7b)

    t_7b128, _ = timed(train7_128_step, K, W)
    del q7b, wsf7b, wsb7b
    P_DROP = 0.05
    wsf7d = ws(F.QLORA_OP_FORWARD | F.QLORA_OP_DROPOUT, sh7["out"], sh7["inp"], M7, r7)
    wsb7d = ws(F.QLORA_OP_BACKWARD | F.QLORA_OP_DROPOUT, sh7["out"], sh7["inp"], M7, r7)

    def train7_drop_step(i):
        _, u = F.qlora_linear_forward(q7, x7, A7, B7, s7, want_u=True, ws=wsf7d, out=h7, dropout=(P_DROP, i))
        F.qlora_linear_backward(q7, x7, dH7, A7, B7, s7, u=u, ws=wsb7d, dropout=(P_DROP, i))

    t_7bd, _ = timed(train7_drop_step, K, W)
    del wsf7d, wsb7d
    ws_ftd = ws(F.QLORA_OP_FORWARD | F.QLORA_OP_DROPOUT, out, inp, Mtrain, r)
    ws_btd = ws(F.QLORA_OP_BACKWARD | F.QLORA_OP_DROPOUT, out, inp, Mtrain, r)

    def train_drop_step(i):
        _, u = F.qlora_linear_forward(qs[0], xt, A, B, scale, want_u=True, ws=ws_ftd, out=ht, dropout=(P_DROP, i))
        F.qlora_linear_backward(qs[0], xt, dH, A, B, scale, u=u, ws=ws_btd, dropout=(P_DROP, i))

    t_trd, _ = timed(train_drop_step, max(K // 2, 3), max(W // 2, 1))
    del ws_ftd, ws_btd
    ng128 = (out * inp // 128 + 255) // 256
    d128_bytes = decode_bytes(out, inp, 1, r, ng128, block=128)
    mg_bytes = out * inp // 2 + out * inp // 64 + 4 * ngroups + 2 * r * (inp + out) + 2 * out * inp
    HB, MF = HBM_PEAK_GBS, MFMA_BF16_PEAK_TFLOPS
    line["merge"] = {
        "workload": "adapter merged into the bf16 base weight, %d x %d, r=%d" % (out, inp, r),
        "ms": round(t_mg, 4), "GBps": round(mg_bytes / (t_mg * 1e-3) / 1e9, 2),
        "frac_hbm_peak": round(mg_bytes / (t_mg * 1e-3) / 1e9 / HB, 4),
    }
    line["adamw_step"] = {
        "workload": "AdamW on the layer's adapters, %d fp32 parameters" % n_ad,
        "ms": round(t_ad, 4), "GBps": round(ad_bytes / (t_ad * 1e-3) / 1e9, 2),
        "frac_hbm_peak": round(ad_bytes / (t_ad * 1e-3) / 1e9 / HB, 4),
    }
    line["block128"] = {
        "workload": "weights quantized in blocks of 128 (double quant, groups of 256 blocks): "
                    "the 70B decode step and the 7B training pass",
        "decode_ms": round(t_d128, 5),
        "decode_GBps": round(d128_bytes / (t_d128 * 1e-3) / 1e9, 2),
        "decode_frac_hbm_peak": round(d128_bytes / (t_d128 * 1e-3) / 1e9 / HB, 4),
        "train_7b_ms": round(t_7b128, 4),
        "train_7b_TFLOPs": round(f7 / (t_7b128 * 1e-3) / 1e12, 2),
        "train_7b_frac_mfma_peak": round(f7 / (t_7b128 * 1e-3) / 1e12 / MF, 4),
    }
    f4_bytes = decode_bytes(out, inp, 1, r, ngroups)
    line["fp4"] = {
        "workload": "weights quantized to FP4 (E2M1 codes, levels value/6; blocks of 64, double quant in groups "
                    "of 256): the 70B decode step and the 7B training pass",
        "decode_ms": round(t_f4, 5),
        "decode_GBps": round(f4_bytes / (t_f4 * 1e-3) / 1e9, 2),
        "decode_frac_hbm_peak": round(f4_bytes / (t_f4 * 1e-3) / 1e9 / HB, 4),
        "train_7b_ms": round(t_7bf4, 4),
        "train_7b_TFLOPs": round(f7 / (t_7bf4 * 1e-3) / 1e12, 2),
        "train_7b_frac_mfma_peak": round(f7 / (t_7bf4 * 1e-3) / 1e12 / MF, 4),
    }
    line["dropout"] = {
        "workload": "the training pass (M=%d) and the 7B training pass with dropout p=%g on the adapter "
                    "input (keep decisions from Philox-4x32-10, a new seed every step)" % (Mtrain, P_DROP),
        "train_ms": round(t_trd, 4),
        "train_TFLOPs": round((ffwd + fbwd) / (t_trd * 1e-3) / 1e12, 2),
        "train_vs_p0": round(t_trd / t_tr, 4),
        "train_7b_ms": round(t_7bd, 4),
        "train_7b_TFLOPs": round(f7 / (t_7bd * 1e-3) / 1e12, 2),
        "train_7b_vs_p0": round(t_7bd / t_7b, 4),
    }


if __name__ == "__main__":
    main()
