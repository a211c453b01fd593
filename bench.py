"""Benchmark of the NF4 QLoRA linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 70b|7b|decode]

Workload (default "70b"): the 70B MLP projection 8192 -> 28672 (W0 [28672, 8192],
99.9% N(0, 0.015^2) entries and 0.1% 0.1 * Student-t(3) outliers), NF4 blocks of
64 with int8 double quantization in groups of 256, r = 64, alpha = 128, synthetic
seeded inputs.  One step is one pass of the layer's hot path:
  * decode: the fused dequant-GEMV forward at M = 1 (u = x A^T, then
    h = x Wb^T + s u B^T), rotating over 5 resident copies of the quantized
    weight (630 MB > the 256 MB last-level cache) so every call streams W from HBM;
  * training: forward (u and h) and backward (dX, dA, dB) at M = 4096.
`value` is the decode throughput in algorithmic GB/s (the headline metric's
first figure); the training pass is reported as bf16 TFLOP/s in the same line.
Inputs are resident in HBM before the timed region starts.  Rank 0 prints one
JSON line.
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
WORKLOADS = {"decode": 2, "7b": 3, "70b": 4}


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


def train_flops(out, inp, M, r):
    fwd = 2 * M * out * inp + 2 * M * r * (inp + out)
    bwd = 2 * M * out * inp + 4 * M * out * r + 4 * M * r * inp
    return fwd, bwd


def cpu_baseline(c, w, x_bits, a_bits, b_bits, scale, budget_s=10.0):
    """The oracle (as it stands) doing the decode step on row samples of the
    same weight, until about `budget_s` seconds of CPU work; GB/s of the same
    algorithmic bytes."""
    from oracle import nf4_oracle as O

    out, inp = w.shape
    rows_per = 16384 * 64 // inp  # 64 double-quant groups per sample
    rng = np.random.default_rng(0)
    # a handful of distinct row samples, quantized once (offline: not timed)
    picks = [int(g) * rows_per for g in rng.choice(out // rows_per, size=min(8, out // rows_per),
                                                   replace=False)]
    prepared = [(g0, O.quantize(np.ascontiguousarray(w[g0:g0 + rows_per]), double_quant=True))
                for g0 in picks]
    ng = (rows_per * inp // 64 + 255) // 256
    done_bytes, spent, samples = 0, 0.0, 0
    while spent < budget_s:
        g0, qt = prepared[samples % len(prepared)]
        t0 = time.perf_counter()
        wb = O.compute_weight(qt, (rows_per, inp))
        _ = O.forward(wb, x_bits, a_bits, b_bits[g0:g0 + rows_per], scale)
        spent += time.perf_counter() - t0
        done_bytes += decode_bytes(rows_per, inp, 1, a_bits.shape[0], ng, with_A=True)
        samples += 1
    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return {
        "value": done_bytes / spent / 1e9,
        "unit": "GB/s",
        "cores": int(blas),
        "kind": "oracle",
        "sample": "%d samples of %d rows x %d (64 double-quant groups each) of the workload weight: "
                  "oracle dequantize + bf16 cast (NumPy elementwise, 1 thread) and the float64 "
                  "forward at M=1 (BLAS, %d threads); %.1f s of CPU work"
                  % (samples, rows_per, inp, blas, spent),
    }


def copy_calibration(torch, dev, K, W, nbytes=512 << 20):
    """A plain copy of known size (nbytes read + nbytes written per launch):
    what the HBM byte counters read for it scales the counters of the layer's
    kernels."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    for _ in range(W):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / K
    print("copy pass: %d bytes read + %d written per launch, %.4f ms/launch (%.1f GB/s)"
          % (nbytes, nbytes, dt * 1e3, 2 * nbytes / dt / 1e9), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="70b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=5)
    ap.add_argument("--only", choices=["decode", "decode_bwd", "train", "multi", "copy"], default=None,
                    help="profile one pass only (no JSON line); 'copy' runs a plain 512 MiB "
                         "device-to-device copy, the calibration for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: sharding the layer over several GPUs is "
              "not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_nf4_quantized_04_amd import nf4qlora as F
    from bit_nf4_quantized_04_amd import workloads as wl

    dev = torch.device("cuda:0")
    if args.only == "copy":
        copy_calibration(torch, dev, args.steps, args.warmup)
        return
    c = WORKLOADS[args.workload]
    sh = wl.SHAPES[c]
    out, inp, r = sh["out"], sh["inp"], sh["r"]
    scale = sh["alpha"] / r
    Mtrain = max(sh["M"])

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- setup (untimed): inputs resident in HBM
    w = wl.weight(c)
    x1_bits = wl.activations(c, 1)
    a_bits, b_bits = wl.adapters(c)
    wt = torch.from_numpy(w).to(dev)
    qs = [F.nf4_quantize(wt, double_quant=True)]
    for _ in range(args.copies - 1):
        q0 = qs[0]
        qs.append(F.NF4Weight(q0.codes.clone(), q0.absmax.clone(), q0.scale_codes.clone(),
                              q0.group_absmax.clone(), out, inp, True))
    del wt
    x1, A, B = bf(x1_bits), bf(a_bits), bf(b_bits)
    xt = bf(wl.activations(c, Mtrain))
    dH = bf(wl.upstream_grad(c, Mtrain))
    ws_f1 = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, out, inp, 1, r), 256),
                        dtype=torch.uint8, device=dev)
    ws_ft = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, out, inp, Mtrain, r), 256),
                        dtype=torch.uint8, device=dev)
    ws_bt = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD, out, inp, Mtrain, r), 256),
                        dtype=torch.uint8, device=dev)
    h1 = torch.empty((1, out), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((Mtrain, out), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    ngroups = (out * inp // 64 + 255) // 256

    def decode_step(i):
        F.qlora_linear_forward(qs[i % len(qs)], x1, A, B, scale, ws=ws_f1, out=h1)

    _, u1 = F.qlora_linear_forward(qs[0], x1, A, B, scale, want_u=True, ws=ws_f1, out=h1)
    dH1 = bf(wl.upstream_grad(c, 1))
    ws_b1 = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD, out, inp, 1, r), 256),
                        dtype=torch.uint8, device=dev)

    def decode_bwd_step(i):
        F.qlora_linear_backward(qs[i % len(qs)], x1, dH1, A, B, scale, u=u1, ws=ws_b1)

    # the multi-adapter forward (its own workload: 64 adapters on a 4096 x 4096 base)
    cm = 5
    shm = wl.SHAPES[cm]
    Mm = max(shm["M"]) if isinstance(shm["M"], (list, tuple)) else shm["M"]
    wtm = torch.from_numpy(wl.weight(cm)).to(dev)
    qm = F.nf4_quantize(wtm, double_quant=True)
    del wtm
    abm, bbm = wl.adapter_bank(cm)
    xm = bf(wl.activations(cm, Mm))
    Abm, Bbm = bf(abm), bf(bbm)
    idsm = torch.from_numpy(wl.adapter_ids(cm, Mm, shm["n_adapters"])).to(dev)
    scm = torch.full((shm["n_adapters"],), shm["alpha"] / shm["r"], dtype=torch.float32, device=dev)
    hm = torch.empty((Mm, shm["out"]), dtype=torch.bfloat16, device=dev)
    wsm = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD_MULTI, shm["out"], shm["inp"], Mm, shm["r"],
                                                  shm["n_adapters"]), 256), dtype=torch.uint8, device=dev)

    def multi_step(i):
        F.qlora_linear_forward_multi(qm, xm, Abm, Bbm, scm, idsm, ws=wsm, out=hm)

    # the 7B MLP projection's training pass (its own workload, M = 2048)
    c7 = WORKLOADS["7b"]
    sh7 = wl.SHAPES[c7]
    M7 = max(sh7["M"])
    q7 = F.nf4_quantize(torch.from_numpy(wl.weight(c7)).to(dev), double_quant=True)
    a7, b7 = wl.adapters(c7)
    A7, B7 = bf(a7), bf(b7)
    x7, dH7 = bf(wl.activations(c7, M7)), bf(wl.upstream_grad(c7, M7))
    s7 = sh7["alpha"] / sh7["r"]
    wsf7 = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD, sh7["out"], sh7["inp"], M7, sh7["r"]), 256),
                       dtype=torch.uint8, device=dev)
    wsb7 = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD, sh7["out"], sh7["inp"], M7, sh7["r"]), 256),
                       dtype=torch.uint8, device=dev)
    h7 = torch.empty((M7, sh7["out"]), dtype=torch.bfloat16, device=dev)

    def train7_step(i):
        _, u = F.qlora_linear_forward(q7, x7, A7, B7, s7, want_u=True, ws=wsf7, out=h7)
        F.qlora_linear_backward(q7, x7, dH7, A7, B7, s7, u=u, ws=wsb7)

    wm = torch.empty((out, inp), dtype=torch.bfloat16, device=dev)

    def merge_step(i):
        F.qlora_merge(qs[i % len(qs)], A, B, scale, out=wm)

    # one AdamW step on the layer's adapters (A and B together), fp32 state in HBM
    n_ad = r * (inp + out)
    pa = torch.randn(n_ad, device=dev)
    ga = torch.randn(n_ad, device=dev) * 1e-3
    ma, va = torch.zeros(n_ad, device=dev), torch.zeros(n_ad, device=dev)
    pab = torch.empty(n_ad, dtype=torch.bfloat16, device=dev)

    def adamw_step(i):
        F.qlora_adamw_step(pa, ga, ma, va, i + 1, 1e-4, 0.9, 0.999, 1e-8, 0.01, p_bf16=pab)

    def train_step(i):
        _, u = F.qlora_linear_forward(qs[0], xt, A, B, scale, want_u=True, ws=ws_ft, out=ht)
        F.qlora_linear_backward(qs[0], xt, dH, A, B, scale, u=u, ws=ws_bt)

    hev = F.HipEvents()

    def timed(step, K, W, hook_events=None):
        """Mean ms per step over K steps (HIP events on the current stream),
        and with hook_events the dominant kernel's duration of every call."""
        for i in range(W):
            step(i)
        torch.cuda.synchronize()
        pairs = [(hev.create(), hev.create()) for _ in range(K)] if hook_events else []
        t0, t1 = hev.create(), hev.create()
        hev.record(t0)
        for i in range(K):
            if hook_events:
                F.nf4_profile_events(*pairs[i])
            step(i)
        hev.record(t1)
        torch.cuda.synchronize()
        F.nf4_profile_events(None, None)
        total = hev.elapsed_ms(t0, t1) / K
        kern = [hev.elapsed_ms(a, b) for a, b in pairs]
        for e in [t0, t1] + [e for p in pairs for e in p]:
            hev.destroy(e)
        return total, kern

    # whole-step timing (no hook), then the dominant kernel with the hook
    K, W = args.steps, args.warmup
    if args.only:
        step = {"decode": decode_step, "decode_bwd": decode_bwd_step, "train": train_step,
                "multi": multi_step}[args.only]
        t, _ = timed(step, K, W)
        print("%s pass: %.4f ms/step over %d steps" % (args.only, t, K), flush=True)
        return
    t_dec, _ = timed(decode_step, K, W)
    _, k_dec = timed(decode_step, K, 1, hook_events=True)
    t_dbw, _ = timed(decode_bwd_step, K, W)
    _, k_dbw = timed(decode_bwd_step, K, 1, hook_events=True)
    t_tr, _ = timed(train_step, max(K // 2, 3), max(W // 2, 1))
    t_mu, _ = timed(multi_step, K, W)
    t_7b, _ = timed(train7_step, K, W)
    t_mg, _ = timed(merge_step, K, W)
    t_ad, _ = timed(adamw_step, K, W)
    ad_bytes = 30 * n_ad  # p, m, v read and written, g read, the bf16 copy written
    # the decode step and the 7B training pass on weights quantized in blocks
    # of 128 (the layer calls expand the scales per 64-element half first)
    wt = torch.from_numpy(w).to(dev)
    q128 = [F.nf4_quantize(wt, double_quant=True, block_size=128)]
    del wt
    for _ in range(2):
        q0 = q128[0]
        q128.append(F.NF4Weight(q0.codes.clone(), q0.absmax.clone(), q0.scale_codes.clone(),
                                q0.group_absmax.clone(), out, inp, True, 256, 128))
    ws_d128 = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD | F.QLORA_OP_BLOCK128, out, inp, 1, r),
                              256), dtype=torch.uint8, device=dev)

    def decode128_step(i):
        F.qlora_linear_forward(q128[i % len(q128)], x1, A, B, scale, ws=ws_d128, out=h1)

    t_d128, _ = timed(decode128_step, K, W)
    del q128
    q7b = F.nf4_quantize(torch.from_numpy(wl.weight(c7)).to(dev), double_quant=True, block_size=128)
    wsf7b = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD | F.QLORA_OP_BLOCK128, sh7["out"], sh7["inp"],
                                                    M7, sh7["r"]), 256), dtype=torch.uint8, device=dev)
    wsb7b = torch.empty(max(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD | F.QLORA_OP_BLOCK128, sh7["out"], sh7["inp"],
                                                    M7, sh7["r"]), 256), dtype=torch.uint8, device=dev)

    def train7_128_step(i):
        _, u = F.qlora_linear_forward(q7b, x7, A7, B7, s7, want_u=True, ws=wsf7b, out=h7)
        F.qlora_linear_backward(q7b, x7, dH7, A7, B7, s7, u=u, ws=wsb7b)

    t_7b128, _ = timed(train7_128_step, K, W)
    del q7b, wsf7b, wsb7b
    # the two training passes with dropout p = 0.05 on the adapter input
    P_DROP = 0.05
    wsf7d = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD | F.QLORA_OP_DROPOUT, sh7["out"], sh7["inp"],
                                                M7, sh7["r"]), dtype=torch.uint8, device=dev)
    wsb7d = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD | F.QLORA_OP_DROPOUT, sh7["out"], sh7["inp"],
                                                M7, sh7["r"]), dtype=torch.uint8, device=dev)

    def train7_drop_step(i):
        _, u = F.qlora_linear_forward(q7, x7, A7, B7, s7, want_u=True, ws=wsf7d, out=h7, dropout=(P_DROP, i))
        F.qlora_linear_backward(q7, x7, dH7, A7, B7, s7, u=u, ws=wsb7d, dropout=(P_DROP, i))

    t_7bd, _ = timed(train7_drop_step, K, W)
    del wsf7d, wsb7d
    ws_ftd = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_FORWARD | F.QLORA_OP_DROPOUT, out, inp, Mtrain, r),
                         dtype=torch.uint8, device=dev)
    ws_btd = torch.empty(F.qlora_workspace_bytes(F.QLORA_OP_BACKWARD | F.QLORA_OP_DROPOUT, out, inp, Mtrain, r),
                         dtype=torch.uint8, device=dev)

    def train_drop_step(i):
        _, u = F.qlora_linear_forward(qs[0], xt, A, B, scale, want_u=True, ws=ws_ftd, out=ht, dropout=(P_DROP, i))
        F.qlora_linear_backward(qs[0], xt, dH, A, B, scale, u=u, ws=ws_btd, dropout=(P_DROP, i))

    t_trd, _ = timed(train_drop_step, max(K // 2, 3), max(W // 2, 1))
    del ws_ftd, ws_btd
    ng128 = (out * inp // 128 + 255) // 256
    d128_bytes = decode_bytes(out, inp, 1, r, ng128, block=128)
    mg_bytes = out * inp // 2 + out * inp // 64 + 4 * ngroups + 2 * r * (inp + out) + 2 * out * inp
    f7 = sum(train_flops(sh7["out"], sh7["inp"], M7, sh7["r"]))
    mu_flops = 2 * Mm * shm["out"] * shm["inp"] + 2 * Mm * shm["r"] * (shm["inp"] + shm["out"])
    # dominant kernels of the training pass: forward product and dX product
    fwd_k, bwd_k = [], []

    def train_fwd(i):
        F.qlora_linear_forward(qs[0], xt, A, B, scale, ws=ws_ft, out=ht)

    _, fwd_k = timed(train_fwd, max(K // 2, 3), 1, hook_events=True)
    _, u = F.qlora_linear_forward(qs[0], xt, A, B, scale, want_u=True, ws=ws_ft, out=ht)

    def train_bwd(i):
        F.qlora_linear_backward(qs[0], xt, dH, A, B, scale, u=u, ws=ws_bt)

    _, bwd_k = timed(train_bwd, max(K // 2, 3), 1, hook_events=True)

    dec_bytes = decode_bytes(out, inp, 1, r, ngroups)
    value = dec_bytes / (t_dec * 1e-3) / 1e9
    kb = gemv_kernel_bytes(out, inp, 1, r, ngroups)
    k_ms = float(np.mean(k_dec))
    achieved = kb / (k_ms * 1e-3) / 1e9
    kbw = dx_gemv_kernel_bytes(out, inp, 1, r, ngroups)
    kbw_ms = float(np.mean(k_dbw))
    ffwd, fbwd = train_flops(out, inp, Mtrain, r)
    tflops = (ffwd + fbwd) / (t_tr * 1e-3) / 1e12
    gemm_flops = 2 * Mtrain * out * (inp + r)
    kf_ms = float(np.mean(fwd_k))
    dx_flops = 2 * Mtrain * out * inp + 2 * Mtrain * r * inp
    kd_ms = float(np.mean(bwd_k))

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(t_dec, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random W0 of the workload's distribution, no trained weights)",
        "config": {
            "workload": "70B MLP 8192->28672 NF4 (block 64) + int8 double quant (group 256), "
                        "r=64 alpha=128; decode M=1 fwd, training M=4096 fwd+bwd"
                        if c == 4 else "workload %d (%d -> %d), r=%d" % (c, inp, out, r),
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
            "kernel": "fused dequant product, M=1", "kernel_ms": round(k_ms, 5),
            "algorithmic_bytes_per_launch": kb,
        },
        "train_7b": {
            "workload": "7B MLP %d->%d NF4 + double quant, r=%d, M=%d, forward + backward" % (
                sh7["inp"], sh7["out"], sh7["r"], M7),
            "ms": round(t_7b, 4), "TFLOPs": round(f7 / (t_7b * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(f7 / (t_7b * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "merge": {
            "workload": "adapter merged into the bf16 base weight, %d x %d, r=%d" % (out, inp, r),
            "ms": round(t_mg, 4), "GBps": round(mg_bytes / (t_mg * 1e-3) / 1e9, 2),
            "frac_hbm_peak": round(mg_bytes / (t_mg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "adamw_step": {
            "workload": "AdamW on the layer's adapters, %d fp32 parameters" % n_ad,
            "ms": round(t_ad, 4), "GBps": round(ad_bytes / (t_ad * 1e-3) / 1e9, 2),
            "frac_hbm_peak": round(ad_bytes / (t_ad * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "block128": {
            "workload": "weights quantized in blocks of 128 (double quant, groups of 256 blocks): "
                        "the 70B decode step and the 7B training pass",
            "decode_ms": round(t_d128, 5),
            "decode_GBps": round(d128_bytes / (t_d128 * 1e-3) / 1e9, 2),
            "decode_frac_hbm_peak": round(d128_bytes / (t_d128 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "train_7b_ms": round(t_7b128, 4),
            "train_7b_TFLOPs": round(f7 / (t_7b128 * 1e-3) / 1e12, 2),
            "train_7b_frac_mfma_peak": round(f7 / (t_7b128 * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "dropout": {
            "workload": "the training pass (M=%d) and the 7B training pass with dropout p=%g on the adapter "
                        "input (keep decisions from Philox-4x32-10, a new seed every step)" % (Mtrain, P_DROP),
            "train_ms": round(t_trd, 4),
            "train_TFLOPs": round((ffwd + fbwd) / (t_trd * 1e-3) / 1e12, 2),
            "train_vs_p0": round(t_trd / t_tr, 4),
            "train_7b_ms": round(t_7bd, 4),
            "train_7b_TFLOPs": round(f7 / (t_7bd * 1e-3) / 1e12, 2),
            "train_7b_vs_p0": round(t_7bd / t_7b, 4),
        },
        "multi_adapter": {
            "workload": "%d adapters r=%d on %d->%d NF4 base, %d tokens" % (
                shm["n_adapters"], shm["r"], shm["inp"], shm["out"], Mm),
            "ms": round(t_mu, 4), "TFLOPs": round(mu_flops / (t_mu * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(mu_flops / (t_mu * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "roofline_decode_bwd": {
            "bound": "hbm", "kernel": "dX and dU pass over the weight rows, M=1",
            "kernel_ms": round(kbw_ms, 5), "algorithmic_bytes_per_launch": kbw,
            "achieved": round(kbw / (kbw_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kbw / (kbw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": measured_traffic("k_dxv"),
        },
        "roofline_train": {
            "bound": "mfma", "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "forward_kernel_ms": round(kf_ms, 4),
            "forward_achieved": round(gemm_flops / (kf_ms * 1e-3) / 1e12, 2),
            "forward_frac": round(gemm_flops / (kf_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "dx_kernel_ms": round(kd_ms, 4),
            "dx_achieved": round(dx_flops / (kd_ms * 1e-3) / 1e12, 2),
            "dx_frac": round(dx_flops / (kd_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic_forward": measured_traffic("k_fwd_rd"),
            "traffic_dx": measured_traffic("k_dx_rd"),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, w, x1_bits, a_bits, b_bits, scale)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
