"""Shared helpers for the GPU parity tests (the oracle side is always computed
from the seeded inputs, never from GPU results)."""

import numpy as np

from oracle import nf4_oracle as O


def dev():
    import torch

    return torch.device("cuda:0")


def bf(bits: np.ndarray):
    """uint16 bf16 bit patterns -> bfloat16 CUDA tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def f32(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def bits_of(t) -> np.ndarray:
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(t) -> np.ndarray:
    return O.bf16_bits_to_f32(bits_of(t)).astype(np.float64)


def assert_close(name, got, ref):
    ok, worst = O.tolerance_ok(got, ref)
    assert ok, "%s: outside |err| <= 1e-2|ref| + 1e-3 rms(ref) (worst %.3f of the bound)" % (name, worst)
    return worst


def oracle_quantize_chunked(w_flat: np.ndarray, dq: bool, group: int = 256, chunk_groups: int = 64):
    """The oracle's quantize over a long flat array, in group-aligned chunks
    (the same result as one call; chunking only bounds memory)."""
    step = 64 * group * chunk_groups
    codes, absmax, sc, ga = [], [], [], []
    for s in range(0, w_flat.size, step):
        q = O.quantize(w_flat[s:s + step], double_quant=dq, dq_group=group)
        codes.append(q["codes"])
        absmax.append(q["absmax"])
        if dq:
            sc.append(q["scale_codes"])
            ga.append(q["group_absmax"])
    out = {"codes": np.concatenate(codes), "absmax": np.concatenate(absmax),
           "scale_codes": None, "group_absmax": None}
    if dq:
        out["scale_codes"] = np.concatenate(sc)
        out["group_absmax"] = np.concatenate(ga)
    return out


def oracle_weight_rows(w: np.ndarray, rows, dq: bool, group: int = 256):
    """Oracle Wb (float64) for selected rows of W [out, in].  Each row is
    quantized inside its whole double-quant group (groups are runs of `group`
    blocks of the flattened tensor), so the group constant is the true one."""
    out, cols = w.shape
    flat = w.reshape(-1)
    gelems = 64 * group
    res = {}
    for o in rows:
        if dq:
            g0 = (o * cols) // gelems
            lo, hi = g0 * gelems, min((g0 + 1) * gelems, flat.size)
            # a row may straddle two groups when cols does not divide the group
            if (o + 1) * cols > hi:
                hi = min(hi + gelems, flat.size)
            q = O.quantize(flat[lo:hi], double_quant=True, dq_group=group)
            wb = O.compute_weight(q, (hi - lo,))
            res[o] = wb[o * cols - lo:(o + 1) * cols - lo]
        else:
            q = O.quantize(w[o:o + 1], double_quant=False)
            res[o] = O.compute_weight(q, (cols,))
    return res


def oracle_weight_cols(w: np.ndarray, cols_idx, dq: bool = True, group: int = 256,
                       chunk_groups: int = 64) -> np.ndarray:
    """Oracle Wb (float64) at every row of the selected columns of W [out, in]:
    the whole tensor is quantized by the oracle in group-aligned chunks (the
    same result as one call) and only the selected columns are kept."""
    out, cols = w.shape
    flat = w.reshape(-1)
    cols_idx = np.asarray(cols_idx)
    res = np.empty((out, cols_idx.size), dtype=np.float64)
    step = 64 * group * chunk_groups
    for lo in range(0, flat.size, step):
        hi = min(lo + step, flat.size)
        q = O.quantize(flat[lo:hi], double_quant=dq, dq_group=group)
        wb = O.compute_weight(q, (hi - lo,))
        r0, r1 = lo // cols, (hi + cols - 1) // cols
        for o in range(r0, r1):
            idx = o * cols + cols_idx
            sel = (idx >= lo) & (idx < hi)
            res[o, sel] = wb[idx[sel] - lo]
    return res


def oracle_rows_dequant(qref, o0: int, o1: int, cols: int, group: int = 256) -> np.ndarray:
    """Oracle Wb (float64) of rows [o0, o1) of a weight the oracle quantized
    as a whole (double quant): the slice of its codes, scale codes and group
    constants, decoded by the oracle.  The slice must start on a group."""
    b0, b1 = o0 * cols // 64, o1 * cols // 64
    assert b0 % group == 0
    g0, g1 = b0 // group, (b1 + group - 1) // group
    part = {"codes": qref["codes"][o0 * cols // 2:o1 * cols // 2], "absmax": qref["absmax"][b0:b1],
            "scale_codes": qref["scale_codes"][b0:b1], "group_absmax": qref["group_absmax"][g0:g1]}
    return O.compute_weight(part, (o1 - o0, cols), dq_group=group)


def weight_from_oracle(F, qref, rows: int, cols: int, dq: bool, group: int = 256):
    """An NF4Weight on the GPU holding the oracle's own storage (codes,
    scales): the layer calls then read exactly what the oracle dequantizes."""
    import torch

    d = dev()
    codes = torch.from_numpy(np.ascontiguousarray(qref["codes"])).to(d)
    absmax = torch.from_numpy(np.ascontiguousarray(qref["absmax"])).to(d)
    sc = ga = None
    if dq:
        sc = torch.from_numpy(np.ascontiguousarray(qref["scale_codes"])).to(d)
        ga = torch.from_numpy(np.ascontiguousarray(qref["group_absmax"])).to(d)
    return F.NF4Weight(codes, absmax, sc, ga, rows, cols, dq, group, 64, qref.get("quant_type", "nf4"))
