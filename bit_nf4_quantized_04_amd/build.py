"""Build libnf4qlora.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m bit_nf4_quantized_04_amd.build

Each .hip file under csrc/ is compiled with hipcc for gfx950 only and the
objects are linked into bit_nf4_quantized_04_amd/libnf4qlora.so.  The
measurement kernels under csrc/calib/ (a plain read and an MFMA loop, the
achievable ceilings the benchmark quotes) go into libnf4calib.so.  Packed
fp32 instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libnf4qlora.so")
CALIB_OUT = os.path.join(HERE, "libnf4calib.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=fast",
    "-fno-strict-aliasing",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    errs = [l for l in res.stderr.splitlines() if "error" in l]
    if errs:
        raise RuntimeError("\n".join(errs))
    return obj


def _torch_lib_dir():
    """The directory of torch's bundled HIP runtime: the library resolves its
    libamdhip64 from there first, so torch and the kernels share one runtime."""
    import importlib.util

    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return None
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def _link(objs, out):
    tmp = out + ".tmp"
    tl = _torch_lib_dir()
    link = ["-L" + tl, "-Wl,-rpath," + tl] if tl else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    calib = sources(os.path.join(CSRC, "calib"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(calib))) as ex:
        objs = list(ex.map(_compile, srcs + calib))
    _link(objs[:len(srcs)], OUT)
    _link(objs[len(srcs):], CALIB_OUT)
    if verbose:
        print("built", OUT, "and", CALIB_OUT)
    return OUT


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
