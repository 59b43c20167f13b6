"""Build libattn.so (the HIP library behind include/attn.h) for gfx950.

Run ``python -m tiled_online_softmax_attn_amd.build`` or call ``build()``.
Every source is compiled with hipcc for gfx950 only; packed-fp32 VALU
instructions are switched off for the device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_kv.hip", "attn_bwd.hip", "softmax_rows.hip", "attn_fwd_mx.hip"]
# the measured-ceiling probes (include/attn_probe.h), a library of their own
PROBE_LIB = os.path.join(PKG, "libattn_probe.so")
PROBE_SOURCES = ["roofline_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-fno-gpu-rdc",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, obj_dir: str, extra: list[str]) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if msgs:
        print(msgs, file=sys.stderr)
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link libattn.so (and libattn_probe.so) in the
    package directory."""
    extra = list(extra or [])
    if verbose:
        extra += ["-Rpass-analysis=kernel-resource-usage"]
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
