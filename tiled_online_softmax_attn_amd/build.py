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
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_kv.hip", "attn_bwd.hip", "attn_bwd_dkdv.hip",
           "softmax_rows.hip", "attn_fwd_mx.hip"]
# Sources whose MFMAs all write ordinary registers (LLVM's VGPR form).  In a
# kernel that also needs accumulation registers the compiler otherwise gives
# every MFMA an accumulation-register destination, and each value the VALU
# reads back costs a v_accvgpr_read.  Bitwise the same results; measured on
# MI355X (B4 H16 N4096 causal): dK/dV 3% faster at d = 128 and 7% at d = 96,
# the d = 256 forward (the only forward kernel that needs accumulation
# registers; the others compile to the same code) 8% faster.  Not
# attn_bwd.hip: its d = 256 dQ kernel is 4% slower in that form.
VGPR_FORM_SOURCES = {"attn_bwd_dkdv.hip", "attn_fwd.hip"}
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


def source_flags(src: str) -> list[str]:
    """Compiler flags of one source beyond FLAGS."""
    return ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src in VGPR_FORM_SOURCES else []


def _compile(src: str, obj_dir: str, extra: list[str]) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *source_flags(src), *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
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
