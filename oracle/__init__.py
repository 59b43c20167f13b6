"""fp64 CPU oracle for scaled-dot-product attention (test infrastructure).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It shares no code with the HIP library in
``tiled_online_softmax_attn_amd`` and never imports it.

The arithmetic lives in ``attn_oracle.c`` (plain C, double precision, S and P
materialised); this module only builds it with gcc, loads it with ctypes and
loops over heads.  What each C function follows on the pages is stated in
that file's header:

* ``softmax_row``   - safe softmax of one row (CS149 Lecture 9 notes
  "Efficiently Evaluating DNNs on GPUs", section 8; PDC notes Lecture 4,
  section 4.13.2).
* ``attn_fwd``      - O = softmax(scale * Q K^T [+ causal mask]) V and the
  per-row logsumexp (CS336 Lecture 5 notes "GPUs, TPUs", sections 8.1, 8.3).
* ``attn_fwd_rows`` - the same definition for selected query rows only.
* ``attn_fwd_rect`` - Nq queries at the end of an Nk-key sequence.
* ``attn_bwd``      - dQ, dK, dV of sum(dO * O) (CS336 L5 notes section 8.4,
  Exercise 9).
* ``attn_bwd_rect`` - the same gradient for Nq queries at the end of an
  Nk-key sequence (the backward of ``attn_fwd_rect``).
* ``attn_bwd_dq_rows`` - dQ for selected query rows only (each row of dQ
  depends on its own rows of P and dP), for sequences too long for the
  whole N x N gradient.
* ``mx_decode``     - values of an MXFP8 tensor (E4M3 codes, one E8M0 scale
  per 32 elements of a row; CS336 L5 notes section 6.2); attention of MXFP8
  inputs is ``attn_fwd`` of the decoded values.

Every function is pinned by ``tests/test_oracle_pins.py`` against values the
pages print, closed forms, brute force in 50-digit decimal arithmetic and
finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_DP = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)


def load(path: str | None = None):
    """Load (building first if needed) the oracle library and declare its ABI.

    With an explicit ``path`` a separate handle is returned (used by the
    tests that build deliberately broken copies of the oracle)."""
    global _lib
    if path is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH) or (
                        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                    build()
                _lib = _declare(ctypes.CDLL(_LIB_PATH))
            return _lib
    return _declare(ctypes.CDLL(path))


def _declare(lib):
    i64 = ctypes.c_int64
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_softmax_row.restype = ctypes.c_int
    lib.oracle_softmax_row.argtypes = [_DP, i64, _DP, _DP, _DP]
    lib.oracle_attn_fwd_head.restype = ctypes.c_int
    lib.oracle_attn_fwd_head.argtypes = [_DP, _DP, _DP, i64, i64, ctypes.c_int,
                                         ctypes.c_double, _DP, _DP, _DP]
    lib.oracle_attn_fwd_rows.restype = ctypes.c_int
    lib.oracle_attn_fwd_rows.argtypes = [_DP, _DP, _DP, i64, i64, ctypes.c_int,
                                         ctypes.c_double, _I64P, i64, _DP, _DP, _DP]
    lib.oracle_attn_fwd_rect.restype = ctypes.c_int
    lib.oracle_attn_fwd_rect.argtypes = [_DP, _DP, _DP, i64, i64, i64, ctypes.c_int,
                                         ctypes.c_double, _DP, _DP, _DP]
    lib.oracle_mx_decode.restype = ctypes.c_int
    lib.oracle_mx_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64, _DP]
    lib.oracle_attn_bwd_head.restype = ctypes.c_int
    lib.oracle_attn_bwd_head.argtypes = [_DP, _DP, _DP, _DP, i64, i64, ctypes.c_int,
                                         ctypes.c_double, _DP, _DP, _DP, _DP, _DP, _DP]
    lib.oracle_attn_bwd_dq_rows.restype = ctypes.c_int
    lib.oracle_attn_bwd_dq_rows.argtypes = [_DP, _DP, _DP, _DP, i64, i64, ctypes.c_int,
                                            ctypes.c_double, _I64P, i64, _DP]
    lib.oracle_attn_bwd_rect.restype = ctypes.c_int
    lib.oracle_attn_bwd_rect.argtypes = [_DP, _DP, _DP, _DP, i64, i64, i64, ctypes.c_int,
                                         ctypes.c_double, _DP, _DP, _DP, _DP, _DP, _DP]
    return lib


def _f64(a) -> np.ndarray:
    """Exact widening to a C-contiguous float64 array (accepts numpy arrays
    and CPU torch tensors of any float dtype)."""
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_DP)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def set_num_threads(n: int, lib=None) -> None:
    """Threads of later calls (for timing); results do not depend on it."""
    (lib or load()).oracle_set_num_threads(int(n))


def softmax_row(x, lib=None):
    """Returns (p, m, l) for one row; -inf entries are masked."""
    lib = lib or load()
    x = _f64(x).reshape(-1)
    p = np.empty_like(x)
    m = ctypes.c_double()
    l = ctypes.c_double()
    _check(lib.oracle_softmax_row(_ptr(x), x.size, _ptr(p), ctypes.byref(m),
                                  ctypes.byref(l)), "softmax_row")
    return p, m.value, l.value


def _heads(a):
    """View [..., N, d] as [G, N, d] with G the product of leading dims."""
    a = _f64(a)
    lead = a.shape[:-2]
    return a.reshape((-1,) + a.shape[-2:]), lead


def attn_fwd(q, k, v, causal: bool, scale: float, return_p: bool = False, lib=None):
    """O and lse for inputs of shape [..., N, d] (any leading head dims).

    Returns (o, lse) or (o, lse, p) with p of shape [..., N, N]."""
    lib = lib or load()
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    G, N, d = qh.shape
    o = np.empty_like(qh)
    lse = np.empty((G, N), dtype=np.float64)
    p = np.empty((G, N, N), dtype=np.float64) if return_p else None
    for g in range(G):
        rc = lib.oracle_attn_fwd_head(
            _ptr(qh[g]), _ptr(kh[g]), _ptr(vh[g]), N, d, int(bool(causal)),
            float(scale), _ptr(o[g]), _ptr(lse[g]),
            _ptr(p[g]) if return_p else ctypes.cast(None, _DP))
        _check(rc, "attn_fwd_head")
    o = o.reshape(lead + (N, d))
    lse = lse.reshape(lead + (N,))
    if return_p:
        return o, lse, p.reshape(lead + (N, N))
    return o, lse


def attn_fwd_rows(q, k, v, causal: bool, scale: float, rows, return_p: bool = False, lib=None):
    """O rows and lse entries of ONE head ([N, d] inputs) for query ``rows``
    (and those rows of P, [len(rows), N], with ``return_p``)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    p = np.empty((rows.size, N), dtype=np.float64) if return_p else None
    rc = lib.oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), N, d, int(bool(causal)),
                                  float(scale), rows.ctypes.data_as(_I64P), rows.size,
                                  _ptr(o), _ptr(lse), _ptr(p) if return_p else ctypes.cast(None, _DP))
    _check(rc, "attn_fwd_rows")
    return (o, lse, p) if return_p else (o, lse)


def attn_fwd_rect(q, k, v, causal: bool, scale: float, return_p: bool = False, lib=None):
    """O and lse of Nq queries ([..., Nq, d]) against Nk keys and values
    ([..., Nk, d]); the queries are the last Nq positions, so under the causal
    mask query i sees keys 0 .. i + Nk - Nq.  With ``return_p`` also P
    ([..., Nq, Nk])."""
    lib = lib or load()
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    G, Nq, d = qh.shape
    Nk = kh.shape[1]
    o = np.empty_like(qh)
    lse = np.empty((G, Nq), dtype=np.float64)
    p = np.empty((G, Nq, Nk), dtype=np.float64) if return_p else None
    for g in range(G):
        rc = lib.oracle_attn_fwd_rect(_ptr(qh[g]), _ptr(kh[g]), _ptr(vh[g]), Nq, Nk, d,
                                      int(bool(causal)), float(scale), _ptr(o[g]), _ptr(lse[g]),
                                      _ptr(p[g]) if return_p else ctypes.cast(None, _DP))
        _check(rc, "attn_fwd_rect")
    if return_p:
        return o.reshape(lead + (Nq, d)), lse.reshape(lead + (Nq,)), p.reshape(lead + (Nq, Nk))
    return o.reshape(lead + (Nq, d)), lse.reshape(lead + (Nq,))


def mx_decode(codes, scales, lib=None) -> np.ndarray:
    """Values of an MXFP8 tensor: ``codes`` uint8 E4M3 of shape [..., d],
    ``scales`` uint8 E8M0 of shape [..., d / 32] (one per 32 elements of a
    row).  Returns float64 [..., d].  Accepts numpy arrays or CPU tensors."""
    lib = lib or load()
    if hasattr(codes, "detach"):
        codes = codes.detach().to("cpu").numpy()
    if hasattr(scales, "detach"):
        scales = scales.detach().to("cpu").numpy()
    codes = np.ascontiguousarray(np.asarray(codes).view(np.uint8))
    scales = np.ascontiguousarray(np.asarray(scales).view(np.uint8))
    d = codes.shape[-1]
    if scales.shape != codes.shape[:-1] + (d // 32,):
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape}")
    out = np.empty(codes.shape, dtype=np.float64)
    rows = codes.size // d
    _check(lib.oracle_mx_decode(codes.ctypes.data, scales.ctypes.data, rows, d, _ptr(out)),
           "mx_decode")
    return out


def attn_bwd(q, k, v, dout, causal: bool, scale: float, lib=None):
    """dq, dk, dv of sum(dout * O) plus the oracle's own (o, lse, D), for
    inputs of shape [..., N, d].  Returns a dict of float64 arrays."""
    lib = lib or load()
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    doh, _ = _heads(dout)
    G, N, d = qh.shape
    out = {name: np.empty_like(qh) for name in ("dq", "dk", "dv", "o")}
    lse = np.empty((G, N), dtype=np.float64)
    D = np.empty((G, N), dtype=np.float64)
    for g in range(G):
        rc = lib.oracle_attn_bwd_head(
            _ptr(qh[g]), _ptr(kh[g]), _ptr(vh[g]), _ptr(doh[g]), N, d,
            int(bool(causal)), float(scale), _ptr(out["dq"][g]), _ptr(out["dk"][g]),
            _ptr(out["dv"][g]), _ptr(out["o"][g]), _ptr(lse[g]), _ptr(D[g]))
        _check(rc, "attn_bwd_head")
    res = {n: a.reshape(lead + (N, d)) for n, a in out.items()}
    res["lse"] = lse.reshape(lead + (N,))
    res["D"] = D.reshape(lead + (N,))
    return res


def attn_bwd_rect(q, k, v, dout, causal: bool, scale: float, lib=None):
    """dq [..., Nq, d], dk, dv [..., Nk, d] of sum(dout * O) for Nq queries
    (the last Nq positions) against Nk keys, plus the oracle's own (o, lse,
    D).  Returns a dict of float64 arrays."""
    lib = lib or load()
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    doh, _ = _heads(dout)
    G, Nq, d = qh.shape
    Nk = kh.shape[1]
    dq = np.empty_like(qh)
    o = np.empty_like(qh)
    dk = np.empty_like(kh)
    dv = np.empty_like(kh)
    lse = np.empty((G, Nq), dtype=np.float64)
    D = np.empty((G, Nq), dtype=np.float64)
    for g in range(G):
        rc = lib.oracle_attn_bwd_rect(
            _ptr(qh[g]), _ptr(kh[g]), _ptr(vh[g]), _ptr(doh[g]), Nq, Nk, d,
            int(bool(causal)), float(scale), _ptr(dq[g]), _ptr(dk[g]), _ptr(dv[g]),
            _ptr(o[g]), _ptr(lse[g]), _ptr(D[g]))
        _check(rc, "attn_bwd_rect")
    return {"dq": dq.reshape(lead + (Nq, d)), "dk": dk.reshape(lead + (Nk, d)),
            "dv": dv.reshape(lead + (Nk, d)), "o": o.reshape(lead + (Nq, d)),
            "lse": lse.reshape(lead + (Nq,)), "D": D.reshape(lead + (Nq,))}


def attn_bwd_dq_rows(q, k, v, dout, causal: bool, scale: float, rows, lib=None):
    """dQ rows of ONE head ([N, d] inputs) for query ``rows``."""
    lib = lib or load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    N, d = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    dq = np.empty((rows.size, d), dtype=np.float64)
    rc = lib.oracle_attn_bwd_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), N, d,
                                     int(bool(causal)), float(scale), rows.ctypes.data_as(_I64P),
                                     rows.size, _ptr(dq))
    _check(rc, "attn_bwd_dq_rows")
    return dq
