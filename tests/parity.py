"""Shared helpers for the GPU parity tests: run the HIP path through the C
ABI, run the fp64 oracle on the same seeded inputs, compare.

Tolerances (stated by the benchmark spec for this path):
* fp32 inputs: max |gpu - oracle| <= 1e-5 on O and lse;
* bf16 inputs: elementwise |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| on O, lse,
  dQ, dK and dV (absolute 2e-2 plus relative 1e-2, the allclose reading).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import tiled_online_softmax_attn_amd as T

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def f32_scale(scale: float) -> float:
    """The scale the kernels receive (a float32), widened for the oracle."""
    return float(np.float32(scale))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def compare(gpu, ref, dtype: torch.dtype, what: str, extra=None) -> dict:
    """Assert the stated tolerance (plus an elementwise rounding bound
    ``extra`` where one is derived for the case); return the error summary."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(ref), 1e-6)).max()) if err.size else 0.0
    if dtype == torch.float32:
        assert max_abs <= F32_ATOL, f"{what}: max abs err {max_abs:.3e} > {F32_ATOL}"
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
        if extra is not None:
            bound = bound + np.asarray(extra, dtype=np.float64)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} elements outside "
                               f"2e-2 + 1e-2|ref| (max abs {max_abs:.3e})")
    return {"max_abs": max_abs, "max_rel": max_rel}


BF16_U = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits, round to nearest)


def bwd_rounding_bound(q, k, v, dout, causal, scale) -> dict:
    """Elementwise bound on what the bf16 rounding points of the backward add
    to dQ, dK and dV, from the oracle's fp64 P (one head, [N, d] inputs, or
    q, dout [Nq, d] at the end of k, v [Nk, d]).

    The kernels round four quantities to bf16 (u = 2^-8 relative each): O
    in the forward, which also carries the rounding of P before P V, so
    D_i = sum_k dO_ik O_ik is off by at most
        dD_i = 2u sum_k |dO_ik| (P |V|)_ik;
    dS = P (dP - D) before dQ and dK; and P before dV.  With everything else
    in fp32,
        |ddQ| <= scale (dD (P |K|) + u |dS| |K|)
        |ddK| <= scale (P^T (dD |Q|) + u |dS|^T |Q|)
        |ddV| <= u P^T |dO|.
    At scale 1/sqrt(d) this stays inside the stated 2e-2 + 1e-2 |ref|; it
    grows with the scale (scale 1.0 makes the logits sqrt(d) times larger)."""
    Q, K, V, dO = (np.asarray(to_np(t) if hasattr(t, "detach") else t, dtype=np.float64)
                   for t in (q, k, v, dout))
    sc = f32_scale(scale)
    if Q.shape[0] == K.shape[0]:
        _, _, P = oracle.attn_fwd(Q, K, V, causal, sc, return_p=True)
    else:  # Nq queries at the end of Nk keys
        _, _, P = oracle.attn_fwd_rect(Q, K, V, causal, sc, return_p=True)
    O = P @ V
    dS = P * (dO @ V.T - (dO * O).sum(1)[:, None])
    u = BF16_U
    dD = 2 * u * (np.abs(dO) * (P @ np.abs(V))).sum(1)
    return {"dq": sc * (dD[:, None] * (P @ np.abs(K)) + u * np.abs(dS) @ np.abs(K)),
            "dk": sc * (P.T @ (dD[:, None] * np.abs(Q)) + u * np.abs(dS).T @ np.abs(Q)),
            "dv": u * P.T @ np.abs(dO)}


def gpu_forward(q, k, v, causal, scale):
    """q, k, v: CPU tensors [B,H,N,d]. Returns CPU (o, lse)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=dev, dtype=torch.float32)
    T.attn_fwd(qd, kd, vd, o, lse, causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_backward(q, k, v, o, lse, dout, causal, scale):
    """All CPU tensors in; runs attn_bwd on the GPU; returns CPU dq, dk, dv."""
    dev = torch.device("cuda:0")
    B, H, N, d = q.shape
    args = [t.to(dev) for t in (q, k, v, o, dout)]
    lse_d = lse.to(dev)
    ws = torch.full((T.attn_bwd_workspace_bytes(B, H, N, d),), 0xFF, device=dev, dtype=torch.uint8)
    dq, dk, dv = (torch.full_like(args[0], float("nan")) for _ in range(3))
    T.attn_bwd(args[0], args[1], args[2], args[3], args[4], lse_d, dq, dk, dv, ws, causal, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def sample_rows(N: int, n_random: int, seed: int) -> np.ndarray:
    """Query rows to check at full size: both ends, tile edges, random."""
    fixed = {0, 1, 2, N - 1, N - 2, N // 2}
    for t in (63, 64, 65, 127, 128, 129, 255, 256):
        if t < N:
            fixed.add(t)
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, N, size=n_random)
    return np.array(sorted(fixed | set(int(x) for x in rnd)), dtype=np.int64)


def oracle_full_fwd(q, k, v, causal, scale):
    return oracle.attn_fwd(to_np(q), to_np(k), to_np(v), causal, f32_scale(scale))


def oracle_rows_fwd(q, k, v, causal, scale, b, h, rows):
    return oracle.attn_fwd_rows(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), causal,
                                f32_scale(scale), rows)


def describe(err: dict) -> str:
    return f"max_abs={err['max_abs']:.3e} max_rel={err['max_rel']:.3e}"


__all__ = ["compare", "bwd_rounding_bound", "fp8_pv_bound", "gpu_forward_fp8", "decode_fp8_v", "gpu_forward", "gpu_backward", "sample_rows", "oracle_full_fwd",
           "oracle_rows_fwd", "to_np", "f32_scale", "log", "describe", "math"]


def gpu_forward_kv(q, k, v, causal, scale, num_splits=0):
    """q [B,H,Nq,d], k, v [B,H,Nk,d] CPU tensors; runs attn_fwd_kv on the GPU
    with a poisoned workspace; returns CPU (o, lse)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device=dev, dtype=torch.float32)
    ws = torch.full((T.attn_fwd_kv_workspace_bytes(B, H, Nq, Nk, d, num_splits),), 0xFF,
                    device=dev, dtype=torch.uint8)
    T.attn_fwd_kv(qd, kd, vd, o, lse, causal, scale, num_splits, ws)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_softmax(x, inplace=False):
    """x [M, N] CPU tensor; runs attn_softmax_rows on the GPU (into a
    NaN-poisoned output, or in place); returns the CPU result."""
    xd = x.to(torch.device("cuda:0"))
    if inplace:
        y = xd
    else:
        y = torch.full_like(xd, float("nan"))
    T.attn_softmax_rows(xd, y)
    torch.cuda.synchronize()
    return y.cpu()


def oracle_softmax_rows(x: np.ndarray, rows=None) -> np.ndarray:
    """fp64 oracle softmax of the given rows of x [M, N] (all by default)."""
    rows = range(x.shape[0]) if rows is None else rows
    return np.stack([oracle.softmax_row(np.ascontiguousarray(x[r], dtype=np.float64))[0]
                     for r in rows])


def gpu_forward_mx(q8, qs, k8, ks, v, causal, scale):
    """MXFP8 inputs (CPU tensors); runs attn_fwd_mx into NaN-poisoned outputs;
    returns CPU (o, lse)."""
    dev = torch.device("cuda:0")
    q8d, qsd, k8d, ksd, vd = (t.to(dev) for t in (q8, qs, k8, ks, v))
    B, H, N, d = q8.shape
    o = torch.full((B, H, N, d), float("nan"), device=dev, dtype=torch.bfloat16)
    lse = torch.full((B, H, N), float("nan"), device=dev, dtype=torch.float32)
    T.attn_fwd_mx(q8d, qsd, k8d, ksd, vd, o, lse, causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_forward_fp8(q8, qs, k8, ks, vt8, vts, causal, scale):
    """FP8 inputs (CPU tensors; V transposed, attn_fwd_fp8's layout); runs
    attn_fwd_fp8 into NaN-poisoned outputs; returns CPU (o, lse)."""
    dev = torch.device("cuda:0")
    ts = [t.to(dev) for t in (q8, qs, k8, ks, vt8, vts)]
    B, H, N, d = q8.shape
    o = torch.full((B, H, N, d), float("nan"), device=dev, dtype=torch.bfloat16)
    lse = torch.full((B, H, N), float("nan"), device=dev, dtype=torch.float32)
    T.attn_fwd_fp8(*ts, o, lse, causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def decode_fp8_v(vt8, vts, N):
    """V [..., N, d] (float64) of attn_fwd_fp8's V^T codes [..., d, ldv] and
    scales [..., d, ldv / 32], decoded by the oracle (keys past N dropped)."""
    vt = oracle.mx_decode(vt8, vts)
    return np.ascontiguousarray(np.swapaxes(vt[..., :N], -1, -2))


E4M3_U = 2.0 ** -4      # relative rounding error of a normal E4M3 value (3 mantissa bits)
E4M3_SUB = 2.0 ** -10   # absolute rounding error below the normal range (half of 2^-9)


def fp8_pv_bound(p: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Elementwise bound on what rounding P to E4M3 adds to O = P V, for one
    head: p [rows, N] the oracle's probabilities, v [N, d].

    The kernel rounds P_hat = 2^(s - m_ref) to nearest even, with m_ref a
    running reference within 8 (log2) of the row maximum, so P_hat <= 2^8
    and the row's largest P_hat is >= 1.  A code's error is at most
    2^-4 P_hat (normal) or 2^-10 (subnormal, or flushed to 0).  Divided by
    the row sum l_hat = P_hat_max / p_max >= 1 / p_max:
        |dO_ic| <= sum_j max(2^-4 p_ij, 2^-10 p_i,max) |V_jc|."""
    pmax = p.max(axis=1, keepdims=True)
    return np.maximum(E4M3_U * p, E4M3_SUB * pmax) @ np.abs(v)
