"""GPU parity of attn_fwd_mx (Q and K in MXFP8: E4M3 codes with one E8M0
scale per 32 elements along d; V bf16) and attn_fwd_fp8 (V too, transposed
with one scale per 32 keys; P rounded to E4M3) against the fp64 oracle: the
oracle decodes the FP8 tensors exactly (oracle.mx_decode) and runs its
attention definition on the decoded values.

attn_fwd_mx: S is exact up to fp32 summation on the scaled FP8 MFMA, and P
and O are rounded to bf16 as in attn_fwd, so the bf16 tolerance applies
(|gpu - oracle| <= 2e-2 + 1e-2 |oracle| on O and lse).  attn_fwd_fp8: the
same plus, on O, the bound that rounding P to E4M3 gives (fp8_pv_bound in
tests/parity.py, from the oracle's own P).

Coverage: d = 64 and 128, both masks, N from 1 to 1000 (tails inside a
tile and several tiles), block scales 2^-2..2^2, 2^-7..2^7 (large logits)
and all 2^0, softmax scales 1.0 and 0.02 besides 1/sqrt(d), the headline
shape at full size on sampled rows, bitwise determinism; for attn_fwd_fp8
NaN codes and NaN scales in the V^T padding past N, which must be ignored.
"""
import numpy as np
import pytest
import torch

import oracle
from attn_inputs import MX_WORKLOADS, make_fp8_v, make_mx_inputs
from tests.parity import (compare, decode_fp8_v, describe, f32_scale, fp8_pv_bound,
                          gpu_forward_fp8, gpu_forward_mx, log, sample_rows, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_online_softmax_attn_amd as T
    T.lib()  # raises if libattn.so is missing: no silent fallback


def _check_all(N, d, causal, seed, lo=125, hi=129, B=1, H=2, scale=None):
    q8, qs, k8, ks, v = make_mx_inputs(B, H, N, d, seed, lo, hi)
    scale = d ** -0.5 if scale is None else scale
    log(f"[mx] N={N} d={d} causal={causal} scales [{lo}, {hi}] seed={seed}")
    o, lse = gpu_forward_mx(q8, qs, k8, ks, v, causal, scale)
    q = oracle.mx_decode(q8, qs)
    k = oracle.mx_decode(k8, ks)
    o_ref, lse_ref = oracle.attn_fwd(q, k, to_np(v), causal, f32_scale(scale))
    eo = compare(to_np(o), o_ref, torch.bfloat16, f"mx O N={N} d={d}")
    el = compare(to_np(lse), lse_ref, torch.bfloat16, f"mx lse N={N} d={d}")
    log(f"    O {describe(eo)} | lse {describe(el)}")


@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 255, 257, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes(N, d, causal):
    _check_all(N, d, causal, seed=700 + N + d)


@pytest.mark.parametrize("lo,hi", [(120, 134), (127, 127)])
@pytest.mark.parametrize("d", [64, 128])
def test_scale_ranges(lo, hi, d):
    _check_all(300, d, True, seed=800 + lo + d, lo=lo, hi=hi)


@pytest.mark.parametrize("scale", [1.0, 0.02])
@pytest.mark.parametrize("N,d", [(257, 64), (1000, 128), (100, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_other_scales(scale, N, d, causal):
    """Softmax scales other than 1/sqrt(d) (peaky and nearly flat rows)."""
    _check_all(N, d, causal, seed=850 + N + d, scale=scale)


def test_workload_sampled_rows():
    w = MX_WORKLOADS["b4_h16_n4096_d128_causal_mxfp8"]
    log(f"[mx] {w.name}: generating inputs")
    q8, qs, k8, ks, v = make_mx_inputs(w.B, w.H, w.N, w.d, w.seed)
    o, lse = gpu_forward_mx(q8, qs, k8, ks, v, w.causal, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in [(0, 0), (3, 15)]:
        rows = sample_rows(w.N, 48, seed=b * 100 + h)
        q = oracle.mx_decode(q8[b, h], qs[b, h])
        k = oracle.mx_decode(k8[b, h], ks[b, h])
        o_ref, l_ref = oracle.attn_fwd_rows(q, k, to_np(v[b, h]), w.causal, f32_scale(w.scale), rows)
        eo = compare(to_np(o[b, h])[rows], o_ref, torch.bfloat16, f"{w.name} O b{b} h{h}")
        el = compare(to_np(lse[b, h])[rows], l_ref, torch.bfloat16, f"{w.name} lse b{b} h{h}")
        log(f"    b{b} h{h} O {describe(eo)} | lse {describe(el)}")


def test_deterministic():
    q8, qs, k8, ks, v = make_mx_inputs(2, 4, 1000, 128, seed=9)
    o1, l1 = gpu_forward_mx(q8, qs, k8, ks, v, True, 128 ** -0.5)
    o2, l2 = gpu_forward_mx(q8, qs, k8, ks, v, True, 128 ** -0.5)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


# ------------------------------------------------------------ attn_fwd_fp8
# Q, K and V all in MXFP8 (V transposed, blocks of 32 keys), P rounded to
# E4M3 for P V.  The oracle is the exact attention of the decoded Q, K, V;
# the GPU differs from it by the bf16 tolerance plus the bound that rounding
# P to E4M3 gives (tests.parity.fp8_pv_bound, from the oracle's own P).
def _check_fp8(N, d, causal, seed, lo=125, hi=129, vlo=125, vhi=129, B=1, H=2, scale=None):
    q8, qs, k8, ks, _ = make_mx_inputs(B, H, N, d, seed, lo, hi)
    # NaN codes and NaN block scales in the padding past N: the kernel must
    # ignore them
    vt8, vts = make_fp8_v(B, H, N, d, seed + 1, vlo, vhi, pad_code=0x7F, pad_scale=255)
    scale = d ** -0.5 if scale is None else scale
    log(f"[fp8] N={N} d={d} causal={causal} scales Q,K [{lo}, {hi}] V [{vlo}, {vhi}] "
        f"softmax scale {scale:.4g} seed={seed}")
    o, lse = gpu_forward_fp8(q8, qs, k8, ks, vt8, vts, causal, scale)
    q = oracle.mx_decode(q8, qs)
    k = oracle.mx_decode(k8, ks)
    v = decode_fp8_v(vt8, vts, N)
    o_ref, lse_ref, p = oracle.attn_fwd(q, k, v, causal, f32_scale(scale), return_p=True)
    for b in range(B):
        for h in range(H):
            bound = fp8_pv_bound(p[b, h], v[b, h])
            eo = compare(to_np(o[b, h]), o_ref[b, h], torch.bfloat16, f"fp8 O N={N} d={d} h{h}",
                         extra=bound)
            el = compare(to_np(lse[b, h]), lse_ref[b, h], torch.bfloat16, f"fp8 lse N={N} d={d}")
            log(f"    b{b} h{h} O {describe(eo)} (max bound {bound.max():.3e}) | lse {describe(el)}")


@pytest.mark.parametrize("N", [1, 17, 64, 65, 100, 129, 255, 257, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_shapes(N, d, causal):
    _check_fp8(N, d, causal, seed=900 + N + d)


@pytest.mark.parametrize("vlo,vhi", [(120, 134), (127, 127)])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_v_scale_ranges(vlo, vhi, d):
    _check_fp8(300, d, True, seed=950 + vlo + d, vlo=vlo, vhi=vhi)


@pytest.mark.parametrize("scale", [1.0, 0.02])
@pytest.mark.parametrize("N,d", [(257, 64), (1000, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_other_scales(scale, N, d, causal):
    _check_fp8(N, d, causal, seed=970 + N + d, scale=scale)


def test_fp8_workload_sampled_rows():
    """B4 H16 N4096 d128 causal at full size, sampled query rows."""
    w = MX_WORKLOADS["b4_h16_n4096_d128_causal_fp8"]
    log(f"[fp8] {w.name}: generating inputs")
    q8, qs, k8, ks, _ = make_mx_inputs(w.B, w.H, w.N, w.d, w.seed)
    vt8, vts = make_fp8_v(w.B, w.H, w.N, w.d, w.seed + 1)
    o, lse = gpu_forward_fp8(q8, qs, k8, ks, vt8, vts, w.causal, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in [(0, 0), (3, 15)]:
        rows = sample_rows(w.N, 48, seed=b * 100 + h)
        q = oracle.mx_decode(q8[b, h], qs[b, h])
        k = oracle.mx_decode(k8[b, h], ks[b, h])
        v = decode_fp8_v(vt8[b, h], vts[b, h], w.N)
        o_ref, l_ref, p = oracle.attn_fwd_rows(q, k, v, w.causal, f32_scale(w.scale), rows,
                                               return_p=True)
        bound = fp8_pv_bound(p, v)
        eo = compare(to_np(o[b, h])[rows], o_ref, torch.bfloat16, f"{w.name} O b{b} h{h}",
                     extra=bound)
        el = compare(to_np(lse[b, h])[rows], l_ref, torch.bfloat16, f"{w.name} lse b{b} h{h}")
        log(f"    b{b} h{h} O {describe(eo)} (max bound {bound.max():.3e}) | lse {describe(el)}")


def test_fp8_deterministic():
    q8, qs, k8, ks, _ = make_mx_inputs(2, 4, 1000, 128, seed=9)
    vt8, vts = make_fp8_v(2, 4, 1000, 128, seed=10)
    o1, l1 = gpu_forward_fp8(q8, qs, k8, ks, vt8, vts, True, 128 ** -0.5)
    o2, l2 = gpu_forward_fp8(q8, qs, k8, ks, vt8, vts, True, 128 ** -0.5)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
