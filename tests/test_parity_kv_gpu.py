"""GPU parity of attn_fwd_kv (Nq queries at the end of an Nk-key cache, key
range split over workgroups and merged) against the fp64 oracle's
oracle_attn_fwd_rect on the same seeded inputs.

Coverage: decode (Nq = 1) and chunked prefill shapes, key counts that are not
tile multiples, Nq = Nk, Nq > 128 (several query tiles), both masks,
d = 32, 64, 96, 128 and 256, scales 1.0 and 0.02 besides 1/sqrt(d), automatic and explicit split counts (including more splits than
tiles, which the library caps), the decode workload at full size, agreement
with attn_fwd when Nq = Nk, a 131077-key cache, and bitwise determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from attn_inputs import KV_WORKLOADS, kv_workload_inputs, make_kv_inputs
from tests.parity import compare, describe, f32_scale, gpu_forward, gpu_forward_kv, log, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_online_softmax_attn_amd as T
    T.lib()  # raises if libattn.so is missing: no silent fallback


def _check(q, k, v, causal, splits, tag, scale=None):
    d = q.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    log(f"[kv] {tag} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} splits={splits}")
    o, lse = gpu_forward_kv(q, k, v, causal, scale, splits)
    o_ref, lse_ref = oracle.attn_fwd_rect(q.double().numpy(), k.double().numpy(),
                                          v.double().numpy(), causal, f32_scale(scale))
    eo = compare(to_np(o), o_ref, torch.bfloat16, f"{tag} O")
    el = compare(to_np(lse), lse_ref, torch.bfloat16, f"{tag} lse")
    log(f"    O {describe(eo)} | lse {describe(el)}")
    return o, lse


@pytest.mark.parametrize("Nk", [1, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_shapes(Nk, d, causal):
    q, k, v = make_kv_inputs(2, 3, 1, Nk, d, seed=100 + Nk + d)
    _check(q, k, v, causal, 0, f"decode Nk={Nk} d={d}")


@pytest.mark.parametrize("Nq,Nk", [(7, 100), (64, 64), (128, 1000), (200, 333), (130, 2049),
                                   (300, 300)])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_shapes(Nq, Nk, d, causal):
    q, k, v = make_kv_inputs(1, 2, Nq, Nk, d, seed=200 + Nq + Nk + d)
    _check(q, k, v, causal, 0, f"prefill Nq={Nq} Nk={Nk} d={d}")


@pytest.mark.parametrize("scale", [1.0, 0.02])
@pytest.mark.parametrize("Nq,Nk,d", [(1, 1000, 128), (7, 100, 64), (200, 333, 96),
                                     (130, 2049, 128), (1, 4097, 256), (100, 300, 32)])
@pytest.mark.parametrize("causal", [True, False])
def test_other_scales(scale, Nq, Nk, d, causal):
    """Scales other than 1/sqrt(d): peaky (1.0) and nearly flat (0.02) rows,
    with the shifted causal mask and ragged key counts."""
    q, k, v = make_kv_inputs(1, 2, Nq, Nk, d, seed=250 + Nq + Nk + d)
    _check(q, k, v, causal, 0, f"scale={scale} Nq={Nq} Nk={Nk} d={d}", scale=scale)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
def test_explicit_splits(splits):
    q, k, v = make_kv_inputs(1, 4, 33, 777, 128, seed=300 + splits)
    _check(q, k, v, True, splits, f"splits={splits}")


def test_split_count_changes_rounding_only():
    q, k, v = make_kv_inputs(1, 2, 5, 3000, 128, seed=401)
    o1, l1 = gpu_forward_kv(q, k, v, True, 128 ** -0.5, 1)
    o9, l9 = gpu_forward_kv(q, k, v, True, 128 ** -0.5, 9)
    assert float((o1.float() - o9.float()).abs().max()) < 2e-2
    assert float((l1 - l9).abs().max()) < 1e-4


def test_square_matches_attn_fwd():
    """Nq = Nk: the same attention as attn_fwd, by a different kernel."""
    q, k, v = make_kv_inputs(1, 4, 257, 257, 128, seed=402)
    for causal in (False, True):
        o_kv, l_kv = _check(q, k, v, causal, 0, f"square causal={causal}")
        o_f, l_f = gpu_forward(q, k, v, causal, 128 ** -0.5)
        assert float((o_kv.float() - o_f.float()).abs().max()) < 2e-2
        assert float((l_kv - l_f).abs().max()) < 1e-3


def test_decode_workload_full():
    w = KV_WORKLOADS["decode_b8_h32_nq1_nk8192_d128"]
    q, k, v = kv_workload_inputs(w)
    _check(q, k, v, w.causal, 0, w.name)


def test_prefill_workload_sampled_heads():
    w = KV_WORKLOADS["prefill_b2_h16_nq512_nk4096_d128"]
    q, k, v = kv_workload_inputs(w)
    log(f"[kv] {w.name} (heads 0 and last against the oracle)")
    o, lse = gpu_forward_kv(q, k, v, w.causal, w.scale, 0)
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        o_ref, lse_ref = oracle.attn_fwd_rect(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                              v[b, h].double().numpy(), w.causal,
                                              f32_scale(w.scale))
        compare(to_np(o[b, h]), o_ref, torch.bfloat16, f"{w.name} O[{b},{h}]")
        compare(to_np(lse[b, h]), lse_ref, torch.bfloat16, f"{w.name} lse[{b},{h}]")


def test_deterministic():
    q, k, v = make_kv_inputs(2, 2, 3, 5000, 128, seed=403)
    o1, l1 = gpu_forward_kv(q, k, v, True, 128 ** -0.5, 0)
    o2, l2 = gpu_forward_kv(q, k, v, True, 128 ** -0.5, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_long_cache(causal):
    """One query against a 131077-key cache (2049 key tiles, many splits)."""
    q, k, v = make_kv_inputs(1, 2, 1, 131077, 128, seed=41)
    _check(q, k, v, causal, 0, "decode Nk=131077 d=128")
