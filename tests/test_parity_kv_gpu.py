"""GPU parity of attn_fwd_kv (Nq queries at the end of an Nk-key cache, key
range split over workgroups and merged) against the fp64 oracle's
oracle_attn_fwd_rect on the same seeded inputs.

Coverage: decode (Nq = 1) and chunked prefill shapes, key counts that are not
tile multiples, Nq = Nk, Nq > 128 (several query tiles), Nq > Nk without the
mask (one chunk and two), both masks,
d = 32, 64, 96, 128 and 256, scales 1.0 and 0.02 besides 1/sqrt(d), automatic and explicit split counts (including more splits than
tiles, which the library caps), the decode workload at full size, agreement
with attn_fwd when Nq = Nk (bit for bit with one key chunk, which runs
attn_fwd's kernel with no workspace), a 131077-key cache, and bitwise
determinism.

attn_bwd_kv (the backward of attn_fwd_kv) against oracle_attn_bwd_rect: the
same (Nq, Nk) shapes and more, d = 32 ... 256, both masks, scales 1.0 and 0.02, Nq > Nk without
the mask, Nq = Nk bit for bit against attn_bwd, and the prefill workload.
"""
import numpy as np
import pytest
import torch

import oracle
from attn_inputs import KV_WORKLOADS, kv_workload_inputs, make_kv_inputs
from tests.parity import (bwd_rounding_bound, compare, describe, f32_scale, gpu_backward,
                          gpu_forward, gpu_forward_kv, log, to_np)

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


@pytest.mark.parametrize("Nq,Nk", [(300, 100), (129, 64), (1000, 129)])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("splits", [0, 2])
def test_more_queries_than_keys(Nq, Nk, d, splits):
    """Without the mask Nq may exceed Nk: every query sees all keys.  The
    automatic plan is one chunk here (the forward kernel alone); two chunks
    take the partial results and the merge (capped at one for Nk = 64)."""
    q, k, v = make_kv_inputs(1, 2, Nq, Nk, d, seed=270 + Nq + Nk + d)
    _check(q, k, v, False, splits, f"Nq={Nq} > Nk={Nk} d={d}")


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


@pytest.mark.parametrize("d", [64, 128])
def test_square_matches_attn_fwd(d):
    """Nq = Nk: the same attention as attn_fwd.  One chunk (the automatic
    plan here: 5 key tiles) runs attn_fwd's kernel, bit for bit; three
    chunks run the partial-result kernel and the merge."""
    q, k, v = make_kv_inputs(1, 4, 257, 257, d, seed=402)
    for causal in (False, True):
        o_f, l_f = gpu_forward(q, k, v, causal, d ** -0.5)
        o1, l1 = _check(q, k, v, causal, 0, f"square d={d} causal={causal} one chunk")
        assert torch.equal(o1, o_f) and torch.equal(l1, l_f)
        o3, l3 = _check(q, k, v, causal, 3, f"square d={d} causal={causal} 3 chunks")
        assert float((o3.float() - o_f.float()).abs().max()) < 2e-2
        assert float((l3 - l_f).abs().max()) < 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_one_chunk_plan_without_workspace(causal):
    """B2 H16 N4096 d64 has 1024 query tiles, so the automatic plan is one
    chunk: no workspace (None is passed), no merge, and attn_fwd's results
    bit for bit; heads 0 and last also against the oracle."""
    import tiled_online_softmax_attn_amd as T
    B, H, N, d = 2, 16, 4096, 64
    assert T.attn_fwd_kv_workspace_bytes(B, H, N, N, d, 0) == 0
    q, k, v = make_kv_inputs(B, H, N, N, d, seed=404)
    log(f"[kv] one-chunk plan B{B} H{H} N{N} d{d} causal={causal}, no workspace")
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=dev, dtype=torch.float32)
    T.attn_fwd_kv(qd, kd, vd, o, lse, causal, d ** -0.5, 0, None)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    o_f, l_f = gpu_forward(q, k, v, causal, d ** -0.5)
    assert torch.equal(o, o_f) and torch.equal(lse, l_f)
    for b, h in [(0, 0), (B - 1, H - 1)]:
        o_ref, lse_ref = oracle.attn_fwd_rect(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                              v[b, h].double().numpy(), causal,
                                              f32_scale(d ** -0.5))
        compare(to_np(o[b, h]), o_ref, torch.bfloat16, f"one chunk O[{b},{h}]")
        compare(to_np(lse[b, h]), lse_ref, torch.bfloat16, f"one chunk lse[{b},{h}]")


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


# ------------------------------------------------------------ attn_bwd_kv
def gpu_backward_kv(q, k, v, o, lse, dout, causal, scale):
    """CPU tensors in; attn_bwd_kv on the GPU into NaN-poisoned outputs with a
    poisoned workspace; returns CPU dq, dk, dv."""
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    qd, kd, vd, od, dod, ld = (t.to(dev) for t in (q, k, v, o, dout, lse))
    ws = torch.full((T.attn_bwd_kv_workspace_bytes(B, H, Nq, Nk, d),), 0xFF, device=dev,
                    dtype=torch.uint8)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    T.attn_bwd_kv(qd, kd, vd, od, dod, ld, dq, dk, dv, ws, causal, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _dout(B, H, Nq, d, seed):
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)


def _check_bwd(q, k, v, causal, tag, seed, scale=None):
    d = q.shape[-1]
    default = scale is None
    scale = d ** -0.5 if default else scale
    do = _dout(*q.shape, seed)
    log(f"[bwd_kv] {tag} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} scale={scale:.4g}")
    o, lse = gpu_forward_kv(q, k, v, causal, scale, 0)
    dq, dk, dv = gpu_backward_kv(q, k, v, o, lse, do, causal, scale)
    ref = oracle.attn_bwd_rect(to_np(q), to_np(k), to_np(v), to_np(do), causal, f32_scale(scale))
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            # at scales other than 1/sqrt(d) the stated tolerance plus the
            # bound the bf16 rounding points of the backward give
            bnd = None if default else bwd_rounding_bound(q[b, h], k[b, h], v[b, h], do[b, h],
                                                          causal, scale)
            for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
                e = compare(to_np(got[b, h]), ref[name][b, h], torch.bfloat16, f"{tag} {name} h{h}",
                            extra=None if bnd is None else bnd[name])
                log(f"    {name} h{h} {describe(e)}")


@pytest.mark.parametrize("Nq,Nk", [(7, 100), (64, 64), (128, 1000), (200, 333), (130, 2049),
                                   (1, 65), (33, 4097), (300, 300)])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_shapes(Nq, Nk, d, causal):
    """Backward of Nq queries at the end of Nk keys against the oracle's
    rectangular gradient: query tiles that straddle the shifted diagonal,
    ragged tails on both sides, a single query."""
    q, k, v = make_kv_inputs(1, 2, Nq, Nk, d, seed=600 + Nq + Nk + d)
    _check_bwd(q, k, v, causal, f"Nq={Nq} Nk={Nk} d={d}", seed=610 + Nq + d)


@pytest.mark.parametrize("scale", [1.0, 0.02])
@pytest.mark.parametrize("Nq,Nk,d", [(7, 100, 64), (130, 2049, 128), (200, 333, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_other_scales(scale, Nq, Nk, d, causal):
    q, k, v = make_kv_inputs(1, 2, Nq, Nk, d, seed=640 + Nq + d)
    _check_bwd(q, k, v, causal, f"scale={scale} Nq={Nq} Nk={Nk} d={d}", seed=645 + Nq,
               scale=scale)


@pytest.mark.parametrize("Nq,Nk", [(300, 100), (129, 64)])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_more_queries_than_keys(Nq, Nk, d):
    """Without the mask Nq may exceed Nk."""
    q, k, v = make_kv_inputs(1, 2, Nq, Nk, d, seed=650 + Nq + d)
    _check_bwd(q, k, v, False, f"Nq={Nq} > Nk={Nk} d={d}", seed=660 + Nq + d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_square_equals_attn_bwd(causal, d):
    """Nq = Nk runs the kernels of attn_bwd with the same offsets: bit for
    bit the same gradients."""
    q, k, v = make_kv_inputs(2, 3, 517, 517, d, seed=670 + d)
    do = _dout(2, 3, 517, d, 671 + d)
    scale = d ** -0.5
    o, lse = gpu_forward(q, k, v, causal, scale)
    a = gpu_backward(q, k, v, o, lse, do, causal, scale)
    b = gpu_backward_kv(q, k, v, o, lse, do, causal, scale)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("Nq,Nk,d", [(130, 2049, 128), (128, 1000, 64), (33, 4097, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_split_dq_deterministic(Nq, Nk, d, causal):
    """Shapes whose dQ is split over the keys (the workspace holds the fp32
    partials): two calls give the same bits, and dQ matches the oracle."""
    from tiled_online_softmax_attn_amd import attn_bwd_kv_workspace_bytes
    B, H = 1, 2
    ws = attn_bwd_kv_workspace_bytes(B, H, Nq, Nk, d)
    assert ws > B * H * Nq * 4 + 256, "this shape is meant to split dQ"
    q, k, v = make_kv_inputs(B, H, Nq, Nk, d, seed=680 + Nq + d)
    do = _dout(B, H, Nq, d, 685 + Nq + d)
    scale = d ** -0.5
    log(f"[bwd_kv] split dQ Nq={Nq} Nk={Nk} d={d} causal={causal} workspace={ws}")
    o, lse = gpu_forward_kv(q, k, v, causal, scale, 0)
    a = gpu_backward_kv(q, k, v, o, lse, do, causal, scale)
    b = gpu_backward_kv(q, k, v, o, lse, do, causal, scale)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    ref = oracle.attn_bwd_rect(to_np(q), to_np(k), to_np(v), to_np(do), causal, f32_scale(scale))
    for h in range(H):
        e = compare(to_np(a[0][0, h]), ref["dq"][0, h], torch.bfloat16, f"split dq h{h}")
        log(f"    dq h{h} {describe(e)}")


def test_backward_prefill_workload():
    """The prefill workload (B2 H16 Nq512 Nk4096 d128 causal): the sum
    invariants on every head, the oracle on two whole heads."""
    w = KV_WORKLOADS["prefill_b2_h16_nq512_nk4096_d128"]
    q, k, v = kv_workload_inputs(w)
    do = _dout(w.B, w.H, w.Nq, w.d, 690)
    log(f"[bwd_kv] {w.name}")
    o, lse = gpu_forward_kv(q, k, v, w.causal, w.scale, 0)
    dq, dk, dv = gpu_backward_kv(q, k, v, o, lse, do, w.causal, w.scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    sdv, sdo = dv.double().sum(2), do.double().sum(2)
    assert torch.allclose(sdv, sdo, atol=2e-2 * w.Nk ** 0.5, rtol=1e-2)
    sdk = dk.double().sum(2)
    assert (sdk.abs() <= 2e-2 * w.Nk ** 0.5 + 1e-2 * dk.double().abs().sum(2)).all()
    for b, h in [(0, 0), (1, 13)]:
        ref = oracle.attn_bwd_rect(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(do[b, h]),
                                   w.causal, f32_scale(w.scale))
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = compare(to_np(got[b, h]), ref[name], torch.bfloat16, f"{w.name} {name} b{b} h{h}")
            log(f"    {name} b{b} h{h} {describe(e)}")
