"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Every test here needs an MI355X and the built library.

Coverage:
* the five workloads at their real shapes (full oracle where it finishes in
  seconds, sampled query rows at the large shapes; the backward on whole heads
  of the backward workload and of the headline shape), the B4 H16 N4096 causal
  shape at d = 96, 32 and 256 (forward only at 256), and B4 H16 N4001 d128
  causal (tail tiles on both loops, forward and backward);
* ragged N (tails that span several tiles), N = 1, both masks,
  d = 32 / 64 / 96 / 128 / 256 (forward, fp32 and bf16; backward, bf16);
* closed forms with exactly representable inputs (Q = 0);
* the dV / dK sum invariants of the backward at full size;
* scales other than 1/sqrt(d) (1.0 and 0.02) on causal and unmasked ragged
  shapes, forward (bf16 and fp32) and backward;
* determinism of the forward and of the backward; the backward's phases one by one
  (attn_bwd = phase 3 then 1, bitwise; phases 0, 1, 2 within the rounding of D); lse at a
  4-byte offset;
* a long sequence (N = 65573, both masks) on sampled rows, forward and backward (dQ rows
  against the oracle's row-wise dQ, dV / dK sum invariants over every key);
* many heads (B = 6, H = 37) of a short sequence, forward and backward.
"""
import numpy as np
import pytest
import torch

import oracle
from attn_inputs import HEADDIM_WORKLOADS, WORKLOADS, make_inputs, workload_inputs
from tests.parity import (bwd_rounding_bound, compare, describe, f32_scale, gpu_backward,
                          gpu_forward, log,
                          oracle_full_fwd, oracle_rows_fwd, sample_rows, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_online_softmax_attn_amd as T
    T.lib()  # raises if libattn.so is missing: no silent fallback


def _fwd_full_check(q, k, v, causal, scale, dtype, tag):
    log(f"[fwd] {tag} shape={tuple(q.shape)} causal={causal} dtype={dtype}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    o_ref, lse_ref = oracle_full_fwd(q, k, v, causal, scale)
    eo = compare(to_np(o), o_ref, dtype, f"{tag} O")
    el = compare(to_np(lse), lse_ref, dtype, f"{tag} lse")
    log(f"    O {describe(eo)} | lse {describe(el)}")
    return o, lse


# ------------------------------------------------------------ small, full oracle
def test_single_head_f32_workload():
    w = WORKLOADS["single_head_f32"]
    q, k, v = workload_inputs(w)
    _fwd_full_check(q, k, v, w.causal, w.scale, w.dtype, w.name)


@pytest.mark.parametrize("name", ["h8_n1024_d64", "h8_n1024_d64_causal"])
def test_h8_n1024_workloads(name):
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    _fwd_full_check(q, k, v, w.causal, w.scale, w.dtype, w.name)


@pytest.mark.parametrize("N", [1, 17, 100, 255, 257, 1000])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_forward(N, d, causal, dtype):
    q, k, v = make_inputs(1, 2, N, d, dtype, seed=100 + N + d)
    _fwd_full_check(q, k, v, causal, d ** -0.5, dtype, f"ragged N={N} d={d}")


@pytest.mark.parametrize("N", [31, 32, 33, 63, 65, 129])
@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_forward_at_workgroup_edges(N, d, causal):
    """The fp32 forward gives each workgroup 32 queries (8 threads per query):
    lengths on either side of one, two and four workgroups, against the fp32
    tolerance."""
    q, k, v = make_inputs(1, 3, N, d, torch.float32, seed=300 + N + d)
    _fwd_full_check(q, k, v, causal, d ** -0.5, torch.float32, f"fp32 edge N={N} d={d}")


@pytest.mark.parametrize("N", [1, 17, 100, 257, 1000])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_backward(N, d, causal):
    q, k, v, do = make_inputs(1, 2, N, d, torch.bfloat16, seed=200 + N + d, with_dout=True)
    scale = d ** -0.5
    log(f"[bwd] ragged N={N} d={d} causal={causal}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    dq, dk, dv = gpu_backward(q, k, v, o, lse, do, causal, scale)
    ref = oracle.attn_bwd(to_np(q), to_np(k), to_np(v), to_np(do), causal, f32_scale(scale))
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        e = compare(to_np(got), ref[name], torch.bfloat16, f"ragged bwd {name}")
        log(f"    {name} {describe(e)}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads(d, causal):
    """222 heads (B*H not a multiple of the 8 XCDs the grid is dealt over) of
    33 queries: the workgroup -> (head, tile) mapping on a wide, shallow grid."""
    q, k, v, do = make_inputs(6, 37, 33, d, torch.bfloat16, seed=300 + d, with_dout=True)
    scale = d ** -0.5
    o, lse = _fwd_full_check(q, k, v, causal, scale, torch.bfloat16, f"many heads d={d}")
    dq, dk, dv = gpu_backward(q, k, v, o, lse, do, causal, scale)
    ref = oracle.attn_bwd(to_np(q), to_np(k), to_np(v), to_np(do), causal, f32_scale(scale))
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        e = compare(to_np(got), ref[name], torch.bfloat16, f"many heads bwd {name}")
        log(f"    {name} {describe(e)}")


def test_q_zero_closed_form():
    """Q = 0 gives S = 0: O is the (prefix) mean of V and lse = ln(#keys)."""
    for causal in (False, True):
        for dtype in (torch.float32, torch.bfloat16):
            _, k, v = make_inputs(1, 1, 300, 64, dtype, seed=7)
            q = torch.zeros_like(k)
            o, lse = gpu_forward(q, k, v, causal, 0.125)
            vv = to_np(v)[0, 0]
            n = np.arange(1, 301)
            want_o = (np.cumsum(vv, 0) / n[:, None]) if causal else np.tile(vv.mean(0), (300, 1))
            want_l = np.log(n) if causal else np.full(300, np.log(300))
            compare(to_np(o)[0, 0], want_o, dtype, "Q=0 O")
            compare(to_np(lse)[0, 0], want_l, dtype, "Q=0 lse")


# ------------------------------------------------------------ scales other than 1/sqrt(d)
# The contract is any finite scale > 0.  A larger scale makes the rows peaky
# (scale 1.0 at d = 128: logits of standard deviation ~11, so the lazy
# reference maximum moves within a tile), a small one flat (0.02: nearly
# uniform rows).  Causal ragged shapes put masked keys in the first tile
# and a tail in the last one.
@pytest.mark.parametrize("scale", [1.0, 0.02])
@pytest.mark.parametrize("N,d", [(100, 32), (257, 64), (255, 96), (1000, 128), (300, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_other_scales_bf16(scale, N, d, causal):
    q, k, v = make_inputs(1, 2, N, d, torch.bfloat16, seed=400 + N + d)
    _fwd_full_check(q, k, v, causal, scale, torch.bfloat16, f"scale={scale} N={N} d={d}")


# fp32: the 1e-5 bound on O and lse is kept; at scale 1.0 the logits and lse
# grow with sqrt(d) and so does their fp32 rounding, so the larger head
# dimensions are taken at the small scale only.
@pytest.mark.parametrize("scale,N,d", [(1.0, 100, 32), (1.0, 257, 64), (0.02, 255, 96),
                                       (0.02, 1000, 128), (0.02, 300, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_other_scales_f32(scale, N, d, causal):
    q, k, v = make_inputs(1, 2, N, d, torch.float32, seed=450 + N + d)
    _fwd_full_check(q, k, v, causal, scale, torch.float32, f"f32 scale={scale} N={N} d={d}")


@pytest.mark.parametrize("scale", [1.0, 0.02])
@pytest.mark.parametrize("N,d", [(100, 32), (257, 64), (255, 96), (300, 128), (130, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_other_scales(scale, N, d, causal):
    q, k, v, do = make_inputs(1, 2, N, d, torch.bfloat16, seed=500 + N + d, with_dout=True)
    log(f"[bwd] scale={scale} N={N} d={d} causal={causal}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    dq, dk, dv = gpu_backward(q, k, v, o, lse, do, causal, scale)
    ref = oracle.attn_bwd(to_np(q), to_np(k), to_np(v), to_np(do), causal, f32_scale(scale))
    # beyond 1/sqrt(d) the bf16 rounding of O, P and dS is amplified by the
    # scale: the stated tolerance plus the bound those rounding points give
    for h in range(q.shape[1]):
        bnd = bwd_rounding_bound(q[0, h], k[0, h], v[0, h], do[0, h], causal, scale)
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = compare(to_np(got[0, h]), ref[name][0, h], torch.bfloat16,
                        f"scale={scale} bwd {name} h{h}", extra=bnd[name])
            log(f"    {name} h{h} {describe(e)} (max bound {bnd[name].max():.3e})")


def test_forward_is_deterministic():
    q, k, v = make_inputs(1, 4, 777, 128, torch.bfloat16, seed=9)
    o1, l1 = gpu_forward(q, k, v, True, 128 ** -0.5)
    o2, l2 = gpu_forward(q, k, v, True, 128 ** -0.5)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_is_deterministic(d):
    """attn_bwd writes every gradient element exactly once (no atomics), so
    two calls on the same inputs and workspace agree bit for bit; d = 64 and
    128 take the two register layouts of the dK/dV kernel."""
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_inputs(2, 3, 777, d, torch.bfloat16, seed=11 + d,
                                                   with_dout=True))
    scale = d ** -0.5
    o, lse = T.flash_attention_forward(q, k, v, True, scale)
    ws = torch.empty(T.attn_bwd_workspace_bytes(2, 3, 777, d), device=dev, dtype=torch.uint8)
    outs = []
    for _ in range(2):
        g = [torch.full_like(q, float("nan")) for _ in range(3)]
        T.attn_bwd(q, k, v, o, do, lse, g[0], g[1], g[2], ws, True, scale)
        torch.cuda.synchronize()
        outs.append(g)
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("d,causal", [(64, True), (128, True), (128, False), (256, True)])
def test_backward_phases(d, causal):
    """attn_bwd is phase 3 (dQ forming D itself) then phase 1 (dK/dV): those
    two phases called one by one give its results bit for bit, and the D
    phase 3 leaves in the workspace is the D of phase 0 up to fp32 rounding
    (the same products summed in another order).  Phases 0, 1, 2 then give
    the same gradients within the rounding that difference in D makes, which
    is far below a bf16 unit."""
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    B, H, N = 1, 3, 333
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, N, d, torch.bfloat16, seed=21 + d,
                                                   with_dout=True))
    scale = d ** -0.5
    o, lse = T.flash_attention_forward(q, k, v, causal, scale)
    ws = torch.empty(T.attn_bwd_workspace_bytes(B, H, N, d), device=dev, dtype=torch.uint8)
    D = ws[: B * H * N * 4].view(torch.float32)
    nan = lambda: [torch.full_like(q, float("nan")) for _ in range(3)]
    ref = nan()
    T.attn_bwd(q, k, v, o, do, lse, ref[0], ref[1], ref[2], ws, causal, scale)
    g31 = nan()
    T.attn_bwd_phase(3, q, k, v, o, do, lse, g31[0], g31[1], g31[2], ws, causal, scale)
    torch.cuda.synchronize()
    d3 = D.clone()
    T.attn_bwd_phase(1, q, k, v, o, do, lse, g31[0], g31[1], g31[2], ws, causal, scale)
    g012 = nan()
    for ph in (0, 1, 2):
        T.attn_bwd_phase(ph, q, k, v, o, do, lse, g012[0], g012[1], g012[2], ws, causal, scale)
    torch.cuda.synchronize()
    d0 = D.clone()
    for a, b in zip(ref, g31):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    d_exact = (do.double() * o.double()).sum(-1).flatten()
    scale_d = (do.double().abs() * o.double().abs()).sum(-1).flatten()
    for dd in (d3, d0):
        # fp32 sums of d products: |error| <= d * 2^-24 * sum |dO O| (plus slack)
        assert torch.all((dd.double() - d_exact).abs() <= 2 * d * 2.0 ** -24 * scale_d + 1e-30)
    for a, b in zip(ref, g012):
        diff = (a.float() - b.float()).abs()
        ulp = a.float().abs().clamp_min(2.0 ** -60) * 2.0 ** -7
        assert torch.all(diff <= ulp + 1e-6), float(diff.max())


def test_lse_at_4_byte_offset():
    """lse is accessed one float at a time, so a view that starts 4 bytes
    into a buffer is accepted and gives the same results as an aligned one."""
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    B, H, N, d = 1, 2, 300, 64
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, N, d, torch.bfloat16, seed=77,
                                                   with_dout=True))
    o_a, lse_a = T.flash_attention_forward(q, k, v, True, 0.125)
    buf = torch.full((B * H * N + 1,), float("nan"), device=dev)
    lse_b = buf[1:].view(B, H, N)
    assert lse_b.data_ptr() % 16 == 4
    o_b = torch.empty_like(q)
    T.attn_fwd(q, k, v, o_b, lse_b, True, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(lse_a, lse_b) and torch.equal(o_a.view(torch.int16), o_b.view(torch.int16))
    g_a = T.flash_attention_backward(q, k, v, o_a, lse_a, do, True, 0.125)
    g_b = T.flash_attention_backward(q, k, v, o_b, lse_b, do, True, 0.125)
    torch.cuda.synchronize()
    for a, b in zip(g_a, g_b):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------ full-size workloads
@pytest.mark.parametrize("name,heads", [
    ("b4_h16_n4096_d128_causal", [(0, 0), (1, 7), (3, 15)]),
    ("h32_n16384_d128_causal_bigqk", [(0, 0), (0, 13), (0, 31)]),
    ("b2_h16_n4096_d64_causal_fwdbwd", [(0, 0), (1, 15)]),
    ("b4_h16_n4096_d96_causal", [(0, 0), (3, 15)]),
    ("b4_h16_n4096_d32_causal", [(0, 0), (2, 9)]),
    ("b4_h16_n4096_d256_causal", [(0, 0), (3, 12)]),
    ("b4_h16_n4001_d128_causal", [(0, 0), (3, 15)]),
])
def test_full_size_forward_sampled_rows(name, heads):
    w = {**WORKLOADS, **HEADDIM_WORKLOADS}[name]
    log(f"[fwd] {name}: generating inputs")
    q, k, v = workload_inputs(w, with_dout=False)
    o, lse = gpu_forward(q, k, v, w.causal, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in heads:
        rows = sample_rows(w.N, 48, seed=b * 100 + h)
        o_ref, l_ref = oracle_rows_fwd(q, k, v, w.causal, w.scale, b, h, rows)
        eo = compare(to_np(o[b, h])[rows], o_ref, w.dtype, f"{name} O b{b} h{h}")
        el = compare(to_np(lse[b, h])[rows], l_ref, w.dtype, f"{name} lse b{b} h{h}")
        log(f"    b{b} h{h} rows={len(rows)} O {describe(eo)} | lse {describe(el)}")


@pytest.mark.parametrize("name,heads", [
    ("b2_h16_n4096_d64_causal_fwdbwd", [(0, 0), (1, 11)]),
    ("b4_h16_n4096_d128_causal", [(3, 14)]),
    ("b4_h16_n4001_d128_causal", [(1, 6)]),
    ("b4_h16_n4096_d96_causal", [(2, 5)]),
    ("b4_h16_n4096_d32_causal", [(1, 3)]),
    ("b4_h16_n4096_d256_causal", [(2, 7)]),
])
def test_fwdbwd_workload_backward(name, heads):
    w = {**WORKLOADS, **HEADDIM_WORKLOADS}[name]
    log(f"[bwd] {w.name}: generating inputs")
    q, k, v, do = workload_inputs(w, with_dout=True)
    o, lse = gpu_forward(q, k, v, w.causal, w.scale)
    dq, dk, dv = gpu_backward(q, k, v, o, lse, do, w.causal, w.scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    # invariants on every head: sum_j dV_j = sum_i dO_i, sum_j dK_j = 0
    sdv = dv.double().sum(2)
    sdo = do.double().sum(2)
    assert torch.allclose(sdv, sdo, atol=2e-2 * w.N ** 0.5, rtol=1e-2)
    sdk = dk.double().sum(2)
    assert (sdk.abs() <= 2e-2 * w.N ** 0.5 + 1e-2 * dk.double().abs().sum(2)).all()
    # element-by-element against the oracle on whole heads
    for b, h in heads:
        log(f"    oracle backward b{b} h{h}")
        ref = oracle.attn_bwd(to_np(q[b, h]), to_np(k[b, h]), to_np(v[b, h]), to_np(do[b, h]),
                              True, f32_scale(w.scale))
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = compare(to_np(got[b, h]), ref[name], w.dtype, f"{w.name} {name} b{b} h{h}")
            log(f"    {name} b{b} h{h} {describe(e)}")


def test_binding_refuses_mismatched_tensors():
    """Every tensor must match the shape and dtype implied by Q and sit on Q's
    GPU; the binding raises before a kernel could read or write past one."""
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 2, 100, 64, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(1, 2, 100, device=dev)
    short = torch.zeros(1, 2, 99, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        T.attn_fwd(q, short, q, torch.empty_like(q), lse, True, 0.125)
    with pytest.raises(ValueError):
        T.attn_fwd(q, q, q, torch.empty_like(q), lse.double(), True, 0.125)
    with pytest.raises(ValueError):
        T.attn_fwd(q, q, q.float(), torch.empty_like(q), lse, True, 0.125)
    with pytest.raises(ValueError):
        T.attn_fwd(q, q, q, torch.empty_like(q), lse.cpu(), True, 0.125)
    ws = torch.empty(T.attn_bwd_workspace_bytes(1, 2, 100, 64), dtype=torch.uint8, device=dev)
    g = [torch.empty_like(q) for _ in range(3)]
    with pytest.raises(ValueError):
        T.attn_bwd(q, q, q, q, q, lse, g[0], short, g[2], ws, True, 0.125)
    with pytest.raises(ValueError):
        T.attn_fwd_kv(q, short, q, torch.empty_like(q), lse, False, 0.125, 0, None)


@pytest.mark.parametrize("causal", [True, False])
def test_long_sequence_forward_sampled_rows(causal):
    """N = 65573 (ragged, 513 query tiles per head): row, tile and workgroup
    indices far beyond the workload sizes; sampled rows against the oracle."""
    N, d = 65573, 128
    q, k, v = make_inputs(1, 2, N, d, torch.bfloat16, seed=21)
    scale = d ** -0.5
    log(f"[fwd] long sequence N={N} d={d} causal={causal}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for h in (0, 1):
        rows = sample_rows(N, 48, seed=31 + h)
        o_ref, l_ref = oracle_rows_fwd(q, k, v, causal, scale, 0, h, rows)
        eo = compare(to_np(o[0, h])[rows], o_ref, torch.bfloat16, f"N={N} O h{h}")
        el = compare(to_np(lse[0, h])[rows], l_ref, torch.bfloat16, f"N={N} lse h{h}")
        log(f"    h{h} O {describe(eo)} | lse {describe(el)}")


@pytest.mark.parametrize("causal", [True, False])
def test_long_sequence_backward(causal):
    """N = 65573 (ragged; 513 query tiles and 513 key blocks per head, offsets
    far beyond the workload sizes): dQ on sampled rows against the oracle's
    row-wise dQ, and the dV / dK sum invariants over every key."""
    N, d = 65573, 128
    q, k, v, do = make_inputs(1, 1, N, d, torch.bfloat16, seed=23, with_dout=True)
    scale = d ** -0.5
    log(f"[bwd] long sequence N={N} d={d} causal={causal}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    dq, dk, dv = gpu_backward(q, k, v, o, lse, do, causal, scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    sdv, sdo = dv.double().sum(2), do.double().sum(2)
    assert torch.allclose(sdv, sdo, atol=2e-2 * N ** 0.5, rtol=1e-2)
    sdk = dk.double().sum(2)
    assert (sdk.abs() <= 2e-2 * N ** 0.5 + 1e-2 * dk.double().abs().sum(2)).all()
    rows = sample_rows(N, 24, seed=41 + causal)
    ref = oracle.attn_bwd_dq_rows(to_np(q[0, 0]), to_np(k[0, 0]), to_np(v[0, 0]), to_np(do[0, 0]),
                                  causal, f32_scale(scale), rows)
    e = compare(to_np(dq[0, 0])[rows], ref, torch.bfloat16, f"N={N} dq rows")
    log(f"    dq rows={len(rows)} {describe(e)}")
