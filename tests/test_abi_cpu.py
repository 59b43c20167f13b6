"""The C-ABI library loads and exports every entry point include/attn.h
declares; host-side argument validation (no GPU work is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


PROBE_HEADER = os.path.join(ROOT, "include", "attn_probe.h")
PROBE_LIB = os.path.join(ROOT, "tiled_online_softmax_attn_amd", "libattn_probe.so")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\**\s+\**(attn_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_every_header_is_covered():
    """include/ holds the two C ABIs checked below and nothing else."""
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["attn.h", "attn_probe.h"]


def test_probe_library_exports_every_declared_symbol():
    names = declared_functions(PROBE_HEADER)
    assert names == ["attn_probe_copy", "attn_probe_exp", "attn_probe_mfma"]
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libattn_probe.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(PROBE_LIB)
    for name in names:
        assert hasattr(lib, name), f"libattn_probe.so does not export {name}"
    # argument checks return before any launch
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_mfma.argtypes = [vp, vp, i, i, i, vp]
    lib.attn_probe_copy.argtypes = [vp, vp, ctypes.c_longlong, vp]
    assert lib.attn_probe_mfma(None, None, 1, 1, 0, None) != 0
    assert lib.attn_probe_mfma(FAKE, FAKE, 1, 1, 3, None) != 0
    assert lib.attn_probe_copy(FAKE, FAKE, 24, None) != 0


def _lib():
    import tiled_online_softmax_attn_amd as T
    try:
        return T.lib()
    except T.AttnLibraryMissing:
        pytest.skip("libattn.so not built (run __graft_entry__.build())")


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(["attn_fwd", "attn_bwd", "attn_bwd_noalloc",
                                           "attn_bwd_phase",
                                           "attn_bwd_workspace_bytes", "attn_fwd_kv",
                                           "attn_fwd_kv_workspace_bytes", "attn_bwd_kv",
                                           "attn_bwd_kv_workspace_bytes", "attn_softmax_rows", "attn_fwd_mx",
                                           "attn_fwd_fp8",
                                           "attn_status_str", "attn_abi_version"])


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libattn.so does not export {name}"
    import tiled_online_softmax_attn_amd as T
    assert set(T.EXPORTS) == set(declared_functions())


def test_status_strings_and_version():
    lib = _lib()
    assert lib.attn_abi_version() == 9
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, 12345]:
        s = lib.attn_status_str(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_workspace_size():
    lib = _lib()
    B, H, N, d = 2, 16, 4096, 64
    n = lib.attn_bwd_workspace_bytes(B, H, N, d, 1)
    need = B * H * N * 4
    assert need <= n <= need + 256
    assert lib.attn_bwd_workspace_bytes(0, 1, 1, 64, 1) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, 1, 80, 1) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, 1, 256, 1) == 256  # d = 256 has a backward
    assert lib.attn_bwd_workspace_bytes(1, 1, 1, 512, 1) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, 1, 64, 0) == 0  # fp32 backward unsupported


# Validation returns before anything touches the GPU, so these run anywhere.
FAKE = 1 << 20  # a 16-byte aligned non-null address, never dereferenced on error paths


@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1), (dict(lse=0), -1),
    (dict(B=0), -2), (dict(H=-1), -2), (dict(N=0), -2),
    (dict(d=80), -4), (dict(d=16), -4), (dict(d=512), -4), (dict(d=0), -4),
    (dict(dtype=7), -3),
    (dict(q=FAKE + 8), -5), (dict(o=FAKE + 2), -5), (dict(lse=FAKE + 2), -5),
    (dict(scale=float("inf")), -6), (dict(scale=float("nan")), -6),
    # the scale must be > 0: zero, negative zero and negative scales are refused
    (dict(scale=0.0), -6), (dict(scale=-0.0), -6), (dict(scale=-0.125), -6),
    (dict(scale=-1e-30), -6),
    # lse needs 4-byte alignment only: this call passes the alignment check and
    # stops at the (later) scale check, so nothing is launched
    (dict(lse=FAKE + 4, scale=0.0), -6),
    # one workgroup per 32 query rows must fit a 32-bit grid: 2^16 heads of
    # 2^20 rows need 2^31 workgroups (refused), 2^20 - 32 rows 2^31 - 2^16
    (dict(H=1 << 16, N=1 << 20), -2),
    (dict(H=1 << 16, N=(1 << 20) - 32, scale=0.0), -6),
])
def test_fwd_validation(args, code):
    lib = _lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, causal=0,
             scale=0.125, dtype=1, stream=None)
    a.update(args)
    rc = lib.attn_fwd(a["q"] or None, a["k"], a["v"], a["o"], a["lse"] or None, a["B"], a["H"],
                      a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(dout=0), -1), (dict(dtype=0), -3), (dict(N=0), -2), (dict(d=80), -4), (dict(d=512), -4),
    (dict(d=256, scale=0.0), -6),
    (dict(ws=0), -7), (dict(ws_bytes=16), -7), (dict(dk=FAKE + 4), -5),
    (dict(lse=FAKE + 2), -5),
    (dict(scale=float("-inf")), -6), (dict(scale=0.0), -6), (dict(scale=-0.0), -6),
    (dict(scale=-0.5), -6), (dict(lse=FAKE + 4, scale=-0.0), -6),
])
def test_bwd_validation(args, code):
    lib = _lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             ws=FAKE, ws_bytes=1 << 30, B=1, H=1, N=16, d=64, causal=1, scale=0.125, dtype=1)
    a.update(args)
    rc = lib.attn_bwd(*(a[n] or None for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk",
                                               "dv", "ws")),
                      a["ws_bytes"], a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"],
                      a["dtype"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(dout=0), -1), (dict(lse=0), -1), (dict(dtype=0), -3), (dict(N=0), -2),
    (dict(d=80), -4), (dict(d=512), -4), (dict(d=256, scale=0.0), -6), (dict(dk=FAKE + 4), -5),
    (dict(lse=FAKE + 2), -5),
    (dict(scale=0.0), -6), (dict(scale=float("nan")), -6),
    # above the 16 MiB static scratch (4194304 query rows), refused before any
    # device call
    (dict(B=1, H=5, N=838861), -9), (dict(B=64, H=64, N=1025), -9),
])
def test_bwd_noalloc_validation(args, code):
    lib = _lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=1, H=1, N=16, d=64, causal=1, scale=0.125, dtype=1)
    a.update(args)
    rc = lib.attn_bwd_noalloc(*(a[n] or None for n in ("q", "k", "v", "o", "dout", "lse", "dq",
                                                       "dk", "dv")),
                              a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"],
                              None)
    assert rc == code


def test_bwd_phase_validation():
    lib = _lib()
    args = [FAKE] * 10 + [1 << 30, 1, 1, 16, 64, 1, 0.125, 1, None]
    assert lib.attn_bwd_phase(4, *args) == -2
    assert lib.attn_bwd_phase(-1, *args) == -2
    bad = list(args)
    bad[9] = None  # workspace
    assert lib.attn_bwd_phase(1, *bad) == -7


def test_kv_workspace_size():
    """Partial O (d floats) and lse (one float) per split, head and query,
    each part rounded up to 256 bytes, when there are two or more chunks;
    none for one chunk.  The automatic split count depends only on the
    shape: about 512 workgroups in all, at least four key tiles a chunk."""
    lib = _lib()
    r256 = lambda x: (x + 255) // 256 * 256
    for B, H, Nq, Nk, d, splits in ((1, 1, 1, 100, 64, 1), (1, 1, 1, 100, 64, 2),
                                    (2, 3, 7, 1000, 128, 5), (1, 1, 5, 64, 32, 9)):
        n = lib.attn_fwd_kv_workspace_bytes(B, H, Nq, Nk, d, splits, 1)
        tiles = (Nk + 63) // 64
        per = -(-tiles // min(splits, tiles))
        eff = -(-tiles // per)
        rows = eff * B * H * Nq
        assert n == (r256(rows * d * 4) + r256(rows * 4) if eff > 1 else 0), (Nk, splits)
    # automatic plans: decode B8 H32 against 8192 keys (256 query tiles) takes
    # 2 chunks; 300 keys (5 tiles) or 1024 query tiles (B2 H16 N4096) take one
    for B, H, Nq, Nk, d, eff in ((8, 32, 1, 8192, 128, 2), (1, 2, 300, 300, 64, 1),
                                 (2, 16, 4096, 4096, 64, 1), (1, 1, 1, 8192, 128, 32)):
        n = lib.attn_fwd_kv_workspace_bytes(B, H, Nq, Nk, d, 0, 1)
        rows = eff * B * H * Nq
        assert n == (r256(rows * d * 4) + r256(rows * 4) if eff > 1 else 0), (B, H, Nq, Nk)
    assert lib.attn_fwd_kv_workspace_bytes(1, 1, 0, 10, 64, 0, 1) == 0
    assert lib.attn_fwd_kv_workspace_bytes(1, 1, 4, 10, 80, 0, 1) == 0
    assert lib.attn_fwd_kv_workspace_bytes(1, 1, 4, 10, 64, -1, 1) == 0
    assert lib.attn_fwd_kv_workspace_bytes(1, 1, 4, 10, 64, 0, 0) == 0  # fp32 unsupported


@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1), (dict(lse=0), -1),
    (dict(B=0), -2), (dict(Nq=0), -2), (dict(Nk=0), -2), (dict(splits=-1), -2),
    (dict(Nq=20, Nk=10, causal=1), -2),
    (dict(d=48), -4), (dict(dtype=0), -3), (dict(dtype=5), -3),
    (dict(k=FAKE + 4), -5), (dict(lse=FAKE + 1), -5), (dict(scale=float("nan")), -6),
    (dict(scale=0.0), -6), (dict(scale=-0.0), -6), (dict(scale=-2.0), -6),
    (dict(lse=FAKE + 4, scale=0.0), -6),
    (dict(ws=0, splits=2), -7), (dict(ws_bytes=8, splits=2), -7),
    (dict(ws=FAKE + 8, splits=2), -5),
    # the merge's grid (one workgroup per 4 query rows) must fit 32 bits too:
    # 2^16 heads of 2^17 queries against 64 keys need 2^31 of them
    (dict(H=1 << 16, Nq=1 << 17, Nk=64, causal=0), -2),
    (dict(H=1 << 16, Nq=(1 << 17) - 4, Nk=64, causal=0, scale=0.0), -6),
])
def test_kv_validation(args, code):
    lib = _lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=4, Nk=100, d=64, causal=1,
             scale=0.125, dtype=1, splits=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(args)
    rc = lib.attn_fwd_kv(a["q"] or None, a["k"], a["v"], a["o"], a["lse"] or None, a["B"],
                         a["H"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"],
                         a["splits"], a["ws"] or None, a["ws_bytes"], None)
    assert rc == code


def test_bwd_kv_workspace_size():
    lib = _lib()
    r256 = lambda x: (x + 255) // 256 * 256

    def expect(B, H, Nq, Nk, d):
        # D, plus the fp32 dQ partials when dQ is split over the keys (attn.h)
        n = r256(B * H * Nq * 4)
        if Nq < Nk:
            w = B * H * -(-Nq // 128)
            T = -(-Nk // 64)
            m = min(-(-512 // w), max(1, T // 8))
            if m > 1:
                per = -(-T // m)
                s = -(-T // per)
                if s > 1:
                    n += r256(s * B * H * Nq * d * 4)
        return n

    for shape in ((2, 16, 512, 4096, 128), (1, 3, 7, 100, 64), (1, 1, 7, 100, 256),
                  (1, 2, 128, 1000, 64), (1, 2, 130, 2049, 128), (8, 32, 512, 4096, 128),
                  (1, 1, 300, 300, 64)):
        assert lib.attn_bwd_kv_workspace_bytes(*shape, 1) == expect(*shape), shape
    # the chunked-prefill shape splits dQ four ways; square and tiny shapes do not
    assert lib.attn_bwd_kv_workspace_bytes(2, 16, 512, 4096, 128, 1) == 2 * 16 * 512 * 4 + 4 * 2 * 16 * 512 * 128 * 4
    assert lib.attn_bwd_kv_workspace_bytes(1, 3, 7, 100, 64, 1) == 256  # 84 bytes, rounded
    assert lib.attn_bwd_kv_workspace_bytes(1, 1, 7, 100, 256, 1) == 256
    assert lib.attn_bwd_kv_workspace_bytes(1, 1, 7, 100, 80, 1) == 0
    assert lib.attn_bwd_kv_workspace_bytes(1, 1, 7, 100, 64, 0) == 0  # bf16 only
    assert lib.attn_bwd_kv_workspace_bytes(1, 1, 0, 100, 64, 1) == 0


@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1), (dict(dv=0), -1), (dict(B=0), -2), (dict(Nq=0), -2), (dict(Nk=0), -2),
    (dict(Nq=20, Nk=10, causal=1), -2), (dict(d=48), -4), (dict(d=256, scale=0.0), -6),
    (dict(dtype=0), -3), (dict(dk=FAKE + 4), -5), (dict(lse=FAKE + 2), -5),
    (dict(scale=0.0), -6), (dict(scale=-1.0), -6), (dict(scale=float("inf")), -6),
    (dict(lse=FAKE + 4, scale=0.0), -6),
    (dict(ws=0), -7), (dict(ws_bytes=8), -7), (dict(ws=FAKE + 8), -5),
])
def test_bwd_kv_validation(args, code):
    lib = _lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             ws=FAKE, ws_bytes=1 << 30, B=1, H=1, Nq=4, Nk=100, d=64, causal=1, scale=0.125,
             dtype=1)
    a.update(args)
    rc = lib.attn_bwd_kv(*(a[n] or None for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk",
                                                  "dv", "ws")),
                         a["ws_bytes"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["causal"],
                         a["scale"], a["dtype"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(x=0), -1), (dict(y=0), -1), (dict(M=0), -2), (dict(N=0), -2), (dict(M=(1 << 40) + 1), -2),
    (dict(M=1 << 30, N=1 << 20), -2),
    # M * N = 2^63 overflows a 64-bit product: refused, not wrapped negative
    (dict(M=1 << 40, N=1 << 23), -2), (dict(M=1 << 40, N=(1 << 31) - 1), -2),
    (dict(M=(1 << 40) - 1, N=1 << 24), -2),
    (dict(dtype=2), -3), (dict(x=FAKE + 4), -5), (dict(y=FAKE + 2), -5),
])
def test_softmax_rows_validation(args, code):
    lib = _lib()
    a = dict(x=FAKE, y=FAKE, M=4, N=100, dtype=1)
    a.update(args)
    assert lib.attn_softmax_rows(a["x"] or None, a["y"] or None, a["M"], a["N"], a["dtype"],
                                 None) == code


@pytest.mark.parametrize("args,code", [
    (dict(q8=0), -1), (dict(k_scale=0), -1), (dict(N=0), -2), (dict(d=96), -4), (dict(d=256), -4),
    (dict(q8=FAKE + 8), -5), (dict(q_scale=FAKE + 2), -5), (dict(d=64, k_scale=FAKE + 1), -5),
    (dict(lse=FAKE + 2), -5),
    (dict(scale=float("nan")), -6), (dict(scale=0.0), -6), (dict(scale=-0.0), -6),
    (dict(scale=-0.1), -6), (dict(lse=FAKE + 4, scale=0.0), -6),
])
def test_fwd_mx_validation(args, code):
    lib = _lib()
    a = dict(q8=FAKE, q_scale=FAKE, k8=FAKE, k_scale=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1,
             N=16, d=128, causal=1, scale=0.1)
    a.update(args)
    rc = lib.attn_fwd_mx(*(a[n] or None for n in ("q8", "q_scale", "k8", "k_scale", "v", "o",
                                                    "lse")),
                         a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], None)
    assert rc == code


def test_binding_refuses_host_tensors():
    """The binding passes raw pointers, so host tensors are refused before any
    library call (they would be dereferenced as device addresses)."""
    import torch
    import tiled_online_softmax_attn_amd as T
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        T.attn_fwd(q, q.clone(), q.clone(), torch.empty_like(q), lse, True, 0.125)
    with pytest.raises(ValueError):
        T.attn_softmax_rows(q, torch.empty_like(q))


@pytest.mark.parametrize("args,code", [
    (dict(q8=0), -1), (dict(vt8=0), -1), (dict(vt_scale=0), -1), (dict(N=0), -2),
    (dict(N=(1 << 26) + 1), -2), (dict(d=96), -4), (dict(d=256), -4),
    (dict(vt8=FAKE + 8), -5), (dict(vt_scale=FAKE + 1), -5), (dict(q_scale=FAKE + 2), -5),
    (dict(lse=FAKE + 2), -5),
    (dict(scale=float("nan")), -6), (dict(scale=0.0), -6), (dict(scale=-0.5), -6),
    # a 2-byte aligned V^T scale pointer and a 4-byte aligned lse pass the
    # alignment checks; the (later) scale check stops the call
    (dict(vt_scale=FAKE + 2, lse=FAKE + 4, scale=0.0), -6),
])
def test_fwd_fp8_validation(args, code):
    lib = _lib()
    a = dict(q8=FAKE, q_scale=FAKE, k8=FAKE, k_scale=FAKE, vt8=FAKE, vt_scale=FAKE, o=FAKE,
             lse=FAKE, B=1, H=1, N=16, d=128, causal=1, scale=0.1)
    a.update(args)
    rc = lib.attn_fwd_fp8(*(a[n] or None for n in ("q8", "q_scale", "k8", "k_scale", "vt8",
                                                     "vt_scale", "o", "lse")),
                          a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], None)
    assert rc == code
