"""Python binding of libattn.so, the MI355X (gfx950) fused attention library.

The functions here marshal arguments only: they read pointers, shapes and the
current HIP stream from torch tensors and call the C ABI declared in
``include/attn.h`` with the same names.  Every step of the computation runs
in the library's HIP kernels; there is no fallback.  If ``libattn.so`` has not
been built (``python -m tiled_online_softmax_attn_amd.build``), importing the
library raises ``AttnLibraryMissing``.

Tensors: Q, K, V, O, dO, dQ, dK, dV are CUDA(HIP) tensors of shape
[B, H, N, d], contiguous, all of one dtype (torch.bfloat16, or torch.float32
for the forward only); lse is float32 [B, H, N].  attn_fwd_kv takes Q and O
of shape [B, H, Nq, d] and K, V of shape [B, H, Nk, d] (bf16).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_DTYPE",
          -4: "ATTN_ERR_HEADDIM", -5: "ATTN_ERR_ALIGN", -6: "ATTN_ERR_SCALE",
          -7: "ATTN_ERR_WORKSPACE", -8: "ATTN_ERR_HIP", -9: "ATTN_ERR_SCRATCH"}
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_phase", "attn_bwd_workspace_bytes",
           "attn_fwd_kv", "attn_fwd_kv_workspace_bytes", "attn_bwd_kv", "attn_bwd_kv_workspace_bytes",
           "attn_softmax_rows", "attn_fwd_mx", "attn_fwd_fp8",
           "attn_status_str", "attn_abi_version")


class AttnLibraryMissing(RuntimeError):
    pass


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_str(code)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattn.so and declare its ABI (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise AttnLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m tiled_online_softmax_attn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.attn_fwd.restype = i
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.attn_bwd.restype = i
        L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                               i, i, i, i, i, f, i, vp]
        L.attn_bwd_noalloc.restype = i
        L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.attn_bwd_phase.restype = i
        L.attn_bwd_phase.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                     i, i, i, i, i, f, i, vp]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.attn_fwd_kv.restype = i
        L.attn_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp,
                                  ctypes.c_size_t, vp]
        L.attn_fwd_kv_workspace_bytes.restype = ctypes.c_size_t
        L.attn_fwd_kv_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.attn_bwd_kv.restype = i
        L.attn_bwd_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                  i, i, i, i, i, i, f, i, vp]
        L.attn_bwd_kv_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd_kv_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.attn_fwd_mx.restype = i
        L.attn_fwd_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        L.attn_fwd_fp8.restype = i
        L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        L.attn_softmax_rows.restype = i
        L.attn_softmax_rows.argtypes = [vp, vp, ctypes.c_longlong, i, i, vp]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_status_str.argtypes = [i]
        L.attn_abi_version.restype = i
        L.attn_abi_version.argtypes = []
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().attn_status_str(int(code)).decode()


def attn_status_str(code: int) -> str:
    return status_str(code)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    return -1


def _stream_handle(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(int(x) for x in q.shape)


def _check_contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d] (lse [B, H, N])")


def _check(where: str, t, shape, dtypes, device) -> None:
    """The kernels see raw pointers and the sizes taken from the first
    tensor, so every other tensor must have exactly the expected shape and
    dtype and live on the same GPU; anything else is refused here rather than
    read or written out of bounds."""
    if t is None:
        return  # the library reports ATTN_ERR_NULL
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{where}: expected a torch.Tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{where}: tensor on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{where}: dtype {t.dtype}, expected one of {dtypes}")


def _check_workspace(where: str, ws, device) -> None:
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"{where}: workspace must be a contiguous tensor on {device}")


def attn_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """Enqueue the forward: o = softmax(scale q k^T [+ causal]) v, lse = row
    logsumexp.  All tensors preallocated by the caller."""
    _check_contig(q, k, v, o, lse)
    B, H, N, d = _shape(q)
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check(f"attn_fwd {name}", t, q.shape, (q.dtype,), q.device)
    _check("attn_fwd lse", lse, (B, H, N), (torch.float32,), q.device)
    rc = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                        int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd")


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int,
                             dtype: torch.dtype = torch.bfloat16) -> int:
    code = ATTN_DTYPE_BF16 if dtype == torch.bfloat16 else ATTN_DTYPE_F32
    return int(lib().attn_bwd_workspace_bytes(B, H, N, d, code))


def _check_bwd(where, q, k, v, o, dout, lse, dq, dk, dv, workspace) -> None:
    B, H, N, _ = _shape(q)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check(f"{where} {name}", t, q.shape, (q.dtype,), q.device)
    _check(f"{where} lse", lse, (B, H, N), (torch.float32,), q.device)
    _check_workspace(where, workspace, q.device)


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
             stream=None) -> None:
    """Enqueue the backward: dq, dk, dv of sum(dout * o).  ``workspace`` is a
    device tensor of at least attn_bwd_workspace_bytes() bytes."""
    _check_contig(q, k, v, o, dout, lse, dq, dk, dv)
    B, H, N, d = _shape(q)
    _check_bwd("attn_bwd", q, k, v, o, dout, lse, dq, dk, dv, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d,
                        int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_bwd")


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float,
                     stream=None) -> None:
    """Enqueue the backward with no workspace: the library's static device
    scratch holds D (B*H*N at most 4194304 rows).  Results equal attn_bwd's
    bit for bit; calls that overlap in time on one GPU race."""
    _check_contig(q, k, v, o, dout, lse, dq, dk, dv)
    B, H, N, d = _shape(q)
    _check_bwd("attn_bwd_noalloc", q, k, v, o, dout, lse, dq, dk, dv, None)
    rc = lib().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                                float(scale), _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_bwd_noalloc")


def attn_bwd_phase(phase: int, q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool,
                   scale: float, stream=None) -> None:
    """Enqueue one phase of the backward (0: D = rowsum(dO * O) into the
    workspace; 1: dK and dV; 2: dQ; 3: dQ forming D itself, i.e. 0 and 2 in
    one launch).  attn_bwd runs phase 3, then phase 1."""
    _check_contig(q, k, v, o, dout, lse, dq, dk, dv)
    B, H, N, d = _shape(q)
    _check_bwd(f"attn_bwd_phase({phase})", q, k, v, o, dout, lse, dq, dk, dv, workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_bwd_phase(int(phase), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                              B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q),
                              _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, f"attn_bwd_phase({phase})")


def attn_fwd_kv_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int = 0,
                                dtype: torch.dtype = torch.bfloat16) -> int:
    code = ATTN_DTYPE_BF16 if dtype == torch.bfloat16 else ATTN_DTYPE_F32
    return int(lib().attn_fwd_kv_workspace_bytes(B, H, Nq, Nk, d, int(num_splits), code))


def attn_fwd_kv(q, k, v, o, lse, causal: bool, scale: float, num_splits: int, workspace,
                stream=None) -> None:
    """Enqueue the forward of Nq queries (the last Nq positions) against Nk
    cached keys and values; the key range is split into ``num_splits`` chunks
    (0 = chosen by the library) whose partial results are merged."""
    _check_contig(q, k, v, o, lse)
    B, H, Nq, d = _shape(q)
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("attn_fwd_kv: k must be a [B, H, Nk, d] tensor")
    Nk = int(k.shape[2])
    _check("attn_fwd_kv k", k, (B, H, Nk, d), (q.dtype,), q.device)
    _check("attn_fwd_kv v", v, (B, H, Nk, d), (q.dtype,), q.device)
    _check("attn_fwd_kv o", o, q.shape, (q.dtype,), q.device)
    _check("attn_fwd_kv lse", lse, (B, H, Nq), (torch.float32,), q.device)
    _check_workspace("attn_fwd_kv", workspace, q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                           int(bool(causal)), float(scale), _dtype_code(q), int(num_splits),
                           _ptr(workspace), ws_bytes, _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_kv")


def attn_bwd_kv_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int,
                                dtype: torch.dtype = torch.bfloat16) -> int:
    code = ATTN_DTYPE_BF16 if dtype == torch.bfloat16 else ATTN_DTYPE_F32
    return int(lib().attn_bwd_kv_workspace_bytes(B, H, Nq, Nk, d, code))


def attn_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
                stream=None) -> None:
    """Enqueue the backward of attn_fwd_kv: q, o, dout, dq [B, H, Nq, d]; k, v,
    dk, dv [B, H, Nk, d]; lse [B, H, Nq]; the queries are the last Nq
    positions.  ``workspace``: at least attn_bwd_kv_workspace_bytes() bytes."""
    _check_contig(q, k, v, o, dout, lse, dq, dk, dv)
    B, H, Nq, d = _shape(q)
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("attn_bwd_kv: k must be a [B, H, Nk, d] tensor")
    Nk = int(k.shape[2])
    for name, t, n in (("k", k, Nk), ("v", v, Nk), ("dk", dk, Nk), ("dv", dv, Nk), ("o", o, Nq),
                       ("dout", dout, Nq), ("dq", dq, Nq)):
        _check(f"attn_bwd_kv {name}", t, (B, H, n, d), (q.dtype,), q.device)
    _check("attn_bwd_kv lse", lse, (B, H, Nq), (torch.float32,), q.device)
    _check_workspace("attn_bwd_kv", workspace, q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_bwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, Nq, Nk, d,
                           int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_bwd_kv")


def attn_fwd_mx(q8, q_scale, k8, k_scale, v, o, lse, causal: bool, scale: float,
                stream=None) -> None:
    """Enqueue the forward with Q and K in MXFP8: q8, k8 E4M3 codes [B, H, N,
    d] (uint8 or float8_e4m3fn tensors), q_scale, k_scale E8M0 codes
    [B, H, N, d / 32] (uint8), v and o bf16 [B, H, N, d], lse fp32 [B, H, N]."""
    _check_contig(q8, q_scale, k8, k_scale, v, o, lse)
    B, H, N, d = _shape(q8)
    codes = (torch.uint8, torch.float8_e4m3fn)
    dev = q8.device
    _check("attn_fwd_mx q8", q8, (B, H, N, d), codes, dev)
    _check("attn_fwd_mx k8", k8, (B, H, N, d), codes, dev)
    _check("attn_fwd_mx q_scale", q_scale, (B, H, N, d // 32), (torch.uint8,), dev)
    _check("attn_fwd_mx k_scale", k_scale, (B, H, N, d // 32), (torch.uint8,), dev)
    _check("attn_fwd_mx v", v, (B, H, N, d), (torch.bfloat16,), dev)
    _check("attn_fwd_mx o", o, (B, H, N, d), (torch.bfloat16,), dev)
    _check("attn_fwd_mx lse", lse, (B, H, N), (torch.float32,), dev)
    rc = lib().attn_fwd_mx(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), _ptr(o),
                           _ptr(lse), B, H, N, d, int(bool(causal)), float(scale),
                           _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_mx")


def fp8_v_row_length(N: int) -> int:
    """Row length (ldv) of the V^T codes attn_fwd_fp8 takes: 64 ceil(N / 64)."""
    return (int(N) + 63) // 64 * 64


def attn_fwd_fp8(q8, q_scale, k8, k_scale, vt8, vt_scale, o, lse, causal: bool, scale: float,
                 stream=None) -> None:
    """Enqueue the FP8 forward: q8, k8 E4M3 codes [B, H, N, d] with E8M0
    scales q_scale, k_scale [B, H, N, d / 32] (as attn_fwd_mx); vt8 the E4M3
    codes of V^T [B, H, d, ldv] (ldv = fp8_v_row_length(N)) with E8M0 scales
    vt_scale [B, H, d, ldv / 32] along the keys; o bf16 [B, H, N, d], lse fp32
    [B, H, N]."""
    _check_contig(q8, q_scale, k8, k_scale, vt8, vt_scale, o, lse)
    B, H, N, d = _shape(q8)
    ldv = fp8_v_row_length(N)
    codes = (torch.uint8, torch.float8_e4m3fn)
    dev = q8.device
    _check("attn_fwd_fp8 q8", q8, (B, H, N, d), codes, dev)
    _check("attn_fwd_fp8 k8", k8, (B, H, N, d), codes, dev)
    _check("attn_fwd_fp8 q_scale", q_scale, (B, H, N, d // 32), (torch.uint8,), dev)
    _check("attn_fwd_fp8 k_scale", k_scale, (B, H, N, d // 32), (torch.uint8,), dev)
    _check("attn_fwd_fp8 vt8", vt8, (B, H, d, ldv), codes, dev)
    _check("attn_fwd_fp8 vt_scale", vt_scale, (B, H, d, ldv // 32), (torch.uint8,), dev)
    _check("attn_fwd_fp8 o", o, (B, H, N, d), (torch.bfloat16,), dev)
    _check("attn_fwd_fp8 lse", lse, (B, H, N), (torch.float32,), dev)
    rc = lib().attn_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vt8),
                            _ptr(vt_scale), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                            float(scale), _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_fp8")


def attn_softmax_rows(x, y, stream=None) -> None:
    """Enqueue y = row-wise softmax of x (both contiguous, same shape and
    dtype, fp32 or bf16; the last dimension is the row; y may be x)."""
    _check_contig(x, y)
    if x.shape != y.shape or x.dtype != y.dtype:
        raise ValueError("x and y must have the same shape and dtype")
    _check("attn_softmax_rows y", y, x.shape, (x.dtype,), x.device)
    if x.device.type != "cuda":
        raise ValueError(f"attn_softmax_rows: tensor on {x.device}, expected a GPU tensor")
    N = int(x.shape[-1]) if x.dim() > 0 else 1
    M = x.numel() // max(N, 1)
    rc = lib().attn_softmax_rows(_ptr(x), _ptr(y), M, N, _dtype_code(x), _stream_handle(stream))
    if rc != 0:
        raise AttnError(rc, "attn_softmax_rows")


# ------------------------------------------------------------ conveniences
def flash_attention_forward(q, k, v, causal: bool = False, scale: float | None = None):
    """Allocate o and lse with torch and run attn_fwd; returns (o, lse)."""
    B, H, N, d = _shape(q)
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    attn_fwd(q, k, v, o, lse, causal, scale)
    return o, lse


def flash_attention_kv(q, k, v, causal: bool = False, scale: float | None = None,
                       num_splits: int = 0, workspace=None):
    """Allocate o, lse (and a workspace if none is given) and run attn_fwd_kv;
    returns (o, lse)."""
    B, H, Nq, d = _shape(q)
    Nk = int(k.shape[2])
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = torch.empty(attn_fwd_kv_workspace_bytes(B, H, Nq, Nk, d, num_splits, q.dtype),
                                device=q.device, dtype=torch.uint8)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    attn_fwd_kv(q, k, v, o, lse, causal, scale, num_splits, workspace)
    return o, lse


def flash_attention_backward(q, k, v, o, lse, dout, causal: bool = False,
                             scale: float | None = None, workspace=None):
    """Allocate dq, dk, dv (and a workspace if none is given) and run attn_bwd."""
    B, H, N, d = _shape(q)
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = torch.empty(attn_bwd_workspace_bytes(B, H, N, d, q.dtype), device=q.device,
                                dtype=torch.uint8)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal, scale)
    return dq, dk, dv


def flash_attention_backward_kv(q, k, v, o, lse, dout, causal: bool = False,
                                scale: float | None = None, workspace=None):
    """Allocate dq, dk, dv (and a workspace if none is given) and run
    attn_bwd_kv."""
    B, H, Nq, d = _shape(q)
    Nk = int(k.shape[2])
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = torch.empty(attn_bwd_kv_workspace_bytes(B, H, Nq, Nk, d, q.dtype),
                                device=q.device, dtype=torch.uint8)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal, scale)
    return dq, dk, dv
