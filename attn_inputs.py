"""Seeded synthetic inputs shared by the tests, the smoke check and bench.py.

This module holds workload shapes and random draws only; none of the
attention arithmetic.  The oracle and the HIP path both consume the tensors
it returns, so they see bit-identical inputs.

Recipe (the pages fix no random generator; this is the plainest reading):
a CPU ``torch.Generator`` seeded with ``seed`` draws Q, K, V and then dO, in
that order, each as ``torch.randn`` in float32 of shape [B, H, N, d].  Q and
K are multiplied by ``qk_std`` (3 for the long-sequence large-logit
workload), and every tensor is then rounded to the working dtype with
``.to(dtype)`` (round-to-nearest-even for bfloat16).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    causal: bool
    seed: int
    qk_std: float = 1.0
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d, halved under the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """2.5 times the forward count (five contractions instead of two)."""
        return 2.5 * self.fwd_flops()


# The five workloads: shapes, dtypes, masks and distributions as specified.
WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 256, 64, torch.float32, False, 1),
    "h8_n1024_d64": Workload("h8_n1024_d64", 1, 8, 1024, 64, torch.bfloat16, False, 2),
    "h8_n1024_d64_causal": Workload("h8_n1024_d64_causal", 1, 8, 1024, 64, torch.bfloat16, True, 2),
    "b4_h16_n4096_d128_causal": Workload("b4_h16_n4096_d128_causal", 4, 16, 4096, 128,
                                         torch.bfloat16, True, 3),
    "h32_n16384_d128_causal_bigqk": Workload("h32_n16384_d128_causal_bigqk", 1, 32, 16384, 128,
                                             torch.bfloat16, True, 4, qk_std=3.0),
    "b2_h16_n4096_d64_causal_fwdbwd": Workload("b2_h16_n4096_d64_causal_fwdbwd", 2, 16, 4096, 64,
                                               torch.bfloat16, True, 5, backward=True),
}

HEADLINE = "b4_h16_n4096_d128_causal"

# The headline shape at the other head dimensions the kernels take (forward
# and backward; d = 256 forward only), and at a length that is a multiple of
# neither tile (4001 = 31 * 128 + 33 queries, 62 * 64 + 33 keys: tail tiles
# on both loops); the pages fix no workload for them.
HEADDIM_WORKLOADS = {
    "b4_h16_n4001_d128_causal": Workload("b4_h16_n4001_d128_causal", 4, 16, 4001, 128,
                                         torch.bfloat16, True, 13, backward=True),
    "b4_h16_n4096_d256_causal": Workload("b4_h16_n4096_d256_causal", 4, 16, 4096, 256,
                                         torch.bfloat16, True, 11),
    "b4_h16_n4096_d96_causal": Workload("b4_h16_n4096_d96_causal", 4, 16, 4096, 96,
                                        torch.bfloat16, True, 9, backward=True),
    "b4_h16_n4096_d32_causal": Workload("b4_h16_n4096_d32_causal", 4, 16, 4096, 32,
                                        torch.bfloat16, True, 10, backward=True),
}


def make_inputs(B: int, H: int, N: int, d: int, dtype: torch.dtype = torch.bfloat16,
                seed: int = 0, qk_std: float = 1.0, with_dout: bool = False):
    """Return CPU tensors (q, k, v[, dout]) of shape [B, H, N, d] in ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    dout = torch.randn(shape, generator=g, dtype=torch.float32) if with_dout else None
    if qk_std != 1.0:
        q = q * qk_std
        k = k * qk_std
    out = [q.to(dtype), k.to(dtype), v.to(dtype)]
    if with_dout:
        out.append(dout.to(dtype))
    return tuple(out)


def workload_inputs(w: Workload, with_dout: bool | None = None):
    if with_dout is None:
        with_dout = w.backward
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_std, with_dout)


@dataclass(frozen=True)
class KvWorkload:
    """Nq queries (the last Nq positions) against an Nk-token key/value
    cache: decode (Nq = 1) and chunked prefill shapes."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: torch.dtype
    causal: bool
    seed: int
    backward: bool = False  # a step is attn_fwd_kv + attn_bwd_kv (dO drawn after V)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def kv_bytes(self) -> float:
        """Bytes of K and V, each read once: the compulsory HBM traffic that
        bounds decode."""
        return 2.0 * self.B * self.H * self.Nk * self.d * torch.finfo(self.dtype).bits / 8

    def flops(self) -> float:
        """4*B*H*Nq*d times the number of visible (query, key) pairs per head."""
        if self.causal:
            off = self.Nk - self.Nq
            pairs = sum(min(self.Nk, i + off + 1) for i in range(self.Nq))
        else:
            pairs = self.Nq * self.Nk
        return 4.0 * self.B * self.H * pairs * self.d


# Decode and chunked-prefill shapes for attn_fwd_kv.  The pages give no decode
# shape; these are typical serving sizes (8 sequences of 8k tokens, 32 heads).
KV_WORKLOADS = {
    "decode_b8_h32_nq1_nk8192_d128": KvWorkload("decode_b8_h32_nq1_nk8192_d128", 8, 32, 1, 8192,
                                                128, torch.bfloat16, True, 6),
    "prefill_b2_h16_nq512_nk4096_d128": KvWorkload("prefill_b2_h16_nq512_nk4096_d128", 2, 16, 512,
                                                   4096, 128, torch.bfloat16, True, 7),
    # the same chunk as a training step: forward and backward
    "prefill_b2_h16_nq512_nk4096_d128_fwdbwd": KvWorkload(
        "prefill_b2_h16_nq512_nk4096_d128_fwdbwd", 2, 16, 512, 4096, 128, torch.bfloat16, True, 7,
        backward=True),
}


def make_kv_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: torch.dtype = torch.bfloat16,
                   seed: int = 0, with_dout: bool = False):
    """CPU tensors q [B, H, Nq, d] and k, v [B, H, Nk, d] (and dO [B, H, Nq,
    d] with ``with_dout``): a seeded CPU generator draws Q, K, V (then dO) in
    that order as float32 N(0, 1), then rounds to ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    out = [q.to(dtype), k.to(dtype), v.to(dtype)]
    if with_dout:
        out.append(torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32).to(dtype))
    return tuple(out)


def kv_workload_inputs(w: KvWorkload):
    return make_kv_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, w.backward)


@dataclass(frozen=True)
class SoftmaxWorkload:
    """Row softmax of an M x N matrix of scores (M rows of N keys)."""
    name: str
    M: int
    N: int
    dtype: torch.dtype
    seed: int
    std: float = 1.0

    def hbm_bytes(self) -> float:
        """Each element read once and written once: the compulsory traffic."""
        return 2.0 * self.M * self.N * torch.finfo(self.dtype).bits / 8


# Attention-score rows: 65536 query rows (B4 H16 N1024) of 4096 keys, the
# score distribution of scale * q.k with unit-normal q and k (N(0, 1)).
SOFTMAX_WORKLOADS = {
    "softmax_m65536_n4096_bf16": SoftmaxWorkload("softmax_m65536_n4096_bf16", 65536, 4096,
                                                 torch.bfloat16, 8),
}


def make_softmax_inputs(M: int, N: int, dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                        std: float = 1.0, mask: str = "none"):
    """CPU tensor [M, N]: a seeded CPU generator draws float32 N(0, std^2),
    then rounds to ``dtype``.  mask="causal" sets entry (r, j) to -inf for
    j > r mod N, the score rows of a causal head (row r = query r mod N)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn((M, N), generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mask == "causal":
        r = torch.arange(M).unsqueeze(1) % N
        j = torch.arange(N).unsqueeze(0)
        x = x.masked_fill(j > r, float("-inf"))
    elif mask != "none":
        raise ValueError(mask)
    return x.to(dtype)


def softmax_workload_inputs(w: SoftmaxWorkload):
    return make_softmax_inputs(w.M, w.N, w.dtype, w.seed, w.std)


def make_mx_inputs(B: int, H: int, N: int, d: int, seed: int = 0, scale_lo: int = 125,
                   scale_hi: int = 129):
    """CPU tensors for the MXFP8 forward: q8, k8 uint8 E4M3 codes [B, H, N, d]
    (float32 N(0, 1) draws cast with torch's float8_e4m3fn conversion), their
    E8M0 scale codes q_scale, k_scale uint8 [B, H, N, d / 32] drawn uniformly
    from [scale_lo, scale_hi] (block scales 2^-2 .. 2^2 by default), and v
    bf16 [B, H, N, d] (N(0, 1)).  Draw order: Q, K, V values, then the Q and
    K scale codes."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    sshape = (B, H, N, d // 32)
    qs = torch.randint(scale_lo, scale_hi + 1, sshape, generator=g, dtype=torch.int32)
    ks = torch.randint(scale_lo, scale_hi + 1, sshape, generator=g, dtype=torch.int32)
    q8 = q.to(torch.float8_e4m3fn).view(torch.uint8)
    k8 = k.to(torch.float8_e4m3fn).view(torch.uint8)
    return q8, qs.to(torch.uint8), k8, ks.to(torch.uint8), v.to(torch.bfloat16)


def make_fp8_v(B: int, H: int, N: int, d: int, seed: int = 0, scale_lo: int = 125,
               scale_hi: int = 129, pad_code: int = 0, pad_scale: int = 127):
    """CPU tensors for V in the layout of the FP8 forward: vt8 uint8 E4M3
    codes of V^T [B, H, d, ldv] (ldv = 64 ceil(N / 64); float32 N(0, 1) draws
    of V [B, H, N, d] cast with torch's float8_e4m3fn conversion, then
    transposed) and their E8M0 scale codes vt_scale uint8 [B, H, d, ldv / 32]
    drawn uniformly from [scale_lo, scale_hi], one per 32 keys.  Keys N ..
    ldv - 1 hold pad_code and blocks wholly past N pad_scale (the kernel must
    ignore both; tests pass NaN codes 0x7F / 0xFF there).  Draw order: V
    values, then the scale codes."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    ldv = (N + 63) // 64 * 64
    v = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    sc = torch.randint(scale_lo, scale_hi + 1, (B, H, d, ldv // 32), generator=g,
                       dtype=torch.int32).to(torch.uint8)
    vt8 = torch.full((B, H, d, ldv), pad_code, dtype=torch.uint8)
    vt8[..., :N] = v.to(torch.float8_e4m3fn).view(torch.uint8).transpose(2, 3)
    first_pad_block = (N + 31) // 32
    sc[..., first_pad_block:] = pad_scale
    return vt8.contiguous(), sc.contiguous()


# The headline shape with Q and K in MXFP8 (seed 12).
MX_WORKLOADS = {
    "b4_h16_n4096_d128_causal_mxfp8": Workload("b4_h16_n4096_d128_causal_mxfp8", 4, 16, 4096, 128,
                                               torch.bfloat16, True, 12),
    # the same with V (and P) in FP8 too (attn_fwd_fp8); V drawn with seed 13
    "b4_h16_n4096_d128_causal_fp8": Workload("b4_h16_n4096_d128_causal_fp8", 4, 16, 4096, 128,
                                             torch.bfloat16, True, 12),
}
