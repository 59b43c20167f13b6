"""GPU parity of attn_softmax_rows (standalone fused row softmax) against the
fp64 oracle's oracle_softmax_row on the same seeded inputs.

Coverage: every dispatch branch of both dtypes (one wave per row; a
workgroup per row with 2, 4 or 16 pieces per thread; the two-pass long-row
kernel), row lengths that are and are not multiples of the 16-byte piece,
N = 1, peaky rows (large logits), rows masked with -inf down to one finite
entry, in place, the bench workload on sampled rows plus all row sums, grid
striding past the workgroup cap of both kernels, and bitwise determinism.

Besides the stated tolerances, every case also meets a tighter bound derived
from the arithmetic: fp32 outputs carry a few fp32 roundings of the exponent
(relative error well under 1e-5); bf16 outputs are one round-to-nearest of
an fp32 value to 8 significant bits, relative error at most 2^-8 (3.9e-3),
checked as 4e-3.
"""
import numpy as np
import pytest
import torch

from attn_inputs import SOFTMAX_WORKLOADS, make_softmax_inputs, softmax_workload_inputs
from tests.parity import compare, describe, gpu_softmax, log, oracle_softmax_rows, to_np

pytestmark = pytest.mark.gpu

TIGHT_REL = {torch.float32: 1e-5, torch.bfloat16: 4e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_online_softmax_attn_amd as T
    T.lib()  # raises if libattn.so is missing: no silent fallback


def _check(y, ref, dtype, tag):
    got = to_np(y)
    e = compare(got, ref, dtype, tag)
    err = np.abs(got - ref)
    bound = TIGHT_REL[dtype] * np.abs(ref) + 1e-12
    bad = err > bound
    assert not bad.any(), f"{tag}: {int(bad.sum())} elements beyond the derived bound"
    log(f"    {tag}: {describe(e)}")


def _case(M, N, dtype, seed, std=1.0, mask="none", inplace=False, tag=""):
    x = make_softmax_inputs(M, N, dtype, seed, std, mask)
    log(f"[softmax] {tag} M={M} N={N} {dtype} std={std} mask={mask} inplace={inplace}")
    y = gpu_softmax(x, inplace)
    ref = oracle_softmax_rows(to_np(x))
    _check(y, ref, dtype, tag or f"M={M} N={N}")


# fp32 branches: N <= 1024 one wave per row; <= 2048, <= 4096, <= 16384 a
# workgroup per row; longer two passes.  bf16: 2048, 4096, 8192, 16384.
SHAPES = [(1, 1), (3, 1), (5, 7), (17, 100), (64, 1000), (9, 1024), (33, 1025), (8, 2048),
          (7, 2047), (6, 2049), (5, 4096), (6, 4100), (4, 8192), (3, 8191), (2, 16384),
          (3, 16383), (2, 16385), (2, 40000), (1, 100003)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_shapes(M, N, dtype):
    _case(M, N, dtype, seed=300 + M + N)


@pytest.mark.parametrize("N", [100, 2048, 4100, 16384, 20000])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_peaky_rows(N, dtype):
    """std 30: row maxima far above the rest, exponents down to -200."""
    _case(7, N, dtype, seed=400 + N, std=30.0)


@pytest.mark.parametrize("N", [64, 1000, 4096, 20000])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_masked_rows(N, dtype):
    """Causal score rows: row r keeps r mod N + 1 entries (row 0 only one)."""
    _case(9, N, dtype, seed=500 + N, mask="causal")


@pytest.mark.parametrize("M,N", [(13, 777), (4, 4096), (2, 30000)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_in_place(M, N, dtype):
    _case(M, N, dtype, seed=600 + N, inplace=True)


def test_single_column_is_one():
    x = make_softmax_inputs(1000, 1, torch.float32, seed=7)
    y = gpu_softmax(x)
    assert torch.equal(y, torch.ones_like(y))


def _sampled(x, y, rows, dtype, tag):
    ref = oracle_softmax_rows(to_np(x[rows]))
    _check(y[rows], ref, dtype, tag)


def _row_sums(y, dtype, tag):
    s = y.double().sum(dim=1)
    dev = float((s - 1).abs().max())
    log(f"    {tag}: max |row sum - 1| = {dev:.3e}")
    assert dev <= TIGHT_REL[dtype], f"{tag}: row sums off by {dev:.3e}"


def test_workload_full():
    """The bench workload at full size: 64 sampled rows against the oracle,
    every row sum equal to 1 within the output rounding."""
    w = SOFTMAX_WORKLOADS["softmax_m65536_n4096_bf16"]
    x = softmax_workload_inputs(w)
    log(f"[softmax] workload {w.name}")
    y = gpu_softmax(x)
    g = torch.Generator().manual_seed(11)
    rows = torch.cat([torch.tensor([0, 1, w.M - 1]), torch.randint(0, w.M, (61,), generator=g)])
    _sampled(x, y, rows, w.dtype, w.name)
    _row_sums(y, w.dtype, w.name)


def test_grid_stride_short_rows():
    """4 * 2^20 + 5 rows of 3: more one-wave-per-row groups than one launch
    holds, so workgroups stride over the rest."""
    M = 4 * (1 << 20) + 5
    x = make_softmax_inputs(M, 3, torch.float32, seed=12)
    log(f"[softmax] grid stride M={M} N=3")
    y = gpu_softmax(x)
    rows = torch.cat([torch.arange(8), torch.arange(M - 300, M)])
    _sampled(x, y, rows, torch.float32, "short-row stride")
    _row_sums(y, torch.float32, "short-row stride")


def test_grid_stride_long_rows():
    """8195 rows of 16400 bf16: past the long-row kernel's workgroup cap."""
    M, N = 8195, 16400
    x = make_softmax_inputs(M, N, torch.bfloat16, seed=13)
    log(f"[softmax] grid stride M={M} N={N}")
    y = gpu_softmax(x)
    rows = torch.tensor([0, 1, 4096, 8191, 8192, 8193, 8194])
    _sampled(x, y, rows, torch.bfloat16, "long-row stride")
    _row_sums(y, torch.bfloat16, "long-row stride")


@pytest.mark.parametrize("N", [1000, 4096, 30000])
def test_deterministic(N):
    x = make_softmax_inputs(64, N, torch.bfloat16, seed=14)
    assert torch.equal(gpu_softmax(x), gpu_softmax(x))
