"""attn_bwd_noalloc (the backward for callers that cannot allocate: D lives
in the library's static device scratch instead of a caller workspace)
against attn_bwd, through the C ABI: two calls in a row, the second on a
smaller input, each bitwise equal to attn_bwd on the same inputs; plus the
size limit of the scratch."""
import pytest
import torch

from attn_inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_online_softmax_attn_amd as T
    T.lib()  # raises if libattn.so is missing: no silent fallback


def _both(B, H, N, d, causal, seed):
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, N, d, torch.bfloat16, seed=seed,
                                                   with_dout=True))
    scale = d ** -0.5
    o, lse = T.flash_attention_forward(q, k, v, causal, scale)
    ref = T.flash_attention_backward(q, k, v, o, lse, do, causal, scale)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    T.attn_bwd_noalloc(q, k, v, o, do, lse, got[0], got[1], got[2], causal, scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs"


def test_two_calls_second_smaller():
    print("[noalloc] call 1: B2 H16 N4096 d64 causal", flush=True)
    _both(2, 16, 4096, 64, True, seed=5)
    print("[noalloc] call 2: B1 H3 N777 d128 non-causal", flush=True)
    _both(1, 3, 777, 128, False, seed=6)


def test_size_limit():
    """B*H*N above 4194304 rows is refused before anything is launched."""
    import tiled_online_softmax_attn_amd as T
    dev = torch.device("cuda:0")
    x = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(16, device=dev)
    p = x.data_ptr()
    L = T.lib()
    # B*H*N = 4194305: one row too many (the pointers are never dereferenced)
    rc = L.attn_bwd_noalloc(p, p, p, p, p, lse.data_ptr(), p, p, p, 1, 5, 838861, 64, 1,
                            0.125, 1, None)
    assert rc == -9
