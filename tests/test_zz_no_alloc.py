"""lq_gemv_noalloc against lq_gemv through the C ABI: the same kernels, so
the same float32 results bit for bit, on two calls in a row (the second with
a smaller input that reuses the scratch the first left behind), for the
one-token, few-token and several-token kernels."""
import numpy as np
import pytest
import torch

from bit_lifted_gemv_amd import lq, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lq.load_library()
    return torch.device("cuda:0")


def _case(dev, m, K, B, seed):
    rng = np.random.default_rng(seed)
    packed = synth.random_sign_words(rng, m, K, ldw=((K + 31) // 32 + 3) // 4 * 4)
    w = torch.from_numpy(packed.view(np.int32)).to(dev)
    s = torch.from_numpy(rng.uniform(0.01, 0.03, m).astype(np.float32)).to(dev)
    a = torch.from_numpy(rng.standard_normal((B, K)).astype(np.float32)).to(dev)
    return w, s, a


@pytest.mark.parametrize("B", [1, 4, 16])
def test_noalloc_matches_gemv_two_calls(dev, B):
    print(f"noalloc B={B}", flush=True)
    for (m, K), seed in (((8192, 68096), 1), ((700, 5120), 2)):   # second call smaller
        w, s, a = _case(dev, m, K, B, seed * 100 + B)
        want = lq.gemv(w, s, a, K)
        got = torch.full((B, m), float("nan"), device=dev)
        lq.gemv_noalloc(w, s, a, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (m, K, B)
