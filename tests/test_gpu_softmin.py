"""GPU parity of the soft-argmin objective that learns M (lq_softmin_grad)
and of the Adam step (lq_adam_update), through the C ABI, against the
float64 oracle (oracle/lq_codebook.py).

Bars: the kernels sum in float32 (chunks of at most 64 codes folded into
totals, samples in fixed slices).  Measured over the cases below the loss is
within 3e-7 relative and the gradient, whose terms partly cancel
(sum_t b_nt = 0 for every sample), within 2e-5 of its largest entry (the
large-T case); the tests allow 1e-5 and 1e-4, a wide margin that still fails
any dropped or mis-signed term (those move the result by O(1)).  Adam: 1e-6
relative, the oracle given the same float hyperparameters as the C ABI."""
import numpy as np
import pytest
import torch

from bit_lifted_gemv_amd import lq
from oracle import lq_codebook as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lq.load_library()
    return torch.device("cuda:0")


def _haar(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))[None, :]


CASES = [  # (d, D, N, T): one code bit, fewer codes than a slice, odd N,
    # T = 0 and a large T, the LQ-16/8 shape, d = D, D = 20 (XM = 24 registers)
    (1, 1, 300, 10.0), (2, 5, 257, 10.0), (4, 8, 1000, 10.0), (3, 10, 700, 0.0),
    (4, 8, 100, 100.0), (6, 12, 513, 10.0), (8, 16, 600, 10.0), (5, 5, 64, 10.0),
    (10, 20, 48, 10.0), (16, 18, 40, 10.0),
]


@pytest.mark.parametrize("d,D,N,T", CASES)
def test_softmin_loss_and_gradient(dev, d, D, N, T):
    print(f"softmin d={d} D={D} N={N} T={T}", flush=True)
    rng = np.random.default_rng(d * 1000 + D * 10 + N)
    M = (_haar(rng, D)[:d] * (0.9 if D > 1 else 0.8)).astype(np.float32)
    W = rng.standard_normal((N, d)).astype(np.float32)
    chunk = max(1, (1 << 22) // ((1 << D) * d))
    ref_loss, ref_g, _ = C.softmin_objective(W, M, T, chunk=chunk)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    loss, grad = lq.softmin_grad(t(W), t(M), T)
    torch.cuda.synchronize()
    loss = float(loss.cpu()[0])
    g = grad.cpu().numpy().astype(np.float64)
    rel_l = abs(loss - ref_loss) / abs(ref_loss)
    scale = np.abs(ref_g).max()
    rel_g = np.abs(g - ref_g).max() / scale if scale > 0 else np.abs(g).max()
    print(f"  loss rel err {rel_l:.2e}  grad err / max|grad| {rel_g:.2e}", flush=True)
    assert rel_l <= 1e-5
    if T == 0.0:
        assert np.abs(g).max() <= 1e-6
    else:
        assert rel_g <= 1e-4


def test_adam_update_matches_oracle(dev):
    rng = np.random.default_rng(3)
    M = rng.standard_normal((8, 16)).astype(np.float32)
    m1 = np.zeros_like(M)
    m2 = np.zeros_like(M)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    Mt, m1t, m2t = t(M), t(m1), t(m2)
    Mr, m1r, m2r = M.astype(np.float64), m1.astype(np.float64), m2.astype(np.float64)
    # the C ABI takes float hyperparameters: give the oracle the same values
    f32 = lambda x: float(np.float32(x))
    for step in (1, 2, 3):
        g = rng.standard_normal(M.shape).astype(np.float32)
        lq.adam_update(Mt, t(g), m1t, m2t, step, 0.01)
        Mr, m1r, m2r = C.adam_step(Mr, g.astype(np.float64), m1r, m2r, step, f32(0.01),
                                   f32(0.9), f32(0.999), f32(1e-8))
    torch.cuda.synchronize()
    np.testing.assert_allclose(Mt.cpu().numpy(), Mr, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(m2t.cpu().numpy(), m2r, rtol=1e-5, atol=1e-12)


def test_learning_on_the_gpu_lowers_objective_and_codebook_error(dev):
    """Adam on GPU gradients from the orthogonal start (LQ-8/4 shape): the
    soft objective falls and the hard nearest-point error of the learned M
    (measured by the oracle) is below the start's."""
    rng = np.random.default_rng(4)
    d, D = 4, 8
    M0 = _haar(rng, D)[:d].astype(np.float32)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    batches = [torch.randn((2048, d), generator=g, device=dev) for _ in range(60)]
    M, losses = lq.learn_m(torch.from_numpy(M0).to(dev), batches, T=10.0, lr=0.01)
    torch.cuda.synchronize()
    ls = [float(x.cpu()[0]) for x in losses]
    assert np.mean(ls[-10:]) < np.mean(ls[:5])
    Wt = np.random.default_rng(5).standard_normal((8000, d))
    _, e0, _ = C.encode_exhaustive(Wt, M0)
    _, e1, _ = C.encode_exhaustive(Wt, M.cpu().numpy())
    assert e1.mean() < e0.mean()
