"""GPU parity of the decode-weights product (lq_gemm_decoded, through the C
ABI) against the float64 oracle's dense route (o = s * (W_hat T^-1 a), which
is this product written out).

Bar: the layer tolerance 2e-3 (e = max over tokens of max_i |o - o_ref| /
max_i |o_ref|).  The decoded weights W_hat are rounded once to float16
(relative 2^-11; s is applied to the float32 sums) and u = T^-1 a once to
float16 (2^-11) after the 16-bit input's own rounding; summed in float32
over n independent terms, the output error is about 2^-11 * sqrt(2/3) ~
4e-4 of the output scale, so 2e-3 keeps a 5x margin."""
import numpy as np
import pytest
import torch

from bit_lifted_gemv_amd import lq, synth
from oracle import lq_oracle as O

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lq.load_library()
    return torch.device("cuda:0")


def _up(x, dtype, dev):
    return lq.to_torch_16(x, dtype).to(dev)


CASES = [  # (m, n, d, D, B, dtype): LQ-40/16, LQ-19/8 (groups straddle words),
    # d = 10 groups across 128-blocks, odd D (partial last chunk), D = d,
    # D = 33 (a 1-sign last chunk), one token, ragged rows
    (256, 512, 16, 40, 130, "bf16"), (200, 1024, 8, 19, 40, "bf16"),
    (130, 1280, 10, 24, 17, "f16"), (64, 384, 3, 7, 33, "bf16"), (48, 512, 8, 8, 20, "f16"),
    (33, 256, 16, 33, 5, "bf16"), (17, 256, 8, 16, 1, "bf16"), (300, 2048, 8, 16, 64, "bf16"),
    (40, 640, 32, 70, 9, "bf16"), (24, 384, 48, 129, 3, "bf16"),
]


@pytest.mark.parametrize("m,n,d,D,B,dt", CASES)
def test_decoded_layer_small(dev, m, n, d, D, B, dt):
    print(f"decoded m={m} n={n} D/d={D}/{d} B={B} {dt}", flush=True)
    L = synth.make_layer(m, n, d, D, B, seed=m + n + B + 7, dtype=dt, outlier_frac=0.01)
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, d, D, dt)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(_up(L.a, dt, dev), path="decoded").cpu().numpy()
    e = O.rel_err_colmax(got, ref)
    print(f"  rel err {e:.3e}", flush=True)
    assert e <= TOL, e
    assert np.isfinite(got).all()


def test_decoded_lq40_16_full_size_sampled(dev):
    """The batch-512 workload (LQ-40/16, 8192 x 8192) on the decode-weights
    path, in the configuration the benchmark times, on sampled rows."""
    cfg = synth.CONFIGS[4]
    L = synth.make_case(cfg, 0, 512)
    print(f"decoded full {cfg.name} {L.m}x{L.n} B=512", flush=True)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(_up(L.a, L.dtype, dev), path="decoded").cpu().numpy()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(L.m - 64, L.m),
                                     rng.choice(L.m, 96, replace=False)]))
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, L.d, L.D, L.dtype, rows=rows)
    e = O.rel_err_colmax(got[:, rows], ref)
    print(f"  rel err {e:.3e}", flush=True)
    assert e <= TOL, e


def test_decoded_many_row_tiles(dev):
    """Many 64-row workgroup tiles (and a ragged last one) with a few
    tokens: every tile's rows land in the right output columns."""
    m, n, d, D, B = 2 * (1 << 27) // 4096 + 48, 4096, 8, 16, 24
    print(f"decoded chunked m={m} n={n}", flush=True)
    L = synth.make_layer(m, n, d, D, B, seed=5, dtype="bf16")
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(_up(L.a, "bf16", dev), path="decoded").cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, m, 997), np.arange(m - 40, m),
                                     np.arange(32768 - 8, 32768 + 8)]))
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, d, D, "bf16", rows=rows)
    e = O.rel_err_colmax(got[:, rows], ref)
    assert e <= TOL, e
