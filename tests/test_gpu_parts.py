"""GPU parity of the lift into the several-token GEMV's operand image
(lq_lift_parts) and of the GEMV on that image (lq_gemv_parts).

The image is decoded here on the CPU from its documented layout (per
512-position span: parts [step][part][half][lane][16 bytes], then int
exponents [step][token]; slot 8 q + t of a word is its position 4 t + q) and
compared value by value with the oracle's lifted activations; the layer
output through lq_lift_parts + lq_gemv_parts is compared with the oracle's
forward pass.

Bars: a decoded value carries 12 significant bits of the float32 lift (three
float8 E4M3 parts of 4 bits each under one power-of-two scale per 128
positions and token), so |dec - ref| <= 2^-11 |ref| + 2^-16 max|ref of the
token| bounds both the part rounding and the float32 lift sums; the layer
output keeps the GEMV's float32 bar of 1e-4 (relative to each token's
largest output).
"""
import numpy as np
import pytest
import torch

from bit_lifted_gemv_amd import lq, synth
from oracle import lq_oracle as O

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
SPAN_POS = 512
PART_BYTES = 4 * 3 * 64 * 32
SPAN_BYTES = PART_BYTES + 4 * 16 * 4


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lq.load_library()
    return torch.device("cuda:0")


def _banner(msg):
    print(msg, flush=True)


def _e4m3(b: np.ndarray) -> np.ndarray:
    """OCP float8 E4M3 (bias 7, no infinities) bytes -> float64."""
    b = b.astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    return sign * val


def decode_image(img: np.ndarray, K: int, B: int) -> np.ndarray:
    """[B][K] float64 values held by an lq_lift_parts image."""
    nsp = img.size // SPAN_BYTES
    spans = img.reshape(nsp, SPAN_BYTES)
    out = np.zeros((B, nsp * SPAN_POS), dtype=np.float64)
    parts = spans[:, :PART_BYTES].reshape(nsp, 4, 3, 2, 64, 16)      # [c][u][p][half][lane][byte]
    expo = spans[:, PART_BYTES:].copy().view(np.int32).reshape(nsp, 4, 16)   # [c][u][token]
    for u in range(4):
        for g in range(4):
            for h in range(2):
                lanes = 16 * (2 * (g & 1) + h) + np.arange(16)            # token n = lane % 16
                by = parts[:, u][:, :, g >> 1][:, :, lanes]               # [c][p][n][16]
                val = np.zeros((nsp, 16, 16))
                for p in range(3):
                    val += _e4m3(by[:, p]) * 2.0 ** (-4 * p)
                val *= 2.0 ** (-expo[:, u, :].astype(np.float64))[:, :, None]
                # byte 4 (2 qq + hh) + j: position 4 (4 hh + j) + 2 h + qq of word 4 g + u
                for qq in range(2):
                    for hh in range(2):
                        for j in range(4):
                            pos = 32 * (4 * g + u) + 4 * (4 * hh + j) + 2 * h + qq
                            col = np.arange(nsp) * SPAN_POS + pos
                            out[:, col] = val[:, :B, 4 * (2 * qq + hh) + j].T
    assert not out[:, K:].any(), "positions past K must be zero"
    return out[:, :K]


IMAGE_CASES = [  # (n, d, D, B, dtype): groups straddling spans, aligned groups,
    # d = 4 (most channels per span), d = 16 and 32, one and sixteen tokens,
    # ragged last span, whole and partial groups of eight spans
    (1024, 8, 19, 16, "bf16"), (2048, 8, 16, 6, "bf16"), (1280, 4, 10, 9, "f16"),
    (512, 16, 40, 16, "bf16"), (1024, 32, 64, 11, "f16"), (1536, 4, 4, 1, "f16"),
    (8192, 8, 19, 16, "bf16"),
]


@pytest.mark.parametrize("n,d,D,B,dt", IMAGE_CASES)
def test_lift_parts_image(dev, n, d, D, B, dt):
    _banner(f"lift parts n={n} D/d={D}/{d} B={B} {dt}")
    L = synth.make_layer(64, n, d, D, B, seed=n + D + B, dtype=dt, outlier_frac=0.01)
    M64, T64, _, a64 = O._inputs64(L.M, L.t_inv, L.s, L.a, dt)
    ref = O.lift(O.transform(a64, T64), M64, d, D)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    a = lq.to_torch_16(L.a, dt).to(dev)
    img = lq.lift_parts(a, dl.t_inv, dl.M, d, D).cpu().numpy()
    assert img.size == lq.lift_parts_size(L.K)
    got = decode_image(img, L.K, B)
    bound = 2.0 ** -11 * np.abs(ref) + 2.0 ** -16 * np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(got - ref)
    _banner(f"  worst err / bound {float((err / bound).max()):.3f}")
    assert (err <= bound).all()


LAYER_CASES = [  # (m, n, d, D, B, dtype)
    (500, 1024, 8, 19, 16, "bf16"), (257, 2048, 8, 16, 6, "bf16"), (130, 1280, 4, 10, 9, "f16"),
    (64, 512, 16, 40, 16, "bf16"), (96, 1024, 32, 64, 11, "f16"), (40, 4096, 8, 8, 3, "bf16"),
    (70, 1536, 4, 4, 1, "f16"), (300, 8192, 8, 19, 16, "bf16"),
]


@pytest.mark.parametrize("m,n,d,D,B,dt", LAYER_CASES)
def test_layer_through_parts(dev, m, n, d, D, B, dt):
    _banner(f"parts layer m={m} n={n} D/d={D}/{d} B={B} {dt}")
    L = synth.make_layer(m, n, d, D, B, seed=m + n + B, dtype=dt, outlier_frac=0.01)
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, d, D, dt)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(lq.to_torch_16(L.a, dt).to(dev), path="parts").cpu().numpy()
    e = O.rel_err_colmax(got, ref)
    _banner(f"  rel err {e:.3e}")
    assert e <= TOL_F32, e


def test_parts_deterministic_and_shared_workspace(dev):
    """Two shapes in turn on one stream (one workspace): each call equals its
    own repeat bit for bit."""
    res = []
    for (m, n, B) in [(300, 8192, 16), (64, 1024, 7), (300, 8192, 16)]:
        L = synth.make_layer(m, n, 8, 19, B, seed=5, dtype="bf16")
        dl = lq.DeviceLayer.from_synth(L, device=dev)
        res.append(dl.forward(lq.to_torch_16(L.a, "bf16").to(dev), path="parts").cpu())
    assert torch.equal(res[0], res[2])


CASES = [c for c in synth.all_cases() if 1 < c[3] <= 16]


@pytest.mark.parametrize("cfg,si,shape,B", CASES,
                         ids=[f"cfg{c.index}-{s[0]}x{s[1]}-B{b}" for c, _, s, b in CASES])
def test_full_size_case_through_parts(dev, cfg, si, shape, B):
    """The several-token workload cases at full size through the parts
    path, sampled rows (first and last 64 plus 96 random) against the oracle."""
    m, n = shape
    _banner(f"full parts {cfg.name} {m}x{n} B={B}")
    L = synth.make_case(cfg, si, B)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(lq.to_torch_16(L.a, L.dtype).to(dev), path="parts").cpu().numpy()
    rng = np.random.default_rng(si + B)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(m - 64, m),
                                     rng.choice(m, size=96, replace=False)]))
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, L.d, L.D, L.dtype, rows=rows)
    e = O.rel_err_colmax(got[:, rows], ref)
    _banner(f"  rel err {e:.3e}")
    assert e <= TOL_F32, e


def test_image_columns_past_B_are_zero(dev):
    """lq_lift_parts writes all 16 token columns, zero past B: the product on
    that image for more tokens than were lifted gives the lifted tokens'
    outputs unchanged and zero for the rest."""
    L = synth.make_layer(200, 2048, 8, 19, 5, seed=11, dtype="bf16")
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    img = lq.lift_parts(lq.to_torch_16(L.a, "bf16").to(dev), dl.t_inv, dl.M, 8, 19)
    five = lq.gemv_parts(dl.w, dl.s, img, L.K, 5).cpu()
    sixteen = lq.gemv_parts(dl.w, dl.s, img, L.K, 16).cpu()
    assert torch.equal(sixteen[:5], five)
    assert not sixteen[5:].abs().any()
