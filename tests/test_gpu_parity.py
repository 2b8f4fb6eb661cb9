"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars (written here, derived in the design notes):
  * sign pack / unpack: bit-exact.
  * layer output: e = max_b max_i |o - o_ref| / max_i |o_ref| <= 2e-3, the
    tolerance stated for 16-bit inputs.  The float32 GEMV path also has to
    stay under 1e-4 (float32 sums of at most ~7e4 terms of random sign
    typically lose ~sqrt(K) * 2^-24 ~ 2e-5 relative; 1e-4 leaves margin and
    still fails any dropped term or wrong sign).
  * lifted activations: float32 output within 1e-5 (relative to the token's
    largest value); 16-bit outputs within one unit of rounding of the float32
    value plus that.
"""
import numpy as np
import pytest
import torch

from bit_lifted_gemv_amd import lq, synth
from oracle import lq_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-3
# The GEMV carries each float32 activation by three float8 parts (12
# significant bits, a relative error of at most 2^-12 per value, independent
# across the K values of a row) and multiplies them by exact float4 signs on
# the matrix cores with float32 accumulation (about K/128 roundings of the
# running sum); the GEMM takes exact 16-bit operands: 1e-4 bounds both with
# a wide margin at every K here.
TOL_F32 = 1e-4
# lq_layer_b1 rounds each activation sum (8 terms) once to float16 after an
# exact power-of-two scaling: relative error <= 2^-11 per table entry,
# independent across the K/8 entries of a row, so the output error is about
# 2^-11/sqrt(3) ~ 3e-4 of the output scale; 1e-3 keeps a 3x margin.
TOL_LUT16 = 1e-3
# With 1 <= B <= 5 lq_gemv carries each activation by three float8 (E4M3)
# parts of 4 significant bits each, every part kept in the normal range by a
# power-of-two column scale per 1024-position slice: 12 significant bits,
# a relative error of at most 2^-12 per value (less than 2^-17 of the
# slice's largest value for the smallest ones), independent across K; the
# products with 0 / 1 sign nibbles are exact and summed in float32, and the
# slice's float32 activation sum turns them into the +-1 product.  Measured
# 1.5e-5 to 3e-5 on the workload shapes; the bar TOL_F32 covers it with
# margin.


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lq.load_library()
    return torch.device("cuda:0")


def _up(x, dtype, dev):
    return lq.to_torch_16(x, dtype).to(dev)


def _banner(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------- sign packing
@pytest.mark.parametrize("rows,K,extra", [(1, 1, 0), (3, 31, 1), (5, 33, 0), (7, 100, 2),
                                          (64, 3072, 0), (4, 68096, 0), (9, 513, 3)])
def test_pack_unpack_bit_exact(dev, rows, K, extra):
    _banner(f"pack rows={rows} K={K}")
    rng = np.random.default_rng(K * 31 + rows)
    sg = synth.random_signs_i8(rng, rows, K)
    sg[rng.random(sg.shape) < 0.05] = 0                      # zeros pack as 0 bits
    ldw = (K + 31) // 32 + extra
    want = O.pack_signs_ref(sg, ldw)
    got = lq.pack_signs(torch.from_numpy(sg).to(dev), ldw=ldw).cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, want)
    back = lq.unpack_signs(torch.from_numpy(want.view(np.int32)).to(dev), K).cpu().numpy()
    np.testing.assert_array_equal(back, O.signs_from_packed(want, K))


def test_pack_empty_is_noop(dev):
    L = lq.lib()
    assert L.lq_pack_signs(None, 0, 0, 0, None, 0, None) == 0
    assert L.lq_unpack_signs(None, 0, 5, 1, None, 5, None) == 0


# ----------------------------------------------------------------- lift
LIFT_CASES = [  # (n, d, D, B, act dtype)
    (1280, 10, 24, 1, "f16"), (640, 10, 24, 3, "bf16"), (1024, 8, 19, 1, "bf16"),
    (512, 8, 20, 16, "bf16"), (256, 16, 40, 33, "bf16"), (384, 8, 16, 4, "f16"),
    (384, 3, 7, 2, "bf16"), (256, 64, 128, 1, "f16"), (1280, 40, 100, 2, "bf16"),
    (640, 32, 80, 20, "f16"),
    # 8 tokens and more (4 and more when n >= 12288) with a and T^-1 of one
    # 16-bit type and d | 128 take the matrix-core lift: ragged token tiles,
    # D % 8 != 0 (a_hat through LDS), d = 4 .. 32
    (1024, 8, 19, 130, "bf16"), (512, 4, 9, 17, "f16"), (384, 16, 40, 257, "f16"),
    (2048, 8, 20, 64, "bf16"), (256, 32, 64, 40, "bf16"), (1024, 16, 40, 8, "f16"),
    (2048, 4, 9, 9, "bf16"), (16384, 8, 19, 4, "bf16"), (12288, 32, 80, 5, "f16"),
    (12160, 8, 19, 4, "bf16"),
]


@pytest.mark.parametrize("n,d,D,B,dt", LIFT_CASES)
def test_lift_float32(dev, n, d, D, B, dt):
    _banner(f"lift n={n} d={d} D={D} B={B} {dt}")
    L = synth.make_layer(8, n, d, D, B, seed=n + d + D + B, dtype=dt)
    ref = O.lift(O.transform(O.decode(L.a, dt), O.decode(L.t_inv, dt)), L.M, d, D)
    got = lq.lift(_up(L.a, dt, dev), _up(L.t_inv, dt, dev), torch.from_numpy(L.M).to(dev), d, D,
                  out_dtype=torch.float32).cpu().numpy()
    err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert err.max() <= 1e-5, err


@pytest.mark.parametrize("odt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("n,d,D,B", [(1024, 8, 19, 5), (1024, 8, 19, 70), (512, 16, 40, 300)])
def test_lift_16bit_outputs(dev, odt, n, d, D, B):
    L = synth.make_layer(4, n, d, D, B, seed=3, dtype="bf16")
    ref = O.lift(O.transform(O.decode(L.a, "bf16"), O.decode(L.t_inv, "bf16")), L.M, d, D)
    got = lq.lift(_up(L.a, "bf16", dev), _up(L.t_inv, "bf16", dev),
                  torch.from_numpy(L.M).to(dev), d, D, out_dtype=odt).float().cpu().numpy()
    u = 2.0 ** -11 if odt == torch.float16 else 2.0 ** -8     # unit roundoff of the output
    bound = u * np.abs(ref) + 1e-5 * np.abs(ref).max(axis=1, keepdims=True)
    assert (np.abs(got - ref) <= bound).all()


# ----------------------------------------------------------------- lift, Kronecker whitening
KRON_CASES = [  # (n, n1, d, D, B, act dtype): n2 = n / n1 <= 128, n2 % d == 0
    (1280, 16, 10, 24, 1, "f16"), (512, 4, 8, 20, 3, "bf16"), (8192, 64, 16, 40, 1, "bf16"),
    (8192, 64, 16, 40, 17, "f16"), (28672, 224, 8, 19, 1, "bf16"), (4096, 32, 8, 20, 5, "f32"),
    (384, 3, 4, 9, 2, "bf16"), (960, 12, 8, 16, 7, "bf16"), (6, 2, 3, 5, 1, "f32"),
    # 16 | n1 and 16 | n2 with d = 1, 2, 4 at a few tokens (n1 = 48: three
    # 16-row blocks; n2 = 16: one column block)
    (3072, 48, 4, 12, 2, "f16"), (2048, 16, 1, 3, 8, "bf16"), (1024, 64, 2, 5, 1, "f32"),
    # 64 tokens and more with small factors take the single-launch kernel:
    # the prefill-scale shape, a ragged last token group, D % 4 != 0, float32
    # activations, several tokens per workgroup
    (8192, 64, 16, 40, 512, "bf16"), (2048, 16, 8, 19, 300, "f16"),
    (4096, 32, 8, 19, 70, "bf16"), (2048, 16, 4, 9, 65, "f16"), (1024, 16, 8, 20, 300, "f32"),
    # 64 tokens and more that the single launch cannot take run the two
    # launches with several column blocks per wave and a ragged last column
    # slab: factors too large for LDS (n1 = 224), D > 64, d > 32
    (28672, 224, 8, 19, 96, "bf16"), (8192, 64, 16, 80, 512, "bf16"),
    (8192, 64, 64, 128, 100, "f16"),
]


def _kron_inputs(n, n1, d, D, B, dt, seed):
    rng = np.random.default_rng(seed)
    f = synth.make_kron_factors(n, d, seed, n1=n1)
    M = (rng.standard_normal((d, D)) / np.sqrt(D)).astype(np.float32)
    a = synth.to_storage(rng.standard_normal((B, n)).astype(np.float32), dt)
    return f, M, a


@pytest.mark.parametrize("n,n1,d,D,B,dt", KRON_CASES)
def test_lift_kron_float32(dev, n, n1, d, D, B, dt):
    _banner(f"lift_kron n={n} n1={n1} d={d} D={D} B={B} {dt}")
    f, M, a = _kron_inputs(n, n1, d, D, B, dt, n + n1 + B)
    ref = O.lift_kron(a, f.s1, f.p1_inv, f.p2_inv, f.s2, M, d, D, dt)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    got = lq.lift_kron(_up(a, dt, dev), t(f.s1), t(f.p1_inv), t(f.p2_inv), t(f.s2), t(M), d, D,
                       out_dtype=torch.float32).cpu().numpy()
    err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert err.max() <= 1e-5, err


@pytest.mark.parametrize("odt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("B", [9, 96])   # two launches / the single-launch kernel
def test_lift_kron_16bit_outputs(dev, odt, B):
    n, n1, d, D = 8192, 64, 16, 40
    f, M, a = _kron_inputs(n, n1, d, D, B, "bf16", 77)
    ref = O.lift_kron(a, f.s1, f.p1_inv, f.p2_inv, f.s2, M, d, D, "bf16")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    got = lq.lift_kron(_up(a, "bf16", dev), t(f.s1), t(f.p1_inv), t(f.p2_inv), t(f.s2), t(M), d, D,
                       out_dtype=odt).float().cpu().numpy()
    u = 2.0 ** -11 if odt == torch.float16 else 2.0 ** -8
    bound = u * np.abs(ref) + 1e-5 * np.abs(ref).max(axis=1, keepdims=True)
    assert (np.abs(got - ref) <= bound).all()


def test_layer_with_kron_whitening_70b_up(dev):
    """The 70B-class up projection (28672 x 8192, LQ-19/8) with the Kronecker
    whitening in place of the block-diagonal T^-1: lift_kron then the
    one-token GEMV, against the oracle's reconstruct route on sampled rows."""
    cfg = synth.CONFIGS[3]
    L = synth.make_case(cfg, 0, 1)
    f = synth.make_kron_factors(L.n, L.d, 123)
    _banner(f"layer kron {L.m}x{L.n} n1={f.n1}")
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    al = lq.lift_kron(_up(L.a, L.dtype, dev), t(f.s1), t(f.p1_inv), t(f.p2_inv), t(f.s2), dl.M,
                      L.d, L.D, out_dtype=torch.float32)
    got = lq.gemv(dl.w, dl.s, al, L.K).cpu().numpy()
    rows = _sample_rows(L.m, np.random.default_rng(5))
    ref = O.forward_kron(L.packed, L.K, L.M, f.s1, f.p1_inv, f.p2_inv, f.s2, L.s, L.a, L.d, L.D,
                         L.dtype, rows=rows)
    assert O.rel_err_colmax(got[:, rows], ref) <= TOL_F32


# ----------------------------------------------------------------- GEMV (lifted product)
GEMV_CASES = [  # (m, K, B): ragged rows, slices and token groups
    (1, 4, 1), (63, 512, 1), (65, 516, 1), (200, 1544, 2), (129, 3072, 3), (300, 2048, 4),
    (77, 1000, 5), (1000, 4100, 16), (4096, 10240, 1), (520, 9216, 7), (200, 40960, 1),
    # one token: a single slice (no split), a 4-position last slice, a ragged
    # 8-row granule, and more slices than workgroups (ranges over > 2 slices)
    (1000, 1024, 1), (37, 1028, 1), (8193, 2048, 1), (64, 300000, 1),
    (300, 41984, 1),    # 41 slices: one past the one-launch kernel's limit at one token
]


@pytest.mark.parametrize("m,K,B", GEMV_CASES)
def test_gemv_lifted_product(dev, m, K, B):
    _banner(f"gemv m={m} K={K} B={B}")
    rng = np.random.default_rng(m * 7 + K + B)
    ldw = ((K + 31) // 32 + 3) // 4 * 4
    packed = synth.random_sign_words(rng, m, K, ldw=ldw)
    al = rng.standard_normal((B, K)).astype(np.float32)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    ref = O.lifted_product(packed, K, al, s)
    got = lq.gemv(torch.from_numpy(packed.view(np.int32)).to(dev), torch.from_numpy(s).to(dev),
                  torch.from_numpy(al).to(dev), K).cpu().numpy()
    e = O.rel_err_colmax(got, ref)
    assert e <= TOL_F32, e


F4_CASES = [  # (m, K, B): 2..5 tokens on the float4-sign / float8-part matrix cores
    (16, 1024, 2),      # one granule, one slice: no partial sums
    (17, 1028, 3),      # a ragged row tile and a 4-position last slice
    (1000, 4100, 5),    # five tokens (15 of 16 columns), ragged slices
    (300, 20480, 4),    # a workgroup range over several slices
    (64, 300000, 2),    # more slices than workgroups: ranges over > 2 slices
    (4096, 10240, 3), (2050, 12288, 4),
]


@pytest.mark.parametrize("m,K,B", F4_CASES)
def test_gemv_few_tokens_float8_parts(dev, m, K, B):
    """2 <= B <= 5 on the float4 / float8 matrix cores, with outlier channels
    (1 % x 20), a slice of zeros, and slices of tiny and huge activations (the
    per-slice column scales keep every part normal)."""
    _banner(f"gemv f4 m={m} K={K} B={B}")
    rng = np.random.default_rng(m * 13 + K + B)
    ldw = ((K + 31) // 32 + 3) // 4 * 4
    packed = synth.random_sign_words(rng, m, K, ldw=ldw)
    al = rng.standard_normal((B, K)).astype(np.float32)
    al[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= 20
    if K > 3 * 1024:
        al[0, 1024:2048] = 0
        al[-1, 2048:3072] *= np.float32(1e-30)
        al[0, 3072:4096] *= np.float32(1e25)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    got = lq.gemv(torch.from_numpy(packed.view(np.int32)).to(dev), torch.from_numpy(s).to(dev),
                  torch.from_numpy(al).to(dev), K).cpu().numpy()
    ref = O.lifted_product(packed, K, al, s)
    e = O.rel_err_colmax(got, ref)
    _banner(f"  rel err {e:.3e}")
    assert np.isfinite(got).all()
    assert e <= TOL_F32, e


F4M_CASES = [  # (m, K, B): 6..16 tokens, the float8 parts as column blocks
    (1, 4, 6),          # one row, one word
    (65, 516, 16),      # a ragged tile and a 4-position last word
    (513, 20480, 11),   # one row past a workgroup's 512
    (520, 9216, 7),
    (8192, 2048, 16),   # many row groups, one span pair per split
    (64, 300000, 9),    # one row group: as many splits as span pairs allow
    (4096, 28672, 16),
]


@pytest.mark.parametrize("m,K,B", F4M_CASES)
def test_gemv_many_tokens_float8_parts(dev, m, K, B):
    """6 <= B <= 16 with the float8 parts as column blocks, with outlier
    channels (1 % x 20), a run of zeros, and runs of tiny and huge activations
    (the per-step exponents keep every part normal)."""
    _banner(f"gemv f4m m={m} K={K} B={B}")
    rng = np.random.default_rng(m * 17 + K + B)
    ldw = ((K + 31) // 32 + 3) // 4 * 4
    packed = synth.random_sign_words(rng, m, K, ldw=ldw)
    al = rng.standard_normal((B, K)).astype(np.float32)
    al[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= 20
    if K > 3 * 1024:
        al[0, 1024:2048] = 0
        al[-1, 2048:3072] *= np.float32(1e-30)
        al[0, 3072:4096] *= np.float32(1e25)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    got = lq.gemv(torch.from_numpy(packed.view(np.int32)).to(dev), torch.from_numpy(s).to(dev),
                  torch.from_numpy(al).to(dev), K).cpu().numpy()
    ref = O.lifted_product(packed, K, al, s)
    e = O.rel_err_colmax(got, ref)
    _banner(f"  rel err {e:.3e}")
    assert np.isfinite(got).all()
    assert e <= TOL_F32, e


F4M_LOOP_CASES = [  # (m, K, B): batches of four row tiles per workgroup
    (36864, 4096, 11),    # one split, 12 tiles per workgroup: 3 batches (odd)
    (65536, 4096, 16),    # one split, 16 tiles per workgroup: 4 batches (even)
    (8192, 65536, 16),    # 16 splits, 32 tiles per workgroup: 8 batches
    (12288, 131072, 6),   # 32 splits, the cap of 84 tiles per workgroup
]


@pytest.mark.parametrize("m,K,B", F4M_LOOP_CASES)
def test_gemv_many_tokens_batch_loops(dev, m, K, B):
    """The many-token product with several batches of row tiles per
    workgroup (both parities of the batch count, the loop over pairs of
    batches, the cap on tiles per workgroup), checked on sampled rows."""
    _banner(f"gemv f4m batches m={m} K={K} B={B}")
    rng = np.random.default_rng(m + K + B)
    ldw = ((K + 31) // 32 + 3) // 4 * 4
    packed = synth.random_sign_words(rng, m, K, ldw=ldw)
    al = rng.standard_normal((B, K)).astype(np.float32)
    al[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= 20
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    got = lq.gemv(torch.from_numpy(packed.view(np.int32)).to(dev), torch.from_numpy(s).to(dev),
                  torch.from_numpy(al).to(dev), K).cpu().numpy()
    rows = _sample_rows(m, np.random.default_rng(m))
    ref = O.lifted_product(packed[rows], K, al, s[rows])
    e = O.rel_err_colmax(got[:, rows], ref)
    _banner(f"  rel err {e:.3e}")
    assert np.isfinite(got).all()
    assert e <= TOL_F32, e


ROWS_CASES = [  # (m, K, B) on the one-launch kernel (every slice in one workgroup's LDS)
    (1, 4, 1),          # one row, one 4-position slice
    (4100, 20480, 1),   # 20 slices; a last workgroup of one row tile
    (2100, 40960, 1),   # 40 slices, the most one token takes
    (4097, 3072, 1),    # a ragged last row tile of one row
    (300, 16384, 2),    # 16 slices, the most two tokens take
    (33, 7200, 3),      # a ragged last slice
    (1000, 8192, 5),    # 8 slices, the most five tokens take
    (16, 1024, 4),      # one granule
]


@pytest.mark.parametrize("m,K,B", ROWS_CASES)
def test_gemv_one_launch(dev, m, K, B):
    """The one-launch kernel (no workspace) at its boundaries, with the same
    outliers, zero slice and tiny / huge slices as the slice-major cases; the
    precision is that of the float8 parts for every token count."""
    _banner(f"gemv one-launch m={m} K={K} B={B}")
    assert lq.gemv_workspace_size(m, K, B) == 0, "shape expected on the one-launch kernel"
    rng = np.random.default_rng(m * 11 + K + B)
    ldw = ((K + 31) // 32 + 3) // 4 * 4
    packed = synth.random_sign_words(rng, m, K, ldw=ldw)
    al = rng.standard_normal((B, K)).astype(np.float32)
    al[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= 20
    if K > 3 * 1024:
        al[0, 1024:2048] = 0
        al[-1, 2048:3072] *= np.float32(1e-30)
        al[0, 3072:4096] *= np.float32(1e25)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    got = lq.gemv(torch.from_numpy(packed.view(np.int32)).to(dev), torch.from_numpy(s).to(dev),
                  torch.from_numpy(al).to(dev), K).cpu().numpy()
    ref = O.lifted_product(packed, K, al, s)
    e = O.rel_err_colmax(got, ref)
    _banner(f"  rel err {e:.3e}")
    assert np.isfinite(got).all()
    assert e <= TOL_F32, e


def test_gemv_few_tokens_scaling_is_exact(dev):
    """2..5 tokens: the float8 parts are formed after a power-of-two scaling
    chosen per slice, so scaling a token by 2^k scales its outputs by exactly
    2^k, and the tokens do not affect each other."""
    _banner("gemv f4 power-of-two scaling")
    rng = np.random.default_rng(19)
    m, K = 700, 5120
    packed = synth.random_sign_words(rng, m, K)
    w = torch.from_numpy(packed.view(np.int32)).to(dev)
    sd = torch.from_numpy(rng.uniform(0.01, 0.03, m).astype(np.float32)).to(dev)
    al = rng.standard_normal((4, K)).astype(np.float32)
    base = lq.gemv(w, sd, torch.from_numpy(al).to(dev), K).cpu().numpy()
    scaled = al.copy()
    scaled[1] = np.ldexp(al[1], 60)
    scaled[3] = np.ldexp(al[3], -60)
    got = lq.gemv(w, sd, torch.from_numpy(scaled).to(dev), K).cpu().numpy()
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[2], base[2])
    assert np.array_equal(got[1], np.ldexp(base[1], 60))
    assert np.array_equal(got[3], np.ldexp(base[3], -60))


@pytest.mark.parametrize("B", [1, 3, 16])
def test_gemv_largest_weight_buffer(dev, B):
    """The largest weight matrix one call accepts, m * ldw * 4 = 2^30 bytes
    (4096 rows of 2^21 lifted positions: 32-bit buffer offsets up to their
    limit, 2048 slices for one token; at 16 tokens 512 splits of K and the
    cap on row tiles per workgroup), checked on sampled rows.  The signs are
    drawn on the device by torch's seeded generator."""
    _banner(f"gemv largest weights 4096 x 2^21 B={B}")
    m, K = 4096, 1 << 21
    ldw = K // 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(77 + B)
    w = torch.randint(-(1 << 31), 1 << 31, (m, ldw), dtype=torch.int64, device=dev,
                      generator=gen).to(torch.int32)
    rng = np.random.default_rng(78 + B)
    al = rng.standard_normal((B, K)).astype(np.float32)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    got = lq.gemv(w, torch.from_numpy(s).to(dev), torch.from_numpy(al).to(dev), K).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(3), np.arange(m - 3, m),
                                     rng.choice(m, size=6, replace=False)]))
    packed = w[torch.from_numpy(rows).to(dev)].cpu().numpy().view(np.uint32)
    ref = O.lifted_product(packed, K, al, s[rows])
    e = O.rel_err_colmax(got[:, rows], ref)
    _banner(f"  rel err {e:.3e}")
    assert e <= TOL_F32, e
    assert np.isfinite(got).all()


def test_gemv_deterministic(dev):
    rng = np.random.default_rng(1)
    m, K = 3000, 19456
    packed = synth.random_sign_words(rng, m, K)
    al = torch.from_numpy(rng.standard_normal((1, K)).astype(np.float32)).to(dev)
    w = torch.from_numpy(packed.view(np.int32)).to(dev)
    s = torch.ones(m, device=dev)
    o1 = lq.gemv(w, s, al, K)
    o2 = lq.gemv(w, s, al, K)
    assert torch.equal(o1, o2)


def test_gemv_token_counts_share_a_workspace(dev):
    """Calls with one m and different B (different kernels and splits) run on
    one workspace, each over what the previous call left in it."""
    _banner("gemv B = 1, 4, 16, 1, 2, 7, 1 on one workspace")
    rng = np.random.default_rng(5)
    m, K = 2050, 12288
    packed = synth.random_sign_words(rng, m, K)
    w = torch.from_numpy(packed.view(np.int32)).to(dev)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    sd = torch.from_numpy(s).to(dev)
    for B in (1, 4, 16, 1, 2, 7, 1):
        al = rng.standard_normal((B, K)).astype(np.float32)
        got = lq.gemv(w, sd, torch.from_numpy(al).to(dev), K).cpu().numpy()
        assert O.rel_err_colmax(got, O.lifted_product(packed, K, al, s)) <= TOL_F32, B


def test_gemv_all_ones_closed_form(dev):
    """All signs +1 (and all -1): out = +-s * sum_k a_lift[k]."""
    m, K = 130, 2560
    al = np.random.default_rng(2).standard_normal((2, K)).astype(np.float32)
    s = np.linspace(0.5, 1.5, m).astype(np.float32)
    for fill, sign in ((0xFFFFFFFF, 1.0), (0, -1.0)):
        packed = np.full((m, K // 32), fill, dtype=np.uint32)
        got = lq.gemv(torch.from_numpy(packed.view(np.int32)).to(dev),
                      torch.from_numpy(s).to(dev), torch.from_numpy(al).to(dev), K).cpu().numpy()
        want = sign * s[None, :] * al.astype(np.float64).sum(axis=1)[:, None]
        assert O.rel_err_colmax(got, want) <= TOL_F32


def test_gemv_one_token_scaling_is_exact(dev):
    """One token: the float8 parts are formed from activations scaled by a
    power of two chosen from their range, so scaling a_lift by 2^k scales
    every output by exactly 2^k (no overflow, no loss for tiny or huge
    activations), and the all-ones closed form holds."""
    _banner("gemv B=1 power-of-two scaling")
    rng = np.random.default_rng(9)
    m, K = 700, 5120
    packed = synth.random_sign_words(rng, m, K)
    w = torch.from_numpy(packed.view(np.int32)).to(dev)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    sd = torch.from_numpy(s).to(dev)
    al = rng.standard_normal((1, K)).astype(np.float32)
    base = lq.gemv(w, sd, torch.from_numpy(al).to(dev), K).cpu().numpy()
    assert O.rel_err_colmax(base, O.lifted_product(packed, K, al, s)) <= TOL_F32
    for k in (-100, 100):
        got = lq.gemv(w, sd, torch.from_numpy(np.ldexp(al, k)).to(dev), K).cpu().numpy()
        assert np.array_equal(got, np.ldexp(base, k)), k
    for fill, sign in ((0xFFFFFFFF, 1.0), (0, -1.0)):
        ones = np.full((m, K // 32), fill, dtype=np.uint32)
        got = lq.gemv(torch.from_numpy(ones.view(np.int32)).to(dev), sd,
                      torch.from_numpy(al).to(dev), K).cpu().numpy()
        want = sign * s[None, :] * al.astype(np.float64).sum(axis=1)[:, None]
        assert O.rel_err_colmax(got, want) <= TOL_F32


# ----------------------------------------------------------------- GEMM
GEMM_CASES = [  # (m, K, B, extra words of row stride)
    (128, 256, 128, 0), (200, 520, 130, 0), (33, 64, 1, 0), (1000, 2048, 300, 0),
    (256, 20480, 64, 0),
    (129, 384, 257, 0),    # an odd number of 128-position steps; ragged row and token tiles
    (70, 40, 5, 0),        # K below one step, odd word stride (ldw = 2)
    (300, 1000, 200, 3),   # K % 128 != 0, padded rows (ldw = 35)
    (1030, 4096, 129, 1),  # several row tiles with a ragged tail, one token past a tile
]


@pytest.mark.parametrize("odt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("m,K,B,pad", GEMM_CASES)
def test_gemm_lifted_product(dev, m, K, B, pad, odt):
    _banner(f"gemm m={m} K={K} B={B} pad={pad} {odt}")
    rng = np.random.default_rng(m + K + B)
    ldw = (K + 31) // 32 + pad
    packed = synth.random_sign_words(rng, m, K, ldw=ldw)
    # bits past K and padding words hold garbage that must not reach the sums
    tail = rng.integers(0, 2**32, size=(m, ldw - K // 32), dtype=np.uint64).astype(np.uint32)
    if K % 32:
        tail[:, 0] &= np.uint32(~((1 << (K % 32)) - 1) & 0xFFFFFFFF)
    packed[:, K // 32:] |= tail
    al = torch.from_numpy(rng.standard_normal((B, K)).astype(np.float32)).to(odt)
    s = rng.uniform(0.01, 0.03, m).astype(np.float32)
    # the oracle sees exactly the stored 16-bit activations
    ref = O.lifted_product(packed, K, al.float().numpy(), s)
    got = lq.gemm(torch.from_numpy(packed.view(np.int32)).to(dev), torch.from_numpy(s).to(dev),
                  al.to(dev), K).cpu().numpy()
    e = O.rel_err_colmax(got, ref)
    assert e <= 1e-4, e   # operands are exact; float32 accumulation only


def test_gemm_longest_lifted_dimension(dev):
    """K = 2^22 (the largest lifted dimension lq_gemm accepts: 16384 steps of
    256 positions), two row tiles and one token tile, checked on sampled rows
    against the oracle.  Signs and activations are drawn on the device by
    torch's seeded generator."""
    _banner("gemm K = 2^22")
    m, K, B = 160, 1 << 22, 16
    ldw = K // 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(91)
    w = torch.randint(-(1 << 31), 1 << 31, (m, ldw), dtype=torch.int64, device=dev,
                      generator=gen).to(torch.int32)
    al = torch.randn((B, K), device=dev, generator=gen).to(torch.float16)
    s = torch.rand(m, device=dev, generator=gen) * 0.02 + 0.01
    got = lq.gemm(w, s, al, K).cpu().numpy()
    rows = np.array([0, 1, 127, 128, 129, 158, 159])
    packed = w[torch.from_numpy(rows).to(dev)].cpu().numpy().view(np.uint32)
    ref = O.lifted_product(packed, K, al.float().cpu().numpy(), s.cpu().numpy()[rows])
    e = O.rel_err_colmax(got[:, rows], ref)
    _banner(f"  rel err {e:.3e}")
    assert e <= 1e-4, e   # operands are exact; float32 accumulation only


def test_gemm_widest_row_stride(dev):
    """ldw = 2^22 words (the largest row stride lq_gemm accepts: the 128 rows
    of a tile span 2^31 bytes, the top of the 32-bit buffer range), a short
    K and garbage in every padding word, two row tiles and a ragged token
    tile, checked on sampled rows against the oracle."""
    _banner("gemm ldw = 2^22")
    m, K, B = 130, 512, 40
    ldw = 1 << 22
    gen = torch.Generator(device=dev)
    gen.manual_seed(93)
    w = torch.randint(-(1 << 31), 1 << 31, (m, ldw), dtype=torch.int64, device=dev,
                      generator=gen).to(torch.int32)
    al = torch.randn((B, K), device=dev, generator=gen).to(torch.bfloat16)
    s = torch.rand(m, device=dev, generator=gen) * 0.02 + 0.01
    got = lq.gemm(w, s, al, K).cpu().numpy()
    rows = np.array([0, 63, 127, 128, 129])
    packed = w[torch.from_numpy(rows).to(dev), : K // 32].cpu().numpy().view(np.uint32)
    ref = O.lifted_product(packed, K, al.float().cpu().numpy(), s.cpu().numpy()[rows])
    e = O.rel_err_colmax(got[:, rows], ref)
    _banner(f"  rel err {e:.3e}")
    assert e <= 1e-4, e


def test_gemm_one_hot_unpacks_signs_exactly(dev):
    """D = d, M = I, T^-1 = I, s = 1, tokens = identity columns: the GEMM
    output is the +-1 sign matrix itself, bit for bit."""
    m, n = 200, 256
    L = synth.make_layer(m, n, 4, 4, 1, seed=5, identity_t=True)
    eye = np.eye(n, dtype=np.float32)
    dl = lq.DeviceLayer(L.packed, np.eye(4, dtype=np.float32), L.t_inv, np.ones(m, np.float32),
                        4, 4, n, "bf16", device=dev)
    for gdt in (torch.float16, torch.bfloat16):
        out = dl.forward(torch.from_numpy(eye).to(dev).to(torch.bfloat16), gemm_dtype=gdt,
                         path="gemm").cpu().numpy()
        np.testing.assert_array_equal(out, O.signs_from_packed(L.packed, n).T.astype(np.float32))


# ----------------------------------------------------------------- whole layer
def test_integer_special_case_exact(dev):
    """D = d, M = I, T^-1 = I, s = 1, small-integer activations: exact integers."""
    m, n, B = 300, 1024, 3
    L = synth.make_layer(m, n, 8, 8, B, seed=6, identity_t=True)
    a_int = np.random.default_rng(4).integers(-20, 21, (B, n)).astype(np.float32)
    a = synth.to_storage(a_int, "bf16")
    dl = lq.DeviceLayer(L.packed, np.eye(8, dtype=np.float32), L.t_inv, np.ones(m, np.float32),
                        8, 8, n, "bf16", device=dev)
    want = O.forward(L.packed, n, np.eye(8, dtype=np.float32), L.t_inv, np.ones(m, np.float32), a,
                     8, 8, "bf16")
    for path in ("gemv", "gemm"):
        got = dl.forward(_up(a, "bf16", dev), path=path).cpu().numpy()
        np.testing.assert_array_equal(got, want)


LAYER_CASES = [  # (m, n, d, D, B, dtype): small layers the oracle does in full
    (130, 1280, 10, 24, 1, "f16"), (257, 1024, 8, 20, 1, "bf16"), (96, 2048, 8, 16, 4, "bf16"),
    (500, 1024, 8, 19, 16, "bf16"), (256, 512, 16, 40, 130, "bf16"),
]


@pytest.mark.parametrize("m,n,d,D,B,dt", LAYER_CASES)
def test_layer_small(dev, m, n, d, D, B, dt):
    _banner(f"layer m={m} n={n} D/d={D}/{d} B={B}")
    L = synth.make_layer(m, n, d, D, B, seed=m + n + B, dtype=dt, outlier_frac=0.01)
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, d, D, dt)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(_up(L.a, dt, dev)).cpu().numpy()
    e = O.rel_err_colmax(got, ref)
    assert e <= TOL, e
    if B <= 16:
        assert e <= TOL_F32, e


def _sample_rows(m, rng, k=96):
    head = np.arange(min(64, m))
    tail = np.arange(max(0, m - 64), m)
    mid = rng.choice(m, size=min(k, m), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


CASES = synth.all_cases()


@pytest.mark.parametrize("cfg,si,shape,B", CASES,
                         ids=[f"cfg{c.index}-{s[0]}x{s[1]}-B{b}" for c, _, s, b in CASES])
def test_full_size_case(dev, cfg, si, shape, B):
    """Every workload case at its full size, in the configuration the
    benchmark runs, checked on sampled rows (first and last 64 rows plus 96
    random ones) against the oracle."""
    m, n = shape
    _banner(f"full {cfg.name} {m}x{n} B={B}")
    L = synth.make_case(cfg, si, B)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    got = dl.forward(_up(L.a, L.dtype, dev)).cpu().numpy()
    rows = _sample_rows(m, np.random.default_rng(si + B))
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, L.d, L.D, L.dtype, rows=rows)
    e = O.rel_err_colmax(got[:, rows], ref)
    _banner(f"  rel err {e:.3e}")
    assert e <= TOL, e
    assert np.isfinite(got).all()


FUSED_CASES = [  # (m, n, d, D, dtype): groups straddling 128-blocks (d = 10), one
    # slice (K <= 1024: no reduction), d = D, d = 64 (the most channels behind
    # a slice), float32 and float16 inputs, ragged rows
    (130, 1280, 10, 24, "f16"), (257, 1024, 8, 20, "bf16"), (96, 2048, 8, 16, "bf16"),
    (64, 384, 3, 7, "bf16"), (33, 256, 4, 4, "bf16"), (50, 4096, 8, 8, "f16"),
    (70, 1280, 64, 64, "bf16"), (41, 1024, 16, 40, "f32"), (300, 8192, 8, 19, "bf16"),
]


@pytest.mark.parametrize("m,n,d,D,dt", FUSED_CASES)
def test_layer_b1_fused(dev, m, n, d, D, dt):
    """The one-token layer with the lift inside the GEMV against the oracle,
    and against the unfused path (lift, then the GEMV) on the same inputs."""
    _banner(f"fused layer m={m} n={n} D/d={D}/{d} {dt}")
    L = synth.make_layer(m, n, d, D, 1, seed=m + n + d, dtype=dt, outlier_frac=0.01)
    ref = O.forward(L.packed, L.K, L.M, L.t_inv, L.s, L.a, d, D, dt)
    dl = lq.DeviceLayer.from_synth(L, device=dev)
    a = _up(L.a, dt, dev)
    fused = dl.forward(a, path="fused").cpu().numpy()
    split = dl.forward(a, path="gemv").cpu().numpy()
    e = O.rel_err_colmax(fused, ref)
    _banner(f"  rel err {e:.3e}  vs unfused {O.rel_err_colmax(fused, split):.3e}")
    assert e <= TOL_LUT16, e
    assert O.rel_err_colmax(fused, split) <= TOL_LUT16
