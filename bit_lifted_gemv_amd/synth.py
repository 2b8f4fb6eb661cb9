"""Seeded synthetic LiftQuant layers (inputs only; no layer arithmetic).

The LiftQuant notes ("LiftQuant: Continuous Bit-Width LLM via Dimensional
Lifting and Projection", section 关键设计 1) store each d-wide weight group as
D one-bit signs and a global projection M (d x D); the inference form
o = diag(s) W_q (M T^-1 a) (section 关键设计 4) also needs a per-layer
transform T^-1, a per-row scale s and activations a.  No trained weights or
datasets exist here, so every layer is drawn from a seeded generator with the
shapes of the 8B / 70B-class projections the notes deploy on.

This module draws the random inputs and converts them to their storage
formats; it computes nothing of the layer itself.  Both the HIP path and the
float64 oracle consume what it returns.

Storage formats (all numpy, host memory):
  packed  uint32 [m][ldw]  bit (k & 31) of word (k >> 5) is 1 iff sign(k) = +1
  M       float32 [d][D]
  t_inv   16-bit [n/128][128][128]  (float16, or bf16 held as uint16 bits)
  s       float32 [m]
  a       16-bit [B][n]              (float16, or bf16 held as uint16 bits)
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

T_BLOCK = 128


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One named LQ-D/d workload: bit-width D/d, shapes, batches, value ranges."""
    index: int                      # 1-based workload number
    name: str
    D: int
    d: int
    shapes: Tuple[Tuple[int, int], ...]   # (m, n) pairs
    batches: Tuple[int, ...]
    act_dtype: str                   # "f16" or "bf16"; T^-1 uses the same type
    s_range: Tuple[float, float]
    outlier_frac: float = 0.0        # fraction of channels scaled by outlier_scale
    outlier_scale: float = 20.0

    @property
    def bits(self) -> float:
        return self.D / self.d


# The five workloads: 2.4-bit single layer, 2.5-bit 8B attention, 2.0-bit
# 8B MLP with outlier channels, 2.375-bit 70B MLP, 2.5-bit prefill GEMM.
CONFIGS: Tuple[LayerConfig, ...] = (
    LayerConfig(1, "LQ-24/10 single linear", 24, 10, ((1280, 1280),), (1,), "f16", (0.01, 0.03)),
    LayerConfig(2, "LQ-20/8 attention projection", 20, 8, ((4096, 4096),), (1,), "bf16", (0.01, 0.03)),
    LayerConfig(3, "LQ-16/8 8B MLP", 16, 8, ((14336, 4096), (4096, 14336)), (1, 4, 16), "bf16",
                (0.01, 0.03), outlier_frac=0.01),
    LayerConfig(4, "LQ-19/8 70B MLP", 19, 8, ((28672, 8192), (8192, 28672)), (1, 4, 16), "bf16",
                (0.005, 0.02)),
    LayerConfig(5, "LQ-40/16 prefill GEMM", 40, 16, ((8192, 8192),), (512,), "bf16", (0.01, 0.03)),
)


def all_cases() -> List[Tuple[LayerConfig, int, Tuple[int, int], int]]:
    """Every (config, shape index, (m, n), batch) case: 15 in total."""
    out = []
    for cfg in CONFIGS:
        for si, shp in enumerate(cfg.shapes):
            for b in cfg.batches:
                out.append((cfg, si, shp, b))
    return out


def lifted_dim(n: int, d: int, D: int) -> int:
    if n % d:
        raise ValueError(f"n={n} is not a multiple of d={d}")
    return n // d * D


def words_per_row(K: int) -> int:
    return (K + 31) // 32


def aligned_row_words(K: int) -> int:
    """Row stride in words that starts every row on a 128-byte line (the
    default for generated layers: rows whose slices straddle lines are read
    twice over by a slice-wise stream)."""
    return (words_per_row(K) + 31) // 32 * 32


# ---------------------------------------------------------------- 16-bit storage
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(np.asarray(x, dtype=np.float32))
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------- draws
def random_sign_words(rng: np.random.Generator, rows: int, K: int,
                      ldw: Optional[int] = None) -> np.ndarray:
    """Bernoulli(0.5) signs drawn directly as packed words: uint32 [rows][ldw].
    Every bit of a uniform random word is an independent fair coin; bits at
    positions >= K and the padding words up to ldw are zero.  Only the
    ceil(K/32) data words of each row are drawn, so the values do not depend
    on ldw."""
    nw = words_per_row(K)
    ldw = nw if ldw is None else ldw
    if ldw < nw:
        raise ValueError("ldw too small")
    data = rng.integers(0, 2**32, size=(rows, nw), dtype=np.uint64).astype(np.uint32)
    if K % 32:
        data[:, -1] &= np.uint32((1 << (K % 32)) - 1)
    w = np.zeros((rows, ldw), dtype=np.uint32)
    w[:, :nw] = data
    return w


def random_signs_i8(rng: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """Unpacked signs as int8 +-1 [rows][K]."""
    return np.where(rng.random((rows, K)) < 0.5, 1, -1).astype(np.int8)


def haar_orthogonal(rng: np.random.Generator, size: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix (float64): QR of a Gaussian matrix,
    columns re-signed by sign(diag R)."""
    g = rng.standard_normal((size, size))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


@dataclasses.dataclass
class Layer:
    """One synthetic layer plus its activations, in storage formats."""
    m: int
    n: int
    d: int
    D: int
    B: int
    packed: np.ndarray      # uint32 [m][ldw]
    M: np.ndarray           # float32 [d][D]
    t_inv: np.ndarray       # 16-bit [n/128][128][128]
    s: np.ndarray           # float32 [m]
    a: np.ndarray           # 16-bit [B][n]
    dtype: str              # storage type of t_inv and a: "f16" | "bf16"
    outliers: np.ndarray    # int64 channel indices scaled before the cast

    @property
    def K(self) -> int:
        return lifted_dim(self.n, self.d, self.D)

    @property
    def ldw(self) -> int:
        return self.packed.shape[1]


def make_layer(m: int, n: int, d: int, D: int, B: int, seed: int, dtype: str = "bf16",
               s_range: Tuple[float, float] = (0.01, 0.03), outlier_frac: float = 0.0,
               outlier_scale: float = 20.0, t_block: int = T_BLOCK, ldw: Optional[int] = None,
               identity_t: bool = False) -> Layer:
    """Draw one layer.  Draw order is fixed: sign words, M, T^-1 blocks, s, a,
    outlier channels.  M ~ N(0, 1/D) (variance 1/D), s ~ U(s_range),
    a ~ N(0, 1) with round(outlier_frac*n) channels scaled in float32 before
    the 16-bit cast, T^-1 = n/t_block Haar orthogonal blocks."""
    if n % t_block:
        raise ValueError("n must be a multiple of the transform block")
    K = lifted_dim(n, d, D)
    rng = np.random.default_rng(seed)
    packed = random_sign_words(rng, m, K, aligned_row_words(K) if ldw is None else ldw)
    M = (rng.standard_normal((d, D)) / np.sqrt(D)).astype(np.float32)
    nb = n // t_block
    if identity_t:
        blocks = np.broadcast_to(np.eye(t_block), (nb, t_block, t_block)).copy()
    else:
        blocks = np.stack([haar_orthogonal(rng, t_block) for _ in range(nb)])
    t_inv = to_storage(blocks, dtype)
    s = rng.uniform(s_range[0], s_range[1], size=m).astype(np.float32)
    a32 = rng.standard_normal((B, n)).astype(np.float32)
    n_out = int(round(outlier_frac * n))
    outliers = np.sort(rng.choice(n, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    if n_out:
        a32[:, outliers] *= np.float32(outlier_scale)
    a = to_storage(a32, dtype)
    return Layer(m, n, d, D, B, packed, M, t_inv, s, a, dtype, outliers.astype(np.int64))


@dataclasses.dataclass
class KronFactors:
    """Kronecker-factored whitening of one layer, in the stored form the lift
    takes: s1 [n], P1^-1 [n1][n1], P2^-1 [n2][n2], s2 [n/d], all float32."""
    n1: int
    n2: int
    s1: np.ndarray
    p1_inv: np.ndarray
    p2_inv: np.ndarray
    s2: np.ndarray


def kron_split(n: int, d: int) -> Tuple[int, int]:
    """n = n1 * n2 with n2 the largest divisor of n that is at most 128 and a
    multiple of d (lift groups stay inside a row of the n1 x n2 reshape)."""
    for n2 in range(min(128, n), 0, -1):
        if n % n2 == 0 and n2 % d == 0:
            return n // n2, n2
    raise ValueError(f"no split of n={n} for d={d}")


def make_kron_factors(n: int, d: int, seed: int, n1: Optional[int] = None) -> KronFactors:
    """Seeded whitening factors: P1, P2 Haar orthogonal (so P^-1 = P^T),
    s1 ~ U(0.5, 2) per channel, s2 ~ U(0.5, 2) per d-group.  Draw order:
    P1, P2, s1, s2."""
    if n1 is None:
        n1, n2 = kron_split(n, d)
    else:
        n2 = n // n1
    rng = np.random.default_rng(seed)
    p1 = haar_orthogonal(rng, n1)
    p2 = haar_orthogonal(rng, n2)
    s1 = rng.uniform(0.5, 2.0, n).astype(np.float32)
    s2 = rng.uniform(0.5, 2.0, n // d).astype(np.float32)
    return KronFactors(n1, n2, s1, np.ascontiguousarray(p1.T).astype(np.float32),
                       np.ascontiguousarray(p2.T).astype(np.float32), s2)


def case_seed(cfg_index: int, shape_index: int) -> int:
    return 1000 * cfg_index + shape_index


def make_case(cfg: LayerConfig, shape_index: int, B: int, m: Optional[int] = None,
              n: Optional[int] = None) -> Layer:
    """The seeded layer of one workload case (optionally with reduced m / n)."""
    mm, nn = cfg.shapes[shape_index]
    return make_layer(m or mm, n or nn, cfg.d, cfg.D, B, case_seed(cfg.index, shape_index),
                      dtype=cfg.act_dtype, s_range=cfg.s_range, outlier_frac=cfg.outlier_frac,
                      outlier_scale=cfg.outlier_scale)
