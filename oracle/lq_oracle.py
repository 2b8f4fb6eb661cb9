"""Float64 CPU oracle for the LiftQuant lift-then-project linear layer.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the
smoke check and by the benchmark's CPU-baseline leg, never by the product
path.  It shares no code with the HIP library and imports nothing from it.

What it computes comes from the LiftQuant notes ("LiftQuant: Continuous
Bit-Width LLM via Dimensional Lifting and Projection"):
  * a d-wide weight group is w = M y with y in {+-1}^D and M of shape d x D,
    so each weight is w_r = sum_j M[r][j] y_j (section 关键设计 1);
  * the layer output is o = diag(s) W_q (M T^-1 a) (section 关键设计 4, and
    the 推理 node of the overview flowchart in 整体框架).
Because y . (M^T x) = (M y) . x for every group, the lifted product equals a
dense mat-vec with the reconstructed weights W_hat[i, g*d + r] =
sum_j M[r][j] y[i, g*D + j].  The oracle is that dense mat-vec, written out
in float64 from the stored inputs, converted exactly.

Readings where the notes are silent (each is also listed with the design
notes of the repository):
  * "M T^-1 a" does not type-check as written (M is d x D); it is read as
    u = T^-1 a followed by the per-group lift a_hat_g = M^T u_g.
  * T^-1 is block-diagonal with square blocks; block q maps a[tb*q + c] to
    u[tb*q + r] by T_q[r][c].  The notes' Kronecker form of the whitening
    (关键设计 3) is the second transform below (transform_kron).
  * the lifted index of sign j of group g is k = g*D + j; bit (k & 31) of
    word (k >> 5) of a row is 1 iff the sign is +1.
  * s is a per-output-row scale applied after the contraction.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "decode", "unpack_bits", "signs_from_packed", "pack_signs_ref", "reconstruct_weights",
    "transform", "lift", "lifted_product", "forward", "forward_lifted", "forward_loops",
    "rel_err_colmax", "kron_inverse_dense", "transform_kron", "lift_kron", "forward_kron",
]


# ------------------------------------------------------------------ storage decode
def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.  bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------------ signs
def unpack_bits(packed: np.ndarray, K: int) -> np.ndarray:
    """uint32 [rows][ldw] -> uint8 {0,1} [rows][K]; bit k&31 of word k>>5."""
    p = np.ascontiguousarray(packed, dtype="<u4")
    rows = p.shape[0]
    bits = np.unpackbits(p.view(np.uint8).reshape(rows, -1), axis=1, bitorder="little")
    return bits[:, :K]


def signs_from_packed(packed: np.ndarray, K: int) -> np.ndarray:
    """uint32 words -> int8 signs: +1 where the bit is 1, -1 where it is 0."""
    return (2 * unpack_bits(packed, K).astype(np.int8) - 1).astype(np.int8)


def pack_signs_ref(signs: np.ndarray, ldw: Optional[int] = None) -> np.ndarray:
    """int8 signs [rows][K] -> uint32 [rows][ldw]; a sign > 0 packs as 1,
    anything else as 0; padding bits are 0."""
    sg = np.asarray(signs)
    rows, K = sg.shape
    nw = (K + 31) // 32
    ldw = nw if ldw is None else ldw
    bits = np.zeros((rows, ldw * 32), dtype=np.uint8)
    bits[:, :K] = sg > 0
    return np.packbits(bits, axis=1, bitorder="little").view("<u4").reshape(rows, ldw).copy()


# ------------------------------------------------------------------ layer pieces
def reconstruct_weights(y: np.ndarray, M: np.ndarray, d: int, D: int) -> np.ndarray:
    """Signs y [rows][K] (+-1) and M [d][D] -> W_hat [rows][n] float64 with
    W_hat[i, g*d + r] = sum_j M[r][j] * y[i, g*D + j]."""
    rows, K = y.shape
    G = K // D
    Mf = decode(M, "f32") if M.dtype != np.float64 else M
    yg = y.reshape(rows, G, D).astype(np.float64)
    w = yg @ Mf.T                        # [rows][G][d]
    return w.reshape(rows, G * d)


def transform(a: np.ndarray, t_inv: np.ndarray) -> np.ndarray:
    """u = blockdiag(T_0 .. T_{nb-1}) a for a [B][n] float64 and blocks
    [nb][tb][tb] float64: u[b, tb*q + r] = sum_c T_q[r][c] a[b, tb*q + c]."""
    B, n = a.shape
    nb, tb, _ = t_inv.shape
    assert nb * tb == n
    ab = a.reshape(B, nb, tb)
    u = np.einsum("qrc,bqc->bqr", t_inv, ab)
    return u.reshape(B, n)


def lift(u: np.ndarray, M: np.ndarray, d: int, D: int) -> np.ndarray:
    """a_hat[b, g*D + j] = sum_r M[r][j] * u[b, g*d + r]  (the per-group M^T)."""
    B, n = u.shape
    G = n // d
    Mf = M.astype(np.float64)
    return (u.reshape(B, G, d) @ Mf).reshape(B, G * D)


# ------------------------------------------------------------------ Kronecker whitening
# 关键设计 3 writes the per-layer whitening as T = diag(s1) (P1 (x) P2) diag(s2),
# P1 and P2 small square matrices, s1 a per-channel scale and s2 a scale that
# is constant over each lift group (so that it folds into M).  The layer
# applies T^-1 = diag(s2)^-1 (P1 (x) P2)^-1 diag(s1)^-1, and
# (P1 (x) P2)^-1 = P1^-1 (x) P2^-1.  Readings: the pages' sqrt(n) x sqrt(n)
# factors are read as n1 x n1 and n2 x n2 with n = n1 n2 (n = 8192 has no
# integer square root); channel c of a is entry (c // n2, c % n2) of the
# n1 x n2 reshape (numpy's row-major order, which is the order np.kron
# uses); the inverses P1^-1, P2^-1 are inputs, as T^-1 is for the
# block-diagonal form; s2 is given per d-wide lift group.

def kron_inverse_dense(s1: np.ndarray, p1_inv: np.ndarray, p2_inv: np.ndarray,
                       s2_group: np.ndarray, d: int) -> np.ndarray:
    """The n x n matrix T^-1 = diag(1/s2) (P1^-1 (x) P2^-1) diag(1/s1), formed
    densely with np.kron (small n only)."""
    s1 = np.asarray(s1, dtype=np.float64)
    s2 = np.repeat(np.asarray(s2_group, dtype=np.float64), d)
    K = np.kron(np.asarray(p1_inv, dtype=np.float64), np.asarray(p2_inv, dtype=np.float64))
    return (K / s2[:, None]) / s1[None, :]


def transform_kron(a: np.ndarray, s1: np.ndarray, p1_inv: np.ndarray, p2_inv: np.ndarray,
                   s2_group: np.ndarray, d: int, dense: Optional[bool] = None) -> np.ndarray:
    """u = T^-1 a for the Kronecker form, a [B][n] float64.  dense=True applies
    the dense matrix of kron_inverse_dense; dense=False uses, per token, the
    n1 x n2 reshape X of a / s1 and u = vec(P1^-1 X P2^-T) / s2 (the Kronecker
    identity in row-major order, pinned against the dense form).  By default
    the dense form is used when n <= 2048."""
    a = np.asarray(a, dtype=np.float64)
    B, n = a.shape
    n1, n2 = p1_inv.shape[0], p2_inv.shape[0]
    assert n1 * n2 == n
    if dense is None:
        dense = n <= 2048
    if dense:
        return a @ kron_inverse_dense(s1, p1_inv, p2_inv, s2_group, d).T
    X = (a / np.asarray(s1, dtype=np.float64)[None, :]).reshape(B, n1, n2)
    Y = np.asarray(p1_inv, dtype=np.float64)[None] @ X @ np.asarray(p2_inv, dtype=np.float64).T[None]
    s2 = np.repeat(np.asarray(s2_group, dtype=np.float64), d)
    return Y.reshape(B, n) / s2[None, :]


def lift_kron(a, s1, p1_inv, p2_inv, s2_group, M, d: int, D: int, dtype: str) -> np.ndarray:
    """a_hat = lift(T^-1 a) with the Kronecker T^-1, from the stored inputs
    (a in `dtype`, the factors, scales and M float32) converted exactly."""
    a64 = decode(a, dtype)
    u = transform_kron(a64, decode(s1, "f32"), decode(p1_inv, "f32"), decode(p2_inv, "f32"),
                       decode(s2_group, "f32"), d)
    return lift(u, decode(M, "f32"), d, D)


def forward_kron(packed: np.ndarray, K: int, M, s1, p1_inv, p2_inv, s2_group, s, a, d: int,
                 D: int, dtype: str, rows: Optional[Sequence[int]] = None,
                 chunk: int = 2048) -> np.ndarray:
    """o by the reconstruct route with the Kronecker T^-1: unpack, W_hat = M y
    per group, u = T^-1 a, o = s * (W_hat u)."""
    M64, s64, a64 = decode(M, "f32"), decode(s, "f32"), decode(a, dtype)
    u = transform_kron(a64, decode(s1, "f32"), decode(p1_inv, "f32"), decode(p2_inv, "f32"),
                       decode(s2_group, "f32"), d)
    idx = np.arange(packed.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((a64.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        w = reconstruct_weights(signs_from_packed(packed[sel], K), M64, d, D)
        out[:, c0:c0 + sel.size] = (w @ u.T).T * s64[sel][None, :]
    return out


def _inputs64(M, t_inv, s, a, dtype):
    return (decode(M, "f32"), decode(t_inv, dtype), decode(s, "f32"), decode(a, dtype))


def forward(packed: np.ndarray, K: int, M: np.ndarray, t_inv: np.ndarray, s: np.ndarray,
            a: np.ndarray, d: int, D: int, dtype: str, rows: Optional[Sequence[int]] = None,
            chunk: int = 2048) -> np.ndarray:
    """o [B][len(rows)] float64 by the reconstruct route: unpack, W_hat = M y per
    group, u = T^-1 a, o = s * (W_hat u).  rows=None means every row."""
    M64, T64, s64, a64 = _inputs64(M, t_inv, s, a, dtype)
    u = transform(a64, T64)                       # [B][n]
    idx = np.arange(packed.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((a64.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        y = signs_from_packed(packed[sel], K)
        w = reconstruct_weights(y, M64, d, D)     # [rows][n]
        out[:, c0:c0 + sel.size] = (w @ u.T).T * s64[sel][None, :]
    return out


def lifted_product(packed: np.ndarray, K: int, a_lift: np.ndarray, s: np.ndarray,
                   rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """o[b, i] = s_i * sum_k sigma_ik a_lift[b, k]  (sigma from the sign bits),
    the contraction that follows the lift, for given lifted activations."""
    al = np.asarray(a_lift, dtype=np.float64)
    idx = np.arange(packed.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    y = signs_from_packed(packed[idx], K).astype(np.float64)
    return (y @ al.T).T * np.asarray(s, dtype=np.float64)[idx][None, :]


def forward_lifted(packed: np.ndarray, K: int, M: np.ndarray, t_inv: np.ndarray, s: np.ndarray,
                   a: np.ndarray, d: int, D: int, dtype: str,
                   rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """o by the lifted route: a_hat = lift(T^-1 a), o = s * (Y a_hat)."""
    M64, T64, s64, a64 = _inputs64(M, t_inv, s, a, dtype)
    ah = lift(transform(a64, T64), M64, d, D)     # [B][K]
    return lifted_product(packed, K, ah, s64, rows)


def forward_loops(packed, K, M, t_inv, s, a, d, D, dtype):
    """Pure-Python loops straight from the definitions (tiny inputs only):
    sign bit by shifting the word, weight w = sum_j M[r][j] y_j, u = T^-1 a
    block by block, o_i = s_i sum_c w_ic u_c."""
    M64, T64, s64, a64 = _inputs64(M, t_inv, s, a, dtype)
    m = packed.shape[0]
    B, n = a64.shape
    nb, tb, _ = T64.shape
    G = n // d
    u = [[0.0] * n for _ in range(B)]
    for b in range(B):
        for q in range(nb):
            for r in range(tb):
                acc = 0.0
                for c in range(tb):
                    acc += float(T64[q, r, c]) * float(a64[b, q * tb + c])
                u[b][q * tb + r] = acc
    out = [[0.0] * m for _ in range(B)]
    for i in range(m):
        w = [0.0] * n
        for g in range(G):
            for r in range(d):
                acc = 0.0
                for j in range(D):
                    k = g * D + j
                    bit = (int(packed[i, k >> 5]) >> (k & 31)) & 1
                    acc += float(M64[r, j]) * (1.0 if bit else -1.0)
                w[g * d + r] = acc
        for b in range(B):
            acc = 0.0
            for c in range(n):
                acc += w[c] * u[b][c]
            out[b][i] = float(s64[i]) * acc
    return np.array(out, dtype=np.float64)


# ------------------------------------------------------------------ error metric
def rel_err_colmax(got: np.ndarray, ref: np.ndarray) -> float:
    """max over tokens b of  max_i |got[b,i] - ref[b,i]| / max_i |ref[b,i]|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())
