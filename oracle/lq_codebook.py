"""CPU oracle for the LiftQuant lattice encoder (nearest point of the projected
1-bit lattice).

TEST INFRASTRUCTURE ONLY.  Imported by the tests and by the benchmark's
CPU-baseline leg, never by the product path; it shares no code with the HIP
library and imports nothing from it.

What it computes comes from the LiftQuant notes ("LiftQuant: Continuous
Bit-Width LLM via Dimensional Lifting and Projection"):
  * a d-wide weight group w is approximated by M y with y in {+-1}^D and M of
    shape d x D (关键设计 1);
  * quantising w means finding the lattice point nearest to w, the inner
    minimum of the objective in 关键设计 2, min over y of ||w - M y||.  Done
    exhaustively that is 2^D candidates (`encode_exhaustive`);
  * the notes cut the search to 2^(D-d) candidates by starting from the
    pseudo-inverse projection and padding an auxiliary vector (关键设计 2).
    `encode_search` is that search under the reading below;
  * Info = -1/2 log2(MSE), the rate of a Gaussian source at distortion MSE,
    links the MSE and Info columns of the Gaussian-source table
    ("Llama-2-7B Wikitext-2 PPL (标准 Gaussian 源)").

Readings where the notes are silent (also listed with the design notes):
  * the auxiliary vector: M is completed to an invertible D x D matrix
    [M; A] (A of shape (D-d) x D, an input), w is padded with an auxiliary
    sign vector v in {+-1}^(D-d), and the candidate is y = sign([M; A]^-1
    [w; v]).  With [M; A] orthogonal (M taken from an orthogonal matrix, the
    initialisation of 关键设计 2, A its remaining rows) this is
    sign(M^+ w + A^T v): the pseudo-inverse start plus an auxiliary part.
    The candidate set is all 2^(D-d) vectors v; the result is the candidate
    nearest to w.
  * sign(0) = +1.
  * enumeration order and ties: candidate t (0 <= t < 2^k) has sign j equal
    to +1 iff bit j of t is set (j < k); among candidates of equal error the
    smallest t wins.
  * distance is the squared Euclidean norm (the same minimiser as the norm).

`dtype` selects the arithmetic: float64 by default; float32 takes the same
decisions in single precision, as a float32 kernel does (the summation order
of a float32 kernel still differs, so near-ties may resolve differently).
"""
from __future__ import annotations

import numpy as np

__all__ = ["sign_table", "encode_exhaustive", "encode_search", "search_matrix",
           "group_errors", "info_bits", "codebook_mse"]


def sign_table(k: int) -> np.ndarray:
    """All 2^k sign vectors in enumeration order: row t, column j is +1 iff
    bit j of t is set, else -1.  int8 [2^k][k]."""
    t = np.arange(1 << k, dtype=np.int64)[:, None]
    bits = (t >> np.arange(k, dtype=np.int64)[None, :]) & 1
    return (2 * bits - 1).astype(np.int8)


def group_errors(W: np.ndarray, M: np.ndarray, Y: np.ndarray) -> np.ndarray:
    """float64 ||w_g - M y_g||^2 for groups W [G][d] and codes Y [G][D]."""
    W = np.asarray(W, dtype=np.float64)
    R = W - np.asarray(Y, dtype=np.float64) @ np.asarray(M, dtype=np.float64).T
    return (R * R).sum(axis=1)


def _argmin_first(err: np.ndarray) -> np.ndarray:
    """Index of the smallest error per row; the first (smallest t) on ties."""
    return np.argmin(err, axis=1)


def encode_exhaustive(W: np.ndarray, M: np.ndarray, dtype=np.float64, chunk: int = 1 << 14):
    """Nearest lattice point by enumerating all 2^D codes (关键设计 2, the
    exponential search the notes start from).

    W: [G][d] groups; M: [d][D].  Returns (codes int8 [G][D], err [G] in
    `dtype`, index t of the chosen code [G])."""
    W = np.asarray(W, dtype=dtype)
    M = np.asarray(M, dtype=dtype)
    d, D = M.shape
    G = W.shape[0]
    Y = sign_table(D).astype(dtype)                     # [2^D][D]
    MY = Y @ M.T                                        # [2^D][d]: every lattice point
    best_e = np.full(G, np.inf, dtype=dtype)
    best_t = np.zeros(G, dtype=np.int64)
    for c0 in range(0, 1 << D, chunk):
        P = MY[c0:c0 + chunk]
        E = ((W[:, None, :] - P[None, :, :]) ** 2).sum(axis=2)    # [G][chunk]
        i = _argmin_first(E)
        e = E[np.arange(G), i]
        better = e < best_e                             # strict: earlier chunks win ties
        best_e = np.where(better, e, best_e)
        best_t = np.where(better, c0 + i, best_t)
    codes = sign_table(D)[best_t]
    return codes, best_e, best_t


def search_matrix(M: np.ndarray, A: np.ndarray) -> np.ndarray:
    """[M; A]^-1 in float64 (the completion must make it invertible)."""
    S = np.vstack([np.asarray(M, dtype=np.float64), np.asarray(A, dtype=np.float64)])
    return np.linalg.inv(S)


def encode_search(W: np.ndarray, M: np.ndarray, A: np.ndarray, dtype=np.float64,
                  chunk: int = 1 << 12):
    """Auxiliary-vector search (关键设计 2, under the reading in the module
    docstring): for every v in {+-1}^(D-d), y(v) = sign([M; A]^-1 [w; v]);
    return the candidate nearest to w.

    W: [G][d]; M: [d][D]; A: [(D-d)][D].  The inverse is formed in float64
    and rounded to `dtype`; the candidates and their errors are evaluated in
    `dtype`.  Returns (codes int8 [G][D], err [G], index t of v [G])."""
    M = np.asarray(M, dtype=np.float64)
    d, D = M.shape
    k = D - d
    Binv = search_matrix(M, A).astype(dtype)           # [D][D]
    Bw, Bv = Binv[:, :d], Binv[:, d:]
    W = np.asarray(W, dtype=dtype)
    Md = M.astype(dtype)
    G = W.shape[0]
    Cw = W @ Bw.T                                       # [G][D]: the start [M; A]^-1 [w; 0]
    V = sign_table(k).astype(dtype)                     # [2^k][k]
    best_e = np.full(G, np.inf, dtype=dtype)
    best_t = np.zeros(G, dtype=np.int64)
    best_y = np.zeros((G, D), dtype=np.int8)
    for c0 in range(0, 1 << k, chunk):
        Pv = V[c0:c0 + chunk] @ Bv.T                    # [chunk][D]: the auxiliary part
        X = Cw[:, None, :] + Pv[None, :, :]             # [G][chunk][D]
        Y = np.where(X >= 0, 1, -1).astype(np.int8)
        R = W[:, None, :] - Y.astype(dtype) @ Md.T      # [G][chunk][d]
        E = (R * R).sum(axis=2)
        i = _argmin_first(E)
        e = E[np.arange(G), i]
        better = e < best_e
        best_e = np.where(better, e, best_e)
        best_t = np.where(better, c0 + i, best_t)
        best_y = np.where(better[:, None], Y[np.arange(G), i], best_y)
    return best_y, best_e, best_t


def info_bits(mse) -> np.ndarray:
    """Info = -1/2 log2(MSE): bits per weight of a unit-variance Gaussian
    source at mean squared error MSE (the Info column of the Gaussian-source
    table is this function of its MSE column)."""
    return -0.5 * np.log2(np.asarray(mse, dtype=np.float64))


def codebook_mse(W: np.ndarray, M: np.ndarray, codes: np.ndarray) -> float:
    """Mean squared error per weight of the encoded groups (float64)."""
    W = np.asarray(W, dtype=np.float64)
    return float(group_errors(W, M, codes).sum() / W.size)
