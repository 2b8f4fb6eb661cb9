"""CPU oracle for the LiftQuant lattice encoder (nearest point of the projected
1-bit lattice) and for learning the projection M.

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
           "group_errors", "info_bits", "codebook_mse", "softmin_objective", "adam_step",
           "learn_m"]


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


# ----------------------------------------------------------- learning M
# 关键设计 2: M* = argmin_M E_{w ~ N}[min_y ||w - M y||], M initialised
# orthogonal, the inner argmin replaced by a soft-argmin at temperature 10 so
# that the objective is differentiable and M is learned end to end.
# Readings (also listed with the design notes):
#   * the candidates are all 2^D codes (enumeration order as above);
#   * soft-argmin: weights p_t = softmax_t(-T e_t) over the squared distances
#     e_t = ||w - M y_t||^2 (T multiplies: T = 10 sharpens), and the soft code
#     y_hat = sum_t p_t y_t replaces the argmin; the loss of a batch is the
#     mean over its samples of ||w - M y_hat||^2;
#   * the optimiser is Adam (the notes name none), textbook form below.


def softmin_objective(W: np.ndarray, M: np.ndarray, T: float, chunk: int = 256):
    """Soft-argmin objective of a batch W [N][d] and its gradient, float64.

    Returns (loss, grad [d][D], y_hat [N][D]).  With r_n = w_n - M y_hat_n,
    loss = mean_n ||r_n||^2.  Gradient, derived by the chain rule through
    y_hat = P Y and P = softmax(-T E):
      g_n  = -2 M^T r_n                      (d loss_n / d y_hat_n)
      a_nt = g_n . y_t,  b_nt = p_nt (a_nt - g_n . y_hat_n)
      dL/dM = (1/N) [ -2 sum_n r_n y_hat_n^T
                      + 2T sum_t (sum_n b_nt w_n - beta_t C_t) y_t^T ],
      C_t = M y_t, beta_t = sum_n b_nt."""
    W = np.asarray(W, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    d, D = M.shape
    N = W.shape[0]
    Y = sign_table(D).astype(np.float64)               # [2^D][D]
    C = Y @ M.T                                         # [2^D][d]
    loss = 0.0
    g_direct = np.zeros((d, D))
    bw = np.zeros((1 << D, d))                          # sum_n b_nt w_n
    beta = np.zeros(1 << D)
    Yhat = np.zeros((N, D))
    for s in range(0, N, chunk):
        Wc = W[s:s + chunk]
        E = ((Wc[:, None, :] - C[None, :, :]) ** 2).sum(axis=2)     # [n][2^D]
        Z = -T * E
        Z -= Z.max(axis=1, keepdims=True)
        P = np.exp(Z)
        P /= P.sum(axis=1, keepdims=True)
        yh = P @ Y
        R = Wc - yh @ M.T
        loss += float((R * R).sum())
        G = -2.0 * R @ M                                # [n][D]
        A = G @ Y.T                                     # [n][2^D]
        gy = (G * yh).sum(axis=1)
        Bm = P * (A - gy[:, None])
        g_direct += -2.0 * R.T @ yh
        bw += Bm.T @ Wc
        beta += Bm.sum(axis=0)
        Yhat[s:s + chunk] = yh
    dC = 2.0 * T * (bw - beta[:, None] * C)            # dL/dC_t, [2^D][d]
    grad = (g_direct + dC.T @ Y) / N
    return loss / N, grad, Yhat


def adam_step(M, grad, m1, m2, step: int, lr: float, b1: float = 0.9, b2: float = 0.999,
              eps: float = 1e-8):
    """One Adam update (textbook, bias-corrected; step counts from 1).
    Returns (M, m1, m2), all float64."""
    m1 = b1 * np.asarray(m1, dtype=np.float64) + (1 - b1) * grad
    m2 = b2 * np.asarray(m2, dtype=np.float64) + (1 - b2) * grad * grad
    mh = m1 / (1 - b1 ** step)
    vh = m2 / (1 - b2 ** step)
    return np.asarray(M, dtype=np.float64) - lr * mh / (np.sqrt(vh) + eps), m1, m2


def learn_m(batches, M0: np.ndarray, T: float, lr: float):
    """Adam on the soft-argmin objective over the given sample batches (one
    step per batch) from M0; returns (M, losses)."""
    M = np.asarray(M0, dtype=np.float64).copy()
    m1 = np.zeros_like(M)
    m2 = np.zeros_like(M)
    losses = []
    for i, W in enumerate(batches, start=1):
        loss, g, _ = softmin_objective(W, M, T)
        M, m1, m2 = adam_step(M, g, m1, m2, i, lr)
        losses.append(loss)
    return M, losses
