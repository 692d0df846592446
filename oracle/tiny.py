"""Explicit-matrix brute force for PaTH attention.  TEST INFRASTRUCTURE ONLY.

A second, independent statement of the definition, used on tiny inputs to pin
the C oracle: every H_s is formed as a d x d matrix and the path product is
multiplied out in full.  Nothing here is shared with the C oracle or with the
HIP library.

Source: "PaTH Attention" technical summary (gist.science 2505.16381),
§2 "Mecanismo Central" (logit k_j^T (prod_{s=j+1..i} H_s) q_i, H_s = I - beta_s
w_s w_s^T, causal softmax) and §2 "Extensões: PaTH-FoX" (additive forget bias).
Product order H_{j+1} H_{j+2} ... H_i (H_i nearest to q_i); empty product = I.
"""
from __future__ import annotations

import numpy as np


def householder(w_s: np.ndarray, beta_s: float) -> np.ndarray:
    """H_s = I - beta_s w_s w_s^T as an explicit matrix."""
    d = w_s.shape[0]
    return np.eye(d) - beta_s * np.outer(w_s, w_s)


def path_product(w: np.ndarray, beta: np.ndarray, j: int, i: int) -> np.ndarray:
    """H_{j+1} H_{j+2} ... H_i, multiplied left to right (identity if j == i)."""
    d = w.shape[1]
    m = np.eye(d)
    for s in range(j + 1, i + 1):
        m = m @ householder(w[s], float(beta[s]))
    return m


def logits(q, k, w, beta, log_forget=None, scale=1.0) -> np.ndarray:
    """Full [L, L] logit matrix of one head; entries above the diagonal are -inf."""
    q, k, w, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, w, beta))
    L = q.shape[0]
    s = np.full((L, L), -np.inf)
    for i in range(L):
        for j in range(i + 1):
            s[i, j] = scale * (k[j] @ path_product(w, beta, j, i) @ q[i])
            if log_forget is not None:
                s[i, j] += float(np.sum(np.asarray(log_forget, dtype=np.float64)[j + 1:i + 1]))
    return s


def attention(q, k, v, w, beta, log_forget=None, scale=1.0):
    """(o [L,d], lse [L]) of one head from the explicit logit matrix."""
    s = logits(q, k, w, beta, log_forget, scale)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    o = (e / l) @ np.asarray(v, dtype=np.float64)
    return o, (m + np.log(l))[:, 0]


def block_product(w, beta) -> np.ndarray:
    """H_0 H_1 ... H_{n-1} of one block as an explicit matrix."""
    return path_product(np.asarray(w, np.float64), np.asarray(beta, np.float64), -1, len(beta) - 1)
