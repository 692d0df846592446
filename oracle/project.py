"""fp64 oracle of the PaTH projection prologue.  TEST INFRASTRUCTURE ONLY.

[PaTH Attention technical summary, gist.science 2505.16381, §2 "Mecanismo
Central"]: the transition vector w_s and the factor beta_s are functions of
the input token x_s, with beta_s = 2 * sigmoid(u^T x_s + b), which lets a
transition have a negative eigenvalue.  The pages give no formula for w_s.
Reading: a per-head linear map of x_s scaled to unit length (the workloads
use unit-norm w), w_s = W_h x_s / max(|W_h x_s|, 1e-12).  [§6 "Limitações"]
mentions clipping beta in training; reading: an optional upper bound,
beta_s = min(beta_s, beta_max).

Shapes: x [T, Dm] (T tokens), Ww [H, d, Dm], u [H, Dm], b [H]
-> w [H, T, d], beta [H, T].  All arithmetic in float64 on the stored values.
"""
from __future__ import annotations

import numpy as np

NORM_FLOOR = 1e-12


def project_wb(x, Ww, u, b, beta_max=None):
    x = np.asarray(x, dtype=np.float64)
    Ww = np.asarray(Ww, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    # v[h, t, :] = W_h x_t
    v = np.einsum("hed,td->hte", Ww, x)
    norm = np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    w = v / np.maximum(norm, NORM_FLOOR)
    z = u @ x.T + b[:, None]  # [H, T]
    beta = 2.0 / (1.0 + np.exp(-z))
    if beta_max is not None:
        beta = np.minimum(beta, beta_max)
    return w, beta
