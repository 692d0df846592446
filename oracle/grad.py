"""fp64 gradients of PaTH attention for the CPU oracle.  TEST INFRASTRUCTURE ONLY.

The forward is written out from its definition [PaTH Attention technical
summary, gist.science 2505.16381, §2 "Mecanismo Central" and §2 "Extensões:
PaTH-FoX"]: for every query i the logit of key j <= i is
    s_ij = scale * k_j . (H_{j+1} ... H_i q_i) + (c_i - c_j),
    H_s = I - beta_s w_s w_s^T,   c_i = sum_{s<=i} log f_s,
o_i = softmax_j(s_ij) v_j.  The transported queries of all rows are carried
together: at step j (from L-1 down to 0) row i >= j holds H_{j+1} ... H_i q_i,
gives s_ij, and then takes H_j.

The gradients are those of the scalar <dO, o> with respect to every input,
obtained by reverse-mode differentiation (torch.autograd, a library routine)
of that plain loop in float64; lse receives no incoming gradient.  Only tests
use this module.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).clone()
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def forward_torch(q, k, v, w, beta, log_forget, scale):
    """The defining loop in torch float64 ops (differentiable).  Returns (o, lse)."""
    L, d = q.shape
    U = q
    cols = []
    for j in range(L - 1, -1, -1):
        cols.append(scale * (U[j:] @ k[j]))          # s_ij for i >= j
        a = U[j:] @ w[j]
        U = torch.cat([U[:j], U[j:] - beta[j] * a[:, None] * w[j][None, :]], dim=0)
    # cols[L-1-j] holds s_ij for i = j..L-1; column j of S is it below j entries of -inf.
    S = torch.stack([torch.cat([torch.full((j,), float("-inf"), dtype=q.dtype), cols[L - 1 - j]])
                     for j in range(L)], dim=1)
    if log_forget is not None:
        c = torch.cumsum(log_forget, 0)
        S = S + (c[:, None] - c[None, :])
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    S = S.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(S, dim=1)
    o = torch.softmax(S, dim=1) @ v
    return o, lse


def path_bwd_head(q, k, v, w, beta, log_forget, scale, do):
    """Gradients of <do, o> for one head: returns dict dq, dk, dv, dw [L,d],
    dbeta [L] and dlog_forget [L] (None without gates), all float64 numpy."""
    xs = {n: _t(x).requires_grad_(True) for n, x in (("q", q), ("k", k), ("v", v), ("w", w), ("beta", beta))}
    lf = _t(log_forget).requires_grad_(True) if log_forget is not None else None
    o, _ = forward_torch(xs["q"], xs["k"], xs["v"], xs["w"], xs["beta"], lf, float(scale))
    loss = (o * _t(do)).sum()
    inputs = [xs[n] for n in ("q", "k", "v", "w", "beta")] + ([lf] if lf is not None else [])
    # w_0 and beta_0 never enter a logit (the product for j = i is empty), so at
    # L = 1 they are unused: their gradient is zero.
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    grads = [torch.zeros_like(x) if g is None else g for x, g in zip(inputs, grads)]
    out = {f"d{n}": g.numpy() for n, g in zip(("q", "k", "v", "w", "beta"), grads)}
    out["dlog_forget"] = grads[5].numpy() if lf is not None else None
    return out
