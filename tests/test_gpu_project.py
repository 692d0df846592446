"""GPU parity of the projection prologue (path_project, through the C ABI)
against the fp64 oracle (oracle/project.py) on the same seeded bf16 inputs.

Bars, from the arithmetic: w is the fp32 result rounded once to bf16, and
|w_e| < 1, so it may differ from the exact value by half a bf16 ulp (2^-9)
plus fp32 accumulation error: max |dw| <= 2.5e-3.  beta stays in fp32:
max |dbeta| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import dependent_position_encoding_fwd_amd as pa
import synthetic
from oracle import project

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W_TOL, B_TOL = 2.5e-3, 1e-4


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(x, Ww, u, b, w, beta, beta_max=None, tokens=None):
    B, L, Dm = x.shape
    xt = _np(x).reshape(B * L, Dm)
    if tokens is not None:
        xt = xt[tokens]
    rw, rb = project.project_wb(xt, _np(Ww), _np(u), _np(b), beta_max)
    gw = _np(w).transpose(1, 0, 2, 3).reshape(Ww.shape[0], B * L, -1)
    gb = _np(beta).transpose(1, 0, 2).reshape(Ww.shape[0], B * L)
    if tokens is not None:
        gw, gb = gw[:, tokens], gb[:, tokens]
    ew, eb = float(np.max(np.abs(gw - rw))), float(np.max(np.abs(gb - rb)))
    print(f"  max|dw|={ew:.3e} max|dbeta|={eb:.3e}", flush=True)
    assert ew <= W_TOL and eb <= B_TOL, (ew, eb)


@pytest.mark.parametrize("B,L,Dm,H,d", [(1, 200, 128, 3, 64), (2, 77, 256, 5, 128), (1, 1, 64, 1, 64),
                                        (1, 300, 192, 65, 64), (3, 128, 512, 16, 64), (1, 513, 320, 4, 64),
                                        (2, 130, 2048, 16, 128), (1, 70, 4096, 2, 64)])
def test_project_small(B, L, Dm, H, d):
    print(f"[project] B={B} L={L} Dm={Dm} H={H} d={d}", flush=True)
    x = synthetic.project_inputs(B, L, Dm, H, d, seed=B * 1000 + L + H)
    g = {n: t.to(DEV) for n, t in x.items()}
    w, beta = pa.path_project(g["x"], g["Ww"], g["u"], g["b"])
    torch.cuda.synchronize()
    _check(x["x"], x["Ww"], x["u"], x["b"], w, beta)


def test_project_clip():
    x = synthetic.project_inputs(1, 150, 128, 4, 64, seed=5)
    x["b"] = x["b"] + 3.0  # most betas near 2
    g = {n: t.to(DEV) for n, t in x.items()}
    w, beta = pa.path_project(g["x"], g["Ww"], g["u"], g["b"], beta_max=1.9)
    torch.cuda.synchronize()
    assert float(beta.max()) <= 1.9
    _check(x["x"], x["Ww"], x["u"], x["b"], w, beta, beta_max=1.9)


def test_project_zero_tokens():
    """x = 0: the projection is the zero vector (w = 0) and beta = 2 sigmoid(b)."""
    x = synthetic.project_inputs(1, 64, 128, 3, 64, seed=6)
    x["x"] = torch.zeros_like(x["x"])
    g = {n: t.to(DEV) for n, t in x.items()}
    w, beta = pa.path_project(g["x"], g["Ww"], g["u"], g["b"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(w).item() == 0
    _check(x["x"], x["Ww"], x["u"], x["b"], w, beta)


def test_project_full_size():
    """The bench workload's shape (B=8, L=4096, Dm=1024, H=16, d=64), every token
    against the oracle (in slices of 2048 tokens); w must also be unit length."""
    B, L, Dm, H, d = 8, 4096, 1024, 16, 64
    x = synthetic.project_inputs(B, L, Dm, H, d, seed=2)
    g = {n: t.to(DEV) for n, t in x.items()}
    w, beta = pa.path_project(g["x"], g["Ww"], g["u"], g["b"])
    torch.cuda.synchronize()
    xt = _np(x["x"]).reshape(B * L, Dm)
    Ww, u, b = _np(x["Ww"]), _np(x["u"]), _np(x["b"])
    gw = _np(w).transpose(1, 0, 2, 3).reshape(H, B * L, d)
    gb = _np(beta).transpose(1, 0, 2).reshape(H, B * L)
    ew = eb = 0.0
    for t0 in range(0, B * L, 2048):
        rw, rb = project.project_wb(xt[t0:t0 + 2048], Ww, u, b)
        ew = max(ew, float(np.max(np.abs(gw[:, t0:t0 + 2048] - rw))))
        eb = max(eb, float(np.max(np.abs(gb[:, t0:t0 + 2048] - rb))))
    print(f"  all {B * L} tokens: max|dw|={ew:.3e} max|dbeta|={eb:.3e}", flush=True)
    assert ew <= W_TOL and eb <= B_TOL, (ew, eb)
    norms = torch.linalg.vector_norm(w.float(), dim=-1)
    assert float((norms - 1).abs().max()) <= 8 * 2.0 ** -9
