"""Pins of the projection-prologue oracle (oracle/project.py) against facts
other than its own formula: torch's linear / normalize / sigmoid routines in
float64, a pure-Python brute force on a tiny case, and invariants of the
definition [PaTH summary (gist.science 2505.16381) §2 "Mecanismo Central":
beta_s = 2 sigmoid(u^T x_s + b)]."""
import math

import numpy as np
import torch

from oracle import project


def _rand(rng, T=7, Dm=12, H=3, d=5):
    return (rng.standard_normal((T, Dm)), rng.standard_normal((H, d, Dm)), rng.standard_normal((H, Dm)),
            rng.standard_normal(H))


def test_matches_torch_library_routines():
    rng = np.random.default_rng(1)
    x, Ww, u, b = _rand(rng)
    w, beta = project.project_wb(x, Ww, u, b)
    xt = torch.tensor(x)
    for h in range(Ww.shape[0]):
        v = torch.nn.functional.linear(xt, torch.tensor(Ww[h]))
        wr = torch.nn.functional.normalize(v, dim=-1, eps=1e-12).numpy()
        br = (2.0 * torch.sigmoid(torch.nn.functional.linear(xt, torch.tensor(u[h][None]), torch.tensor(b[h:h + 1]))))
        np.testing.assert_allclose(w[h], wr, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(beta[h], br.numpy()[:, 0], rtol=1e-13, atol=1e-14)


def test_brute_force_loops():
    rng = np.random.default_rng(2)
    x, Ww, u, b = _rand(rng, T=3, Dm=4, H=2, d=3)
    w, beta = project.project_wb(x, Ww, u, b)
    for h in range(2):
        for t in range(3):
            v = [sum(float(Ww[h, e, c]) * float(x[t, c]) for c in range(4)) for e in range(3)]
            n = math.sqrt(sum(vi * vi for vi in v))
            for e in range(3):
                assert abs(w[h, t, e] - v[e] / n) < 1e-14
            z = sum(float(u[h, c]) * float(x[t, c]) for c in range(4)) + float(b[h])
            assert abs(beta[h, t] - 2.0 / (1.0 + math.exp(-z))) < 1e-14


def test_invariants():
    rng = np.random.default_rng(3)
    x, Ww, u, b = _rand(rng)
    w, beta = project.project_wb(x, Ww, u, b)
    # unit vectors, beta in (0, 2)
    np.testing.assert_allclose(np.linalg.norm(w, axis=-1), 1.0, rtol=1e-14)
    assert np.all(beta > 0) and np.all(beta < 2)
    # w does not depend on the scale of x
    w2, _ = project.project_wb(3.5 * x, Ww, u, b)
    np.testing.assert_allclose(w2, w, rtol=1e-13, atol=1e-14)
    # sigmoid symmetry: with b = 0, beta(-x) = 2 - beta(x)
    _, bp = project.project_wb(x, Ww, u, np.zeros_like(b))
    _, bm = project.project_wb(-x, Ww, u, np.zeros_like(b))
    np.testing.assert_allclose(bp + bm, 2.0, rtol=1e-14)
    # x = 0: beta = 2 sigmoid(b) and the projection is the zero vector
    wz, bz = project.project_wb(np.zeros_like(x), Ww, u, b)
    np.testing.assert_allclose(bz, np.repeat((2.0 / (1.0 + np.exp(-b)))[:, None], x.shape[0], axis=1), rtol=1e-15)
    assert np.all(wz == 0.0)


def test_clip_caps_beta():
    rng = np.random.default_rng(4)
    x, Ww, u, b = _rand(rng)
    _, beta = project.project_wb(x, Ww, u, b + 3.0)
    _, clipped = project.project_wb(x, Ww, u, b + 3.0, beta_max=1.9)
    assert np.all(clipped <= 1.9)
    np.testing.assert_array_equal(clipped, np.minimum(beta, 1.9))
