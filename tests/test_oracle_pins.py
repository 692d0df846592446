"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The oracle (oracle/path_oracle.c) is the yardstick for every GPU parity test,
so it is itself checked here against things other than itself:
  * a hand-worked example (tests/golden/hand_example_d2_L3.json);
  * exact rational arithmetic on tiny inputs (fractions.Fraction);
  * an independent explicit-matrix brute force (oracle/tiny.py);
  * library routines in special cases: beta = 0 reduces PaTH to causal softmax
    attention (torch scaled_dot_product_attention, fp64 on the CPU), and a
    constant forget gate reduces the FoX bias to ALiBi's linear distance bias;
  * closed forms (d = 1; all w equal with beta = 2) and invariants (H orthogonal
    for beta = 2, |w| = 1; w_0, beta_0 never enter; lse normalises the softmax);
  * the UT identity P = I - W^T T^{-1} W (UT transform bullet of §3) against the
    explicitly multiplied block product, and T T^{-1} = I;
  * the in-place decode update (§3 "Inferência") against forward rows.
Sources: "PaTH Attention" summary (gist.science 2505.16381) §2 "Mecanismo
Central", §2 "Extensões: PaTH-FoX", §3 "Treinamento e Inferência Eficientes".
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import grad, tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_head(rng, L, d, unit_w=True, beta_max=2.0):
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    w = rng.standard_normal((L, d))
    if unit_w:
        w /= np.linalg.norm(w, axis=1, keepdims=True)
    beta = rng.uniform(0.0, beta_max, size=L)
    return q, k, v, w, beta


def test_hand_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_example_d2_L3.json")))
    inp = g["inputs"]
    q, k, w, beta = (np.array(inp[n], dtype=np.float64) for n in ("q", "k", "w", "beta"))
    lf = np.array(inp["log_forget"])
    for lg_key, log_forget in (("expected_logits", None), ("expected_fox_logits", lf)):
        exp = np.array([[(-np.inf if x is None else x) for x in row] for row in g[lg_key]])
        got = oracle.path_logits(q, k, w, beta, log_forget, scale=1.0)
        np.testing.assert_allclose(got, exp, rtol=0, atol=1e-13)


def _frac_logits(q, k, w, beta, scale):
    """Exact rational logits: apply H_i, H_{i-1}, ... to q_i with Fractions."""
    L, d = len(q), len(q[0])
    out = {}
    for i in range(L):
        u = list(q[i])
        for j in range(i, -1, -1):
            out[(i, j)] = scale * sum(k[j][t] * u[t] for t in range(d))
            c = beta[j] * sum(w[j][t] * u[t] for t in range(d))
            u = [u[t] - c * w[j][t] for t in range(d)]
    return out


def test_exact_rational_logits():
    rng = np.random.default_rng(11)
    L, d = 9, 4
    # dyadic rationals: exactly representable in fp64, exact in Fraction
    q, k, w = (np.round(rng.standard_normal((L, d)) * 8) / 8 for _ in range(3))
    beta = np.round(rng.uniform(0, 2, size=L) * 16) / 16
    fq, fk, fw = ([[Fraction(float(x)) for x in row] for row in a] for a in (q, k, w))
    fb = [Fraction(float(b)) for b in beta]
    exact = _frac_logits(fq, fk, fw, fb, Fraction(1, 2))
    got = oracle.path_logits(q, k, w, beta, None, scale=0.5)
    for (i, j), val in exact.items():
        assert abs(got[i, j] - float(val)) <= 1e-12 * max(1.0, abs(float(val)))
    assert np.all(np.isneginf(got[np.triu_indices(L, 1)]))


@pytest.mark.parametrize("L,d,fox,scale", [(1, 3, False, 1.0), (7, 3, False, 0.7), (16, 8, True, 1.0),
                                           (21, 5, True, 0.25), (24, 16, False, 0.125)])
def test_c_oracle_matches_explicit_matrices(L, d, fox, scale):
    rng = np.random.default_rng(L * 100 + d)
    q, k, v, w, beta = _rand_head(rng, L, d)
    lf = np.log(1.0 / (1.0 + np.exp(-rng.normal(3, 1, size=L)))) if fox else None
    ref_s = tiny.logits(q, k, w, beta, lf, scale)
    got_s = oracle.path_logits(q, k, w, beta, lf, scale)
    np.testing.assert_allclose(got_s, ref_s, rtol=1e-12, atol=1e-12)
    ref_o, ref_lse = tiny.attention(q, k, v, w, beta, lf, scale)
    o, lse = oracle.path_fwd_head(q, k, v, w, beta, lf, scale)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_row_subset_matches_full():
    rng = np.random.default_rng(3)
    q, k, v, w, beta = _rand_head(rng, 40, 8)
    o, lse = oracle.path_fwd_head(q, k, v, w, beta, None, 0.3)
    rows = [39, 0, 17, 17, 5]
    o2, lse2 = oracle.path_fwd_head(q, k, v, w, beta, None, 0.3, rows=rows)
    np.testing.assert_array_equal(o2, o[rows])
    np.testing.assert_array_equal(lse2, lse[rows])


@pytest.mark.parametrize("L,d,scale", [(33, 8, 1.0), (64, 16, 0.25), (5, 64, 0.125)])
def test_beta_zero_is_causal_softmax_attention(L, d, scale):
    rng = np.random.default_rng(L + d)
    q, k, v, w, _ = _rand_head(rng, L, d)
    beta = np.zeros(L)
    o, lse = oracle.path_fwd_head(q, k, v, w, beta, None, scale)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)
    s = scale * (tq @ tk.transpose(-1, -2))[0, 0]
    s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_constant_forget_gate_is_alibi():
    """log f_s = -lam: the FoX bias is -lam (i - j), ALiBi's linear distance bias."""
    rng = np.random.default_rng(5)
    L, d, lam, scale = 48, 8, 0.37, 0.5
    q, k, v, w, beta = _rand_head(rng, L, d)
    lf = np.full(L, -lam)
    # with beta = 0: exactly SDPA with the ALiBi additive mask
    zero = np.zeros(L)
    o, lse = oracle.path_fwd_head(q, k, v, w, zero, lf, scale)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    bias = np.where(j <= i, -lam * (i - j), -np.inf)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(bias),
                                                           scale=scale)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)
    # with general beta: FoX logits minus plain logits is exactly the ALiBi bias
    s_fox = oracle.path_logits(q, k, w, beta, lf, scale)
    s_plain = oracle.path_logits(q, k, w, beta, None, scale)
    tri = np.broadcast_to(j <= i, (L, L))
    np.testing.assert_allclose(s_fox[tri] - s_plain[tri], bias[tri], rtol=0, atol=1e-12)


def test_reflections_are_orthogonal_transport():
    """beta = 2, |w| = 1: every H_s is orthogonal, so the transported query keeps its norm.
    With keys e_b in d separate heads, sum_b s_ij(e_b)^2 = |q_i|^2 for every j <= i."""
    rng = np.random.default_rng(7)
    L, d = 20, 6
    q, _, _, w, _ = _rand_head(rng, L, d)
    beta = np.full(L, 2.0)
    tot = np.zeros((L, L))
    for b in range(d):
        kb = np.zeros((L, d))
        kb[:, b] = 1.0
        s = oracle.path_logits(q, kb, w, beta, None, 1.0)
        tot += np.where(np.isfinite(s), s, 0.0) ** 2
    qn = np.sum(q * q, axis=1)
    for i in range(L):
        np.testing.assert_allclose(tot[i, :i + 1], qn[i], rtol=1e-12)
    # and H_s is symmetric and squares to I
    hs = tiny.householder(w[3], 2.0)
    np.testing.assert_allclose(hs @ hs.T, np.eye(d), atol=1e-14)
    np.testing.assert_allclose(hs @ hs, np.eye(d), atol=1e-14)


def test_closed_form_equal_reflections():
    """All w_s = w (unit), beta = 2: the path product is (I - 2ww^T)^(i-j)."""
    rng = np.random.default_rng(9)
    L, d = 17, 5
    q, k, _, _, _ = _rand_head(rng, L, d)
    wv = rng.standard_normal(d)
    wv /= np.linalg.norm(wv)
    w = np.tile(wv, (L, 1))
    s = oracle.path_logits(q, k, w, np.full(L, 2.0), None, 1.0)
    R = np.eye(d) - 2 * np.outer(wv, wv)
    for i in range(L):
        for j in range(i + 1):
            ref = k[j] @ q[i] if (i - j) % 2 == 0 else k[j] @ R @ q[i]
            assert abs(s[i, j] - ref) < 1e-12


def test_closed_form_d1():
    """d = 1: s_ij = k_j q_i prod_{s=j+1..i} (1 - beta_s w_s^2)."""
    rng = np.random.default_rng(13)
    L = 30
    q, k, w = (rng.standard_normal((L, 1)) for _ in range(3))
    beta = rng.uniform(0, 2, size=L)
    s = oracle.path_logits(q, k, w, beta, None, 1.0)
    for i in range(L):
        for j in range(i + 1):
            f = np.prod([1.0 - beta[t] * w[t, 0] ** 2 for t in range(j + 1, i + 1)])
            assert abs(s[i, j] - k[j, 0] * q[i, 0] * f) <= 1e-12 * max(1.0, abs(s[i, j]))


def test_first_transition_never_enters():
    """w_0, beta_0 appear in no product prod_{s=j+1..i} with j >= 0."""
    rng = np.random.default_rng(17)
    L, d = 25, 7
    q, k, v, w, beta = _rand_head(rng, L, d)
    o1, lse1 = oracle.path_fwd_head(q, k, v, w, beta, None, 0.8)
    w2, b2 = w.copy(), beta.copy()
    w2[0] = rng.standard_normal(d)
    b2[0] = 1.9
    o2, lse2 = oracle.path_fwd_head(q, k, v, w2, b2, None, 0.8)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(lse1, lse2)


def test_lse_normalises_softmax():
    rng = np.random.default_rng(19)
    L, d = 50, 8
    q, k, v, w, beta = _rand_head(rng, L, d)
    lf = -rng.uniform(0, 0.2, size=L)
    s = oracle.path_logits(q, k, w, beta, lf, 1.0)
    _, lse = oracle.path_fwd_head(q, k, v, w, beta, lf, 1.0)
    np.testing.assert_allclose(np.sum(np.exp(s - lse[:, None]), axis=1), 1.0, rtol=1e-13)


def test_decode_steps_reproduce_forward_rows():
    """§3 "Inferência": keeping keys updated in place (k_j <- H_t k_j) and appending
    each new key untransformed gives, at step t, exactly row t of the forward."""
    rng = np.random.default_rng(23)
    L, d, scale = 40, 8, 0.6
    q, k, v, w, beta = _rand_head(rng, L, d)
    o_ref, lse_ref = oracle.path_fwd_head(q, k, v, w, beta, None, scale)
    kc = np.zeros((0, d))
    for t in range(L):
        o, lse, kc_new = oracle.path_decode_head(q[t], k[t], v[t], w[t], beta[t], kc, v[:t], scale)
        np.testing.assert_allclose(o, o_ref[t], rtol=1e-12, atol=1e-12)
        assert abs(lse - lse_ref[t]) < 1e-12
        kc = np.concatenate([kc_new, k[t:t + 1]], axis=0)


def test_fox_decode_steps_reproduce_brute_force_rows():
    """§2 "Extensões: PaTH-FoX" with §3 "Inferência": the gated decode step, fed the
    running prefixes c_j of log f, gives at step t row t of the brute-force gated
    attention (explicit Householder products plus sum_{j<s<=t} log f_s), and the
    prefix it returns is the plain cumulative sum."""
    rng = np.random.default_rng(31)
    L, d, scale = 24, 6, 0.8
    q, k, v, w, beta = _rand_head(rng, L, d)
    lf = -rng.uniform(0.0, 0.7, size=L)
    lf[5] = 0.0                     # an open gate
    o_ref, lse_ref = tiny.attention(q, k, v, w, beta, lf, scale)
    kc = np.zeros((0, d))
    cum = np.zeros((0,))
    for t in range(L):
        o, lse, kc_new, ct = oracle.path_decode_fox_head(q[t], k[t], v[t], w[t], beta[t], lf[t], kc, v[:t],
                                                         cum, scale)
        np.testing.assert_allclose(o, o_ref[t], rtol=1e-11, atol=1e-11)
        assert abs(lse - lse_ref[t]) < 1e-11
        assert abs(ct - np.sum(lf[:t + 1])) < 1e-13
        kc = np.concatenate([kc_new, k[t:t + 1]], axis=0)
        cum = np.append(cum, ct)


def test_fox_decode_open_gates_is_plain_decode():
    """log f = 0 everywhere: every bias vanishes and the gated step is the plain one."""
    rng = np.random.default_rng(37)
    n, d = 17, 8
    q_t, k_t, v_t, w_t = (rng.standard_normal(d) for _ in range(4))
    kc, vc = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o0, lse0, k0 = oracle.path_decode_head(q_t, k_t, v_t, w_t, 0.7, kc, vc, 0.5)
    o1, lse1, k1, ct = oracle.path_decode_fox_head(q_t, k_t, v_t, w_t, 0.7, 0.0, kc, vc, np.zeros(n), 0.5)
    assert np.array_equal(o0, o1) and lse0 == lse1 and np.array_equal(k0, k1) and ct == 0.0


def test_fox_decode_closed_gate_keeps_only_new_key():
    """A (numerically) closed gate at t, log f_t = -800, leaves the new key alone in the
    softmax: o = v_t and lse = scale * q_t . k_t."""
    rng = np.random.default_rng(41)
    n, d = 9, 8
    q_t, k_t, v_t, w_t = (rng.standard_normal(d) for _ in range(4))
    kc, vc = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    cum = np.cumsum(-rng.uniform(0, 0.3, size=n))
    o, lse, _, ct = oracle.path_decode_fox_head(q_t, k_t, v_t, w_t, 0.4, -800.0, kc, vc, cum, 1.1)
    np.testing.assert_allclose(o, v_t, atol=1e-300)
    assert abs(lse - 1.1 * float(q_t @ k_t)) < 1e-12
    assert ct == cum[-1] - 800.0


def test_decode_update_is_householder():
    rng = np.random.default_rng(29)
    n, d = 12, 6
    kc = rng.standard_normal((n, d))
    wt = rng.standard_normal(d)
    wt /= np.linalg.norm(wt)
    _, _, upd = oracle.path_decode_head(rng.standard_normal(d), rng.standard_normal(d),
                                        rng.standard_normal(d), wt, 1.3, kc, rng.standard_normal((n, d)))
    np.testing.assert_allclose(upd, kc @ tiny.householder(wt, 1.3).T, atol=1e-13)


@pytest.mark.parametrize("n,d", [(64, 16), (64, 64), (37, 8), (1, 4)])
def test_ut_identity(n, d):
    """§3 UT transform: H_0 ... H_{n-1} = I - W^T T^{-1} W."""
    rng = np.random.default_rng(n * 7 + d)
    q, k, _, w, beta = _rand_head(rng, n, d)
    beta[::5] = 0.0            # identity transitions
    beta[1::7] = 1.0           # singular H when |w| = 1
    tinv = oracle.ut_tinv(w, beta)
    _, _, pT = oracle.block_adjust(q, k, w, beta)
    P_explicit = tiny.block_product(w, beta)
    np.testing.assert_allclose(pT.T, P_explicit, atol=1e-12)
    np.testing.assert_allclose(np.eye(d) - w.T @ tinv @ w, P_explicit, atol=1e-11)
    assert np.all(np.tril(tinv, -1) == 0.0)


def test_tinv_inverts_T():
    """T = diag(1/beta) + strict_upper(W W^T) (beta > 0) and the oracle's T^{-1} is its inverse."""
    rng = np.random.default_rng(31)
    n, d = 64, 64
    _, _, _, w, beta = _rand_head(rng, n, d)
    beta = np.clip(beta, 0.05, None)
    T = np.diag(1.0 / beta) + np.triu(w @ w.T, 1)
    tinv = oracle.ut_tinv(w, beta)
    np.testing.assert_allclose(T @ tinv, np.eye(n), atol=1e-10)


def test_boundary_adjusted_qk_and_block_scan():
    """qhat_r = H_0..H_r q_r, khat_c = (H_{c+1}..H_{n-1})^T k_c, and for i in block m,
    j in block n < m: s_ij = khat_j^T P_{n+1} ... P_{m-1} qhat_i (the right-to-left
    block scan of §3 "Algoritmo Estilo FlashAttention")."""
    rng = np.random.default_rng(37)
    C, nb, d = 8, 4, 5
    L = C * nb
    q, k, v, w, beta = _rand_head(rng, L, d)
    s = oracle.path_logits(q, k, w, beta, None, 1.0)
    qh, kh, P = [], [], []
    for n in range(nb):
        sl = slice(n * C, (n + 1) * C)
        a, b, pt = oracle.block_adjust(q[sl], k[sl], w[sl], beta[sl])
        qh.append(a)
        kh.append(b)
        P.append(pt.T)
        for r in range(C):
            ref = tiny.path_product(w[sl], beta[sl], -1, r) @ q[sl][r]
            np.testing.assert_allclose(a[r], ref, atol=1e-12)
            refk = tiny.path_product(w[sl], beta[sl], r, C - 1).T @ k[sl][r]
            np.testing.assert_allclose(b[r], refk, atol=1e-12)
    for m in range(nb):
        for n in range(m):
            M = np.eye(d)
            for t in range(n + 1, m):
                M = M @ P[t]
            blk = kh[n] @ M @ qh[m].T          # [key, query]
            np.testing.assert_allclose(blk.T, s[m * C:(m + 1) * C, n * C:(n + 1) * C], atol=1e-11)


def test_prefix_sum():
    x = np.array([0.5, -1.25, 2.0, 0.125])
    np.testing.assert_array_equal(oracle.prefix_sum(x), np.array([0.5, -0.75, 1.25, 1.375]))


# --- gradients (oracle/grad.py) -------------------------------------------

def _bwd_case(rng, L, d, fox):
    q, k, v, w, beta = _rand_head(rng, L, d)
    lf = -rng.uniform(0.0, 0.5, size=L) if fox else None
    do = rng.standard_normal((L, d))
    return q, k, v, w, beta, lf, do


def test_grad_forward_loop_matches_c_oracle():
    """The differentiable loop computes the same o, lse as the C oracle."""
    rng = np.random.default_rng(43)
    q, k, v, w, beta, lf, _ = _bwd_case(rng, 37, 8, True)
    o_c, lse_c = oracle.path_fwd_head(q, k, v, w, beta, lf, 0.7)
    T = grad._t
    o_t, lse_t = grad.forward_torch(T(q), T(k), T(v), T(w), T(beta), T(lf), 0.7)
    np.testing.assert_allclose(o_t.numpy(), o_c, atol=1e-12)
    np.testing.assert_allclose(lse_t.numpy(), lse_c, atol=1e-12)


@pytest.mark.parametrize("fox", [False, True])
def test_grad_matches_central_differences_of_c_oracle(fox):
    """Every gradient against the directional derivative of <dO, o> taken by
    central differences of the independent C forward."""
    rng = np.random.default_rng(47 + fox)
    L, d, scale = 21, 6, 0.9
    q, k, v, w, beta, lf, do = _bwd_case(rng, L, d, fox)
    g = grad.path_bwd_head(q, k, v, w, beta, lf, scale, do)
    args = {"q": q, "k": k, "v": v, "w": w, "beta": beta}
    if fox:
        args["log_forget"] = lf

    def loss(a):
        o, _ = oracle.path_fwd_head(a["q"], a["k"], a["v"], a["w"], a["beta"], a.get("log_forget"), scale)
        return float(np.sum(o * do))

    eps = 1e-5
    for name in args:
        delta = rng.standard_normal(np.shape(args[name]))
        ap = dict(args); ap[name] = args[name] + eps * delta
        am = dict(args); am[name] = args[name] - eps * delta
        fd = (loss(ap) - loss(am)) / (2 * eps)
        an = float(np.sum(g["d" + name] * delta))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_grad_beta_zero_is_softmax_attention_grad():
    """beta = 0: every H is I, so dq, dk, dv are those of causal softmax attention
    (torch's scaled_dot_product_attention differentiated in float64) and dw = 0."""
    rng = np.random.default_rng(53)
    L, d, scale = 30, 8, 0.6
    q, k, v, w, _, _, do = _bwd_case(rng, L, d, False)
    beta = np.zeros(L)
    g = grad.path_bwd_head(q, k, v, w, beta, None, scale, do)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=True,
                                                         scale=scale)[0]
    rq, rk, rv = torch.autograd.grad((o * torch.tensor(do)).sum(), (tq, tk, tv))
    np.testing.assert_allclose(g["dq"], rq.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], rk.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], rv.numpy(), atol=1e-12)
    assert np.all(g["dw"] == 0.0)


def test_grad_single_token_has_no_transition_gradient():
    """L = 1: o = v_0 whatever q, k, w, beta are, so only dv is non-zero."""
    rng = np.random.default_rng(59)
    q, k, v, w, beta, _, do = _bwd_case(rng, 1, 5, False)
    g = grad.path_bwd_head(q, k, v, w, beta, None, 1.0, do)
    np.testing.assert_allclose(g["dv"], do, atol=1e-15)
    for n in ("dq", "dk", "dw", "dbeta"):
        assert np.all(g[n] == 0.0), n


# ---- the C reverse mode of the defining loop (oracle.path_bwd_head) ---------------

@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("L", [1, 2, 37, 70])
def test_c_reverse_mode_matches_autograd_of_the_loop(L, fox):
    """The hand-derived reverse mode in C against torch.autograd of the same
    definition written in torch ops (oracle/grad.py): every gradient."""
    rng = np.random.default_rng(61 + L + fox)
    q, k, v, w, beta, lf, do = _bwd_case(rng, L, 8, fox)
    beta[min(3, L - 1)] = 1.0      # a singular H (unit w, beta = 1) must not matter
    ref = grad.path_bwd_head(q, k, v, w, beta, lf, 0.7, do)
    got = oracle.path_bwd_head(q, k, v, w, beta, lf, 0.7, do)
    for n in ("dq", "dk", "dv", "dw", "dbeta") + (("dlog_forget",) if fox else ()):
        np.testing.assert_allclose(got[n], ref[n], atol=1e-11, rtol=1e-11, err_msg=n)
    assert (got["dlog_forget"] is None) == (not fox)


@pytest.mark.parametrize("fox", [False, True])
def test_c_reverse_mode_matches_central_differences(fox):
    """Every gradient of the C reverse mode against central differences of the
    C forward along a random direction."""
    rng = np.random.default_rng(67 + fox)
    L, d, scale = 33, 5, 0.8
    q, k, v, w, beta, lf, do = _bwd_case(rng, L, d, fox)
    g = oracle.path_bwd_head(q, k, v, w, beta, lf, scale, do)
    args = {"q": q, "k": k, "v": v, "w": w, "beta": beta}
    if fox:
        args["log_forget"] = lf

    def loss(a):
        o, _ = oracle.path_fwd_head(a["q"], a["k"], a["v"], a["w"], a["beta"], a.get("log_forget"), scale)
        return float(np.sum(o * do))

    eps = 1e-5
    for name in args:
        delta = rng.standard_normal(np.shape(args[name]))
        ap = dict(args); ap[name] = args[name] + eps * delta
        am = dict(args); am[name] = args[name] - eps * delta
        fd = (loss(ap) - loss(am)) / (2 * eps)
        an = float(np.sum(g["d" + name] * delta))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_c_reverse_mode_beta_zero_is_softmax_attention_grad():
    """beta = 0: dq, dk, dv are those of causal softmax attention (torch's
    scaled_dot_product_attention differentiated in float64) and dw = 0."""
    rng = np.random.default_rng(71)
    L, d, scale = 40, 8, 0.6
    q, k, v, w, _, _, do = _bwd_case(rng, L, d, False)
    beta = np.zeros(L)
    g = oracle.path_bwd_head(q, k, v, w, beta, None, scale, do)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=True,
                                                         scale=scale)[0]
    rq, rk, rv = torch.autograd.grad((o * torch.tensor(do)).sum(), (tq, tk, tv))
    np.testing.assert_allclose(g["dq"], rq.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], rk.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], rv.numpy(), atol=1e-12)
    assert np.all(g["dw"] == 0.0)
