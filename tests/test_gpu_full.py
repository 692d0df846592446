"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: every output of every head is compared with the fp64
oracle, element by element.

  * L=4096 (B=8, H=16, d=64, scale 1/8), L=16384 (B=1, H=16, d=64, 10 % of
    tokens with beta near 2) and L=8192 with forget gates (B=4, H=16,
    d=128): every (b, h, i) row of o and lse, in AUTO and ACCURATE precision.
    The oracle runs once per workload and serves both precisions.
  * The cache-8192 decode step (B=64, H=16, d=64), plain and gated: every
    head's o, lse, updated key cache and appended slot.
  * The scan variants those workloads leave out (gated at d = 64, ungated at
    d = 128) at L = 4096, every row of 8 heads.

The worst errors of each workload, and where they occur, are printed.  Bars
(element-wise max-abs): o <= 2e-2 (bf16 storage), lse <= 1e-3; the updated
bf16 keys within half a bf16 ulp (+1e-5) of the exact fp64 update.
"""
import functools
import time

import numpy as np
import pytest
import torch

import dependent_position_encoding_fwd_amd as pa
import oracle
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_O, TOL_LSE = 2e-2, 1e-3


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@functools.lru_cache(maxsize=1)
def _reference(cfg_id):
    """Seeded inputs of a forward workload and the oracle's o, lse for all of it."""
    c = synthetic.CONFIGS[cfg_id]
    x = synthetic.config_inputs(cfg_id)
    t0 = time.time()
    ro, rl = oracle.path_fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["log_forget"], c.scale)
    print(f"[full] oracle for config {cfg_id} ({c.desc}): {time.time() - t0:.1f} s on "
          f"{oracle.num_threads()} threads", flush=True)
    return x, ro, rl


def _worst(err):
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    return float(err[i]), tuple(int(v) for v in i)


def _run_config(cfg_id, precision):
    c = synthetic.CONFIGS[cfg_id]
    print(f"[full] config {cfg_id} {c.desc} precision={precision}", flush=True)
    x, ro, rl = _reference(cfg_id)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}
    o, lse = pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_forget"], scale=c.scale,
                              precision=precision)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln))
    eo, wo = _worst(np.abs(on - ro))
    el, wl = _worst(np.abs(ln - rl))
    print(f"    all {c.B * c.H} heads x {c.L} rows: max|do|={eo:.3e} at (b,h,i,e)={wo}  "
          f"max|dlse|={el:.3e} at (b,h,i)={wl}", flush=True)
    assert eo <= TOL_O, (eo, wo)
    assert el <= TOL_LSE, (el, wl)


@pytest.mark.parametrize("precision", ["auto", "accurate"])
def test_config2_full(precision):
    _run_config(2, precision)


@pytest.mark.parametrize("precision", ["auto", "accurate"])
def test_config3_full(precision):
    _run_config(3, precision)


@pytest.mark.parametrize("precision", ["auto", "accurate"])
def test_config4_full(precision):
    _run_config(4, precision)


def _bf16_ulp(x):
    ax = np.maximum(np.abs(x), 1e-30)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@pytest.mark.parametrize("fox", [False, True])
def test_decode_config5_full(fox):
    """Every head of the cache-8192 decode step: o, lse, every updated key, the
    appended slot, and (gated) the new gate prefix."""
    c = synthetic.CONFIGS[5]
    n, cap = c.cache_len, c.capacity
    print(f"[full] decode {c.desc} fox={fox}", flush=True)
    x = synthetic.decode_inputs(c.B, c.H, c.d, n, cap, c.dtype, c.seed, fox=fox)
    g = {k: v.to(DEV) for k, v in x.items()}
    if fox:
        cum = torch.cumsum(x["log_f_cache"].double(), dim=-1).float()
        cum_dev = cum.to(DEV)
        o, lse = pa.path_decode_step_fox(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["log_f_t"],
                                         g["k_cache"], g["v_cache"], cum_dev, n, scale=c.scale)
    else:
        o, lse = pa.path_decode_step(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["k_cache"],
                                     g["v_cache"], n, scale=c.scale)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    kc = g["k_cache"].cpu()
    vc = g["v_cache"].cpu()
    cc = cum_dev.cpu() if fox else None
    worst_o = worst_l = worst_k = 0.0
    t0 = time.time()
    for b in range(c.B):
        for h in range(c.H):
            if fox:
                ro, rl, kupd, _ = oracle.path_decode_fox_head(
                    x["q_t"][b, h], x["k_t"][b, h], x["v_t"][b, h], x["w_t"][b, h], float(x["beta_t"][b, h]),
                    float(x["log_f_t"][b, h]), x["k_cache"][b, h, :n], x["v_cache"][b, h, :n], cum[b, h, :n],
                    c.scale)
                # the new prefix is one fp32 addition, c_{n-1} + log f_t
                assert torch.equal(cc[b, h, n], cum[b, h, n - 1] + x["log_f_t"][b, h])
            else:
                ro, rl, kupd = oracle.path_decode_head(x["q_t"][b, h], x["k_t"][b, h], x["v_t"][b, h],
                                                       x["w_t"][b, h], float(x["beta_t"][b, h]),
                                                       x["k_cache"][b, h, :n], x["v_cache"][b, h, :n], c.scale)
            eo = float(np.max(np.abs(on[b, h] - ro)))
            el = abs(float(ln[b, h]) - rl)
            got = kc[b, h, :n].double().numpy()
            ek = float(np.max(np.abs(got - kupd) / (0.5 * _bf16_ulp(kupd) + 1e-5)))
            worst_o, worst_l, worst_k = max(worst_o, eo), max(worst_l, el), max(worst_k, ek)
            assert eo <= TOL_O, (b, h, eo)
            assert el <= TOL_LSE, (b, h, el)
            assert ek <= 1.0, (b, h, ek)
    print(f"    all {c.B * c.H} heads ({time.time() - t0:.1f} s of oracle): max|do|={worst_o:.3e} "
          f"max|dlse|={worst_l:.3e} key error / (half ulp + 1e-5) <= {worst_k:.3f}", flush=True)
    # the new token lands at slot n; nothing else moves
    assert torch.equal(kc[:, :, n], x["k_t"]) and torch.equal(vc[:, :, n], x["v_t"])
    assert torch.equal(vc[:, :, :n], x["v_cache"][:, :, :n])
    if fox:
        assert torch.equal(cc[:, :, :n], cum[:, :, :n])


@pytest.mark.parametrize("precision", ["auto", "accurate"])
@pytest.mark.parametrize("d,fox", [(64, True), (128, False)])
def test_long_other_kernel_variants(d, fox, precision):
    """The scan variants the five workloads leave out, at training length: gated
    attention at d = 64 and ungated at d = 128 (B=1, H=8, L=4096, scale 1/8),
    every row of every head against the oracle."""
    B, H, L, scale = 1, 8, 4096, 0.125
    print(f"[full] B={B} H={H} L={L} d={d} fox={fox} precision={precision}", flush=True)
    x = synthetic.fwd_inputs(B, H, L, d, "bf16", seed=4000 + d + int(fox), fox=fox)
    ro, rl = oracle.path_fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["log_forget"], scale)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}
    o, lse = pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_forget"], scale=scale,
                              precision=precision)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln))
    eo, wo = _worst(np.abs(on - ro))
    el, wl = _worst(np.abs(ln - rl))
    print(f"    all {B * H} heads x {L} rows: max|do|={eo:.3e} at {wo}  max|dlse|={el:.3e} at {wl}", flush=True)
    assert eo <= TOL_O, (eo, wo)
    assert el <= TOL_LSE, (el, wl)
