"""GPU parity of the backward pass: path_attn_bwd (through the C ABI) against
the fp64 gradients of the oracle (oracle/grad.py) on identical seeded inputs.

The oracle differentiates <dO, o> in float64 from the stored input values:
torch.autograd of the defining loop (oracle/grad.py) up to L = 600, and at
training length (L = 4096 and 8192, whole heads) the hand-written C reverse
mode of the same loop (oracle.path_bwd_head), pinned against the former.
The backward is fed the oracle's o (stored in the input dtype) and lse (fp32),
as a forward would hand them over.  Bar, for every gradient tensor G: the
largest element error is at most tol * max|G_ref|, with tol = 1e-4 for fp32
storage and 2e-2 for bf16 storage (the gradients are rounded to bf16, and the
softmax row terms D_i = dO_i . o_i use the bf16-rounded o).

A gradient tensor can vanish exactly: with one key (L = 1) the softmax weight
is 1 whatever the logit, so dq, dk, dw and dbeta are 0 and the kernel returns
the fp32 rounding of dS = p (dO . v - dO . o), two equal dot products summed
in different orders.  A relative bar is undefined there, so for a reference
tensor that is exactly zero (and only then) the bar is tol times 1 % of
max|dv_ref|, the scale of the incoming gradient p^T dO.
"""
import numpy as np
import pytest
import torch

import dependent_position_encoding_fwd_amd as pa
import oracle
import synthetic
from oracle import grad

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _cmp(name, got, ref, tol, floor):
    err = float(np.max(np.abs(_np(got) - ref))) if ref.size else 0.0
    mag = float(np.max(np.abs(ref))) if ref.size else 0.0
    print(f"  {name}: max|err|={err:.3e} max|ref|={mag:.3e} ratio={err / max(mag, 1e-30):.2e}", flush=True)
    assert mag > 0 or floor is not None, (name, "reference is exactly zero")
    assert err <= tol * (mag if mag > 0 else floor), (name, err, mag, floor)


def _bwd_case(B, H, L, d, dtype, scale, seed, fox, chain_forward=False, mutate=None):
    print(f"[bwd] B={B} H={H} L={L} d={d} {dtype} scale={scale} fox={fox} seed={seed} "
          f"chain_forward={chain_forward} mutate={mutate is not None}", flush=True)
    x = synthetic.fwd_inputs(B, H, L, d, dtype, seed, fox=fox)
    if mutate is not None:
        mutate(x)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(B, H, L, d, generator=g).to(synthetic.DTYPES[dtype])
    refs = {}
    o_ref = np.zeros((B, H, L, d))
    lse_ref = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            lf = None if x["log_forget"] is None else x["log_forget"][b, h]
            r = grad.path_bwd_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["w"][b, h], x["beta"][b, h], lf,
                                   scale, do[b, h])
            T = grad._t
            ot, lt = grad.forward_torch(T(x["q"][b, h]), T(x["k"][b, h]), T(x["v"][b, h]), T(x["w"][b, h]),
                                        T(x["beta"][b, h]), None if lf is None else T(lf), scale)
            o_ref[b, h], lse_ref[b, h] = ot.numpy(), lt.numpy()
            for n, val in r.items():
                if val is not None:
                    refs.setdefault(n, np.zeros((B, H) + val.shape))[b, h] = val
    gx = {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}
    if chain_forward:
        o, lse = pa.path_attn_fwd(gx["q"], gx["k"], gx["v"], gx["w"], gx["beta"], gx["log_forget"], scale=scale)
    else:
        o = torch.tensor(o_ref).to(synthetic.DTYPES[dtype]).to(DEV)
        lse = torch.tensor(lse_ref, dtype=torch.float32).to(DEV)
    dq, dk, dv, dw, dbeta, dlf = pa.path_attn_bwd(gx["q"], gx["k"], gx["v"], gx["w"], gx["beta"], o, lse,
                                                  do.to(DEV), gx["log_forget"], scale=scale)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    floor = 1e-2 * float(np.max(np.abs(refs["dv"])))
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dw", dw), ("dbeta", dbeta)):
        _cmp(name, got, refs[name], tol, floor)
    if fox:
        _cmp("dlog_forget", dlf, refs["dlog_forget"], tol, floor)
    else:
        assert dlf is None


@pytest.mark.parametrize("L,d,fox", [(1, 64, False), (64, 64, True), (200, 64, False), (200, 64, True),
                                     (130, 128, True), (300, 128, False)])
def test_bwd_f32(L, d, fox):
    _bwd_case(1, 2, L, d, "f32", 0.3, seed=L + d + fox, fox=fox)


@pytest.mark.parametrize("L,d,fox", [(200, 64, True), (130, 128, False), (40, 64, False), (128, 64, True),
                                     (40, 128, False), (200, 128, True)])
def test_bwd_bf16(L, d, fox):
    _bwd_case(1, 2, L, d, "bf16", 0.3, seed=L + d + 7 * fox, fox=fox)


def _special_transitions(x):
    """Tokens t = 0 (mod 7) get beta = 0 (H = I), t = 3 (mod 7) beta = 2 with a
    unit w (an exact reflection), and t = 5 (mod 7) a w of norm 1.25 with
    beta = 1 / |w|^2 (H a projection: singular)."""
    L = x["beta"].shape[-1]
    t = torch.arange(L)
    dt = x["w"].dtype
    w = x["w"].double()
    beta = x["beta"].clone()
    beta[..., t % 7 == 0] = 0.0
    beta[..., t % 7 == 3] = 2.0
    w[..., t % 7 == 5, :] *= 1.25
    n2 = (w[..., t % 7 == 5, :] ** 2).sum(-1)
    beta[..., t % 7 == 5] = (1.0 / n2).to(beta.dtype)
    x["w"] = w.to(dt)
    x["beta"] = beta


@pytest.mark.parametrize("fox", [False, True])
def test_bwd_special_transitions_f32(fox):
    """beta = 0, exact reflections and singular (projection) transitions, over
    three blocks with a ragged end: the in-block gradients, whose triangular
    factor carries no division by beta or by 1 - beta |w|^2, stay exact."""
    _bwd_case(1, 2, 150, 64, "f32", 0.3, seed=150 + fox, fox=fox, mutate=_special_transitions)


@pytest.mark.parametrize("fox,d", [(False, 64), (True, 64), (False, 128), (True, 128)])
def test_bwd_special_transitions_bf16(fox, d):
    """The same transitions with bf16 storage, through the 16-bit cross-block
    kernels and the matrix-form in-block kernels: w is rounded to bf16 after
    scaling, so the projections are singular only up to that rounding."""
    _bwd_case(1, 2, 150, d, "bf16", 0.3, seed=151 + fox + (d - 64), fox=fox, mutate=_special_transitions)


def test_bwd_long_f32():
    """Ten blocks: transports across up to nine block transitions."""
    _bwd_case(1, 1, 600, 64, "f32", 0.25, seed=600, fox=True)


def test_bwd_after_gpu_forward_bf16():
    """The backward fed the GPU forward's own o and lse."""
    _bwd_case(2, 2, 257, 64, "bf16", 0.125, seed=257, fox=False, chain_forward=True)


def test_bwd_deterministic_up_to_atomics():
    """Two runs agree to fp32 summation-order differences."""
    x = synthetic.fwd_inputs(1, 2, 300, 64, "f32", 11, fox=True)
    g = {n: t.to(DEV) for n, t in x.items()}
    do = torch.randn(1, 2, 300, 64, generator=torch.Generator().manual_seed(5)).to(DEV)
    o, lse = pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_forget"], scale=0.5)
    r1 = pa.path_attn_bwd(g["q"], g["k"], g["v"], g["w"], g["beta"], o, lse, do, g["log_forget"], scale=0.5)
    r2 = pa.path_attn_bwd(g["q"], g["k"], g["v"], g["w"], g["beta"], o, lse, do, g["log_forget"], scale=0.5)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("fox", [False, True])
def test_bwd_full_length_directional(fox):
    """At the L = 4096 workload length (64 blocks, 2016 block pairs per head),
    where the fp64 gradient oracle is too slow, the gradients must give the
    directional derivative of f = sum(dO * o) along a random direction of all
    inputs: sum_x <grad_x, v_x> against the central difference
    (f(x + v) - f(x - v)) / 2 of the GPU forward (fp32).  The O(|v|^3) error and
    fp32 rounding of f keep the two within 1 % of each other."""
    B, H, L, d, scale = 1, 2, 4096, 64, 0.125
    x = synthetic.fwd_inputs(B, H, L, d, "f32", 4096 + fox, fox=fox)
    gen = torch.Generator().manual_seed(77 + fox)
    names = ["q", "k", "v", "w", "beta"] + (["log_forget"] if fox else [])
    g = {n: x[n].to(DEV) for n in names}
    do = torch.randn(B, H, L, d, generator=gen).to(DEV)
    step = {n: (1e-3 * torch.randn(g[n].shape, generator=gen)).to(DEV) for n in names}

    def f(sign):
        y = {n: g[n] + sign * step[n] for n in names}
        o, _ = pa.path_attn_fwd(y["q"], y["k"], y["v"], y["w"], y["beta"], y.get("log_forget"), scale=scale)
        return float((o.double() * do.double()).sum())

    o, lse = pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g.get("log_forget"), scale=scale)
    grads = pa.path_attn_bwd(g["q"], g["k"], g["v"], g["w"], g["beta"], o, lse, do, g.get("log_forget"), scale=scale)
    torch.cuda.synchronize()
    gmap = dict(zip(["q", "k", "v", "w", "beta", "log_forget"], grads))
    dirder = sum(float((gmap[n].double() * step[n].double()).sum()) for n in names)
    fd = (f(1.0) - f(-1.0)) / 2.0
    print(f"  L={L} fox={fox}: <grad, v> = {dirder:.6e}, central difference = {fd:.6e}", flush=True)
    assert abs(dirder - fd) <= 1e-2 * abs(fd), (dirder, fd)


def _bwd_full_heads(H, L, d, dtype, scale, seed, fox):
    """Whole heads at training length, every gradient element against the C
    reverse mode of the defining loop (oracle.path_bwd_head); the backward is
    fed the oracle's o (stored in the input dtype) and lse."""
    print(f"[bwd-full] H={H} L={L} d={d} {dtype} scale={scale} fox={fox} seed={seed}", flush=True)
    x = synthetic.fwd_inputs(1, H, L, d, dtype, seed, fox=fox)
    do = torch.randn(1, H, L, d, generator=torch.Generator().manual_seed(seed + 1000)).to(synthetic.DTYPES[dtype])
    refs, o_ref, lse_ref = {}, np.zeros((1, H, L, d)), np.zeros((1, H, L))
    for h in range(H):
        lf = None if x["log_forget"] is None else x["log_forget"][0, h]
        args = (x["q"][0, h], x["k"][0, h], x["v"][0, h], x["w"][0, h], x["beta"][0, h], lf, scale)
        o_ref[0, h], lse_ref[0, h] = oracle.path_fwd_head(*args)
        r = oracle.path_bwd_head(*args, do[0, h])
        for n, val in r.items():
            if val is not None:
                refs.setdefault(n, np.zeros((1, H) + val.shape))[0, h] = val
    gx = {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}
    o = torch.tensor(o_ref).to(synthetic.DTYPES[dtype]).to(DEV)
    lse = torch.tensor(lse_ref, dtype=torch.float32).to(DEV)
    grads = pa.path_attn_bwd(gx["q"], gx["k"], gx["v"], gx["w"], gx["beta"], o, lse, do.to(DEV), gx["log_forget"],
                             scale=scale)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dw", "dbeta") + (("dlog_forget",) if fox else ())
    for name, got in zip(names, grads):
        _cmp(name, got, refs[name], TOL[dtype], None)


def test_bwd_full_length_elementwise_bf16():
    """Four whole heads of the L = 4096 workload (d = 64, scale 1/8, bf16): 64
    blocks, 2016 block pairs per head, every gradient element."""
    _bwd_full_heads(4, 4096, 64, "bf16", 0.125, 4100, False)


def test_bwd_full_length_elementwise_bf16_gated_ragged():
    """One gated head past the workload length with a ragged end (L = 4133:
    65 blocks, the last of 37 tokens), bf16 at d = 64: the 16-bit cross-block
    kernels with gates, every gradient element."""
    _bwd_full_heads(1, 4133, 64, "bf16", 0.125, 4103, True)


def test_bwd_full_length_elementwise_f32_gated():
    _bwd_full_heads(1, 4096, 64, "f32", 0.125, 4101, True)


def test_bwd_full_length_elementwise_d128_gated():
    """One whole head at the gated d = 128 workload's length (L = 8192, bf16)."""
    _bwd_full_heads(1, 8192, 128, "bf16", 1.0, 4102, True)
