"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars (element-wise max-abs, on identical seeded inputs):
  o: <= 2e-2 for bf16 storage, <= 1e-4 for fp32 storage;  lse: <= 1e-3.
Prepare intermediates are fp32 arithmetic: compared at 2e-5 absolute (their
magnitudes are O(1): |tinv| <= ~2, unit-norm w).
Decode cache: the updated bf16 key must be the round-to-nearest of the exact
fp64 value up to fp32 evaluation error (<= half a bf16 ulp + 1e-5); the new
slot must equal k_t, v_t bit for bit; slots past it must be untouched.
"""
import numpy as np
import pytest
import torch

import dependent_position_encoding_fwd_amd as pa
import oracle
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_O = {"bf16": 2e-2, "f32": 1e-4}
TOL_LSE = 1e-3


def _dev(x):
    return {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in x.items()}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _fwd_case(B, H, L, d, dtype, scale, seed, fox=False, near2=0.0, beta_override=None, precision="auto"):
    print(f"[fwd] B={B} H={H} L={L} d={d} {dtype} scale={scale} fox={fox} seed={seed} "
          f"beta={beta_override} prec={precision}", flush=True)
    x = synthetic.fwd_inputs(B, H, L, d, dtype, seed, near2_frac=near2, fox=fox)
    if beta_override is not None:
        x["beta"] = torch.full_like(x["beta"], float(beta_override))
    g = _dev(x)
    o, lse = pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_forget"], scale=scale,
                              precision=precision)
    torch.cuda.synchronize()
    ro, rl = oracle.path_fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["log_forget"], scale)
    eo = np.max(np.abs(_np(o) - ro))
    el = np.max(np.abs(_np(lse) - rl))
    print(f"    max|do|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert np.all(np.isfinite(_np(o))) and np.all(np.isfinite(_np(lse)))
    assert eo <= TOL_O[dtype], eo
    assert el <= TOL_LSE, el
    return o, lse


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_small(dtype, L, d):
    _fwd_case(1, 2, L, d, dtype, 1.0, seed=L * 7 + d)


@pytest.mark.parametrize("L", [129, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fox", [False, True])
def test_fwd_bf16_accurate(L, d, fox):
    _fwd_case(1, 3, L, d, "bf16", 1.0, seed=L + d + fox, fox=fox, precision="accurate")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_fox(dtype, d):
    _fwd_case(2, 2, 300, d, dtype, 1.0, seed=d + 3, fox=True)


@pytest.mark.parametrize("BH", [(1, 8), (2, 8), (3, 8)])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_xcd_head_order(BH, d):
    # B*H a multiple of 8: workgroups are dealt to the 8 XCDs by head, heads in
    # pairs (8: one unpaired head per XCD; 16: one pair; 24: a pair and one unpaired)
    B, H = BH
    _fwd_case(B, H, 330, d, "bf16", 0.5, seed=B * 10 + d, fox=(B == 2))


@pytest.mark.parametrize("beta", [0.0, 1.0, 2.0])
def test_fwd_beta_edges(beta):
    # beta = 1 with unit w makes every H singular; beta = 0 is plain attention
    _fwd_case(1, 2, 260, 64, "bf16", 0.5, seed=int(beta * 10) + 1, beta_override=beta)


def test_fwd_near2_and_scale():
    _fwd_case(1, 3, 384, 64, "bf16", 1.0, seed=41, near2=0.1)
    _fwd_case(1, 3, 384, 64, "bf16", 0.125, seed=42)


def test_fwd_config1_full():
    c = synthetic.CONFIGS[1]
    _fwd_case(c.B, c.H, c.L, c.d, c.dtype, c.scale, c.seed)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_deterministic_and_stages(d):
    x = _dev(synthetic.fwd_inputs(1, 4, 333, d, "bf16", 5, fox=True))
    args = (x["q"], x["k"], x["v"], x["w"], x["beta"], x["log_forget"])
    o1, l1 = pa.path_attn_fwd(*args, scale=0.3)
    o2, l2 = pa.path_attn_fwd(*args, scale=0.3)
    ws = pa.path_fwd_stage_prepare(*args, scale=0.3)
    o3, l3 = pa.path_fwd_stage_scan(*args[:5], ws, log_forget=args[5], scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_prepare_parity(dtype, d):
    B, H, L = 1, 2, 200
    x = synthetic.fwd_inputs(B, H, L, d, dtype, 77 + d, fox=True)
    x["beta"][0, 0, 5] = 0.0
    x["beta"][0, 1, 70] = 1.0
    g = _dev(x)
    out = pa.path_prepare(g["q"], g["k"], g["w"], g["beta"], g["log_forget"])
    torch.cuda.synchronize()
    Nb = (L + 63) // 64
    for b in range(B):
        for h in range(H):
            for n in range(Nb):
                sl = slice(n * 64, min(L, (n + 1) * 64))
                cnt = sl.stop - sl.start
                tinv = oracle.ut_tinv(x["w"][b, h, sl], x["beta"][b, h, sl])
                qh, kh, pt = oracle.block_adjust(x["q"][b, h, sl], x["k"][b, h, sl], x["w"][b, h, sl],
                                                 x["beta"][b, h, sl])
                gt = _np(out["tinv"][b, h, n])
                np.testing.assert_allclose(gt[:cnt, :cnt], tinv, atol=2e-5)
                assert np.all(gt[cnt:, :] == 0) and np.all(gt[:, cnt:] == 0)
                np.testing.assert_allclose(_np(out["qhat"][b, h, sl]), qh, atol=2e-5)
                np.testing.assert_allclose(_np(out["khat"][b, h, sl]), kh, atol=2e-5)
                np.testing.assert_allclose(_np(out["pT"][b, h, n]), pt, atol=2e-5)
            np.testing.assert_allclose(_np(out["cum"][b, h]), oracle.prefix_sum(x["log_forget"][b, h]), atol=1e-5)


def _bf16_ulp(x):
    ax = np.maximum(np.abs(x), 1e-30)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def _decode_case(B, H, d, n, cap, dtype, scale, seed, heads_to_check=None, fox=False, log_f_t=None):
    print(f"[decode] B={B} H={H} d={d} len={n} cap={cap} {dtype} seed={seed} fox={fox} log_f_t={log_f_t}",
          flush=True)
    x = synthetic.decode_inputs(B, H, d, n, cap, dtype, seed, fox=fox)
    g = _dev(x)
    if fox:
        if log_f_t is not None:
            x["log_f_t"] = torch.full_like(x["log_f_t"], float(log_f_t))
            g["log_f_t"] = x["log_f_t"].to(DEV)
        # Cache state: running gate prefixes c_j of the cached tokens (fp64 sums
        # stored fp32); slots past the cache hold a sentinel that must survive.
        cum = torch.cumsum(x["log_f_cache"].double(), dim=-1).float()
        cum[..., n:] = 12345.0
        cum_dev = cum.to(DEV)
        o, lse = pa.path_decode_step_fox(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["log_f_t"],
                                         g["k_cache"], g["v_cache"], cum_dev, n, scale=scale)
    else:
        o, lse = pa.path_decode_step(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["k_cache"],
                                     g["v_cache"], n, scale=scale)
    torch.cuda.synchronize()
    heads = heads_to_check or [(b, h) for b in range(B) for h in range(H)]
    kc_gpu = g["k_cache"]
    for (b, h) in heads:
        if fox:
            ro, rl, kupd, _ = oracle.path_decode_fox_head(
                x["q_t"][b, h], x["k_t"][b, h], x["v_t"][b, h], x["w_t"][b, h], float(x["beta_t"][b, h]),
                float(x["log_f_t"][b, h]), x["k_cache"][b, h, :n], x["v_cache"][b, h, :n], cum[b, h, :n], scale)
            # The new prefix is one fp32 addition, c_{n-1} + log f_t (c_{-1} = 0).
            prev = cum[b, h, n - 1] if n > 0 else torch.zeros((), dtype=torch.float32)
            want = prev + x["log_f_t"][b, h]
            got_c = cum_dev[b, h].cpu()
            assert torch.equal(got_c[n], want)
            assert torch.equal(got_c[:n], cum[b, h, :n]) and torch.equal(got_c[n + 1:], cum[b, h, n + 1:])
        else:
            ro, rl, kupd = oracle.path_decode_head(x["q_t"][b, h], x["k_t"][b, h], x["v_t"][b, h], x["w_t"][b, h],
                                                   float(x["beta_t"][b, h]), x["k_cache"][b, h, :n],
                                                   x["v_cache"][b, h, :n], scale)
        assert np.max(np.abs(_np(o[b, h]) - ro)) <= TOL_O[dtype]
        assert abs(float(lse[b, h]) - rl) <= TOL_LSE
        got = _np(kc_gpu[b, h, :n])
        if dtype == "bf16":
            assert np.all(np.abs(got - kupd) <= 0.5 * _bf16_ulp(kupd) + 1e-5)
        else:
            assert np.all(np.abs(got - kupd) <= 1e-5)
        assert torch.equal(kc_gpu[b, h, n].cpu(), x["k_t"][b, h])
        assert torch.equal(g["v_cache"][b, h, n].cpu(), x["v_t"][b, h])
        if n + 1 < cap:
            assert torch.equal(kc_gpu[b, h, n + 1:].cpu(), x["k_cache"][b, h, n + 1:])
        assert torch.equal(g["v_cache"][b, h, :n].cpu(), x["v_cache"][b, h, :n])
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [0, 1, 100, 1024, 1500])
def test_decode_small(dtype, d, n):
    _decode_case(2, 3, d, n, n + 7, dtype, 1.0, seed=n + d)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [0, 1, 100, 1500])
def test_decode_fox_small(dtype, d, n):
    _decode_case(2, 3, d, n, n + 7, dtype, 1.0, seed=n + d + 7, fox=True)


@pytest.mark.parametrize("log_f_t", [0.0, -800.0])
def test_decode_fox_open_and_closed_gate(log_f_t):
    """An open gate at t (log f_t = 0) and a closed one (-800: every cached key's
    weight underflows to 0, so o = v_t and lse is the new key's logit)."""
    o, lse = _decode_case(2, 2, 64, 700, 720, "f32", 0.7, seed=5, fox=True, log_f_t=log_f_t)
    if log_f_t < -100:
        x = synthetic.decode_inputs(2, 2, 64, 700, 720, "f32", 5, fox=True)
        assert torch.allclose(o.cpu(), x["v_t"], atol=1e-6)


@pytest.mark.parametrize("d", [64, 128])
def test_fox_decode_from_empty_matches_forward_rows(d):
    """Gated decode steps from an empty cache, each appending its key and its gate
    prefix, reproduce the gated forward's rows; the prefix cache they build is the
    running sum of the gates."""
    L, B, H = 96, 1, 2
    x = synthetic.fwd_inputs(B, H, L, d, "f32", 321, fox=True)
    ro, rl = oracle.path_fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], x["log_forget"], 0.5)
    g = _dev(x)
    kc = torch.zeros(B, H, L, d, device=DEV)
    vc = torch.zeros(B, H, L, d, device=DEV)
    cc = torch.zeros(B, H, L, device=DEV)
    for t in range(L):
        o, lse = pa.path_decode_step_fox(g["q"][:, :, t].contiguous(), g["k"][:, :, t].contiguous(),
                                         g["v"][:, :, t].contiguous(), g["w"][:, :, t].contiguous(),
                                         g["beta"][:, :, t].contiguous(), g["log_forget"][:, :, t].contiguous(),
                                         kc, vc, cc, t, scale=0.5)
        assert np.max(np.abs(_np(o) - ro[:, :, t])) <= 1e-4
        assert np.max(np.abs(_np(lse) - rl[:, :, t])) <= 1e-4
    want = np.stack([[oracle.prefix_sum(x["log_forget"][b, h]) for h in range(H)] for b in range(B)])
    assert np.max(np.abs(_np(cc) - want)) <= 1e-4


def test_decode_after_prefill_matches_forward_rows():
    """Decode steps on the GPU, with the cache updated in place, reproduce the
    forward's rows (both checked against the oracle's forward)."""
    L, d, B, H = 96, 64, 1, 2
    x = synthetic.fwd_inputs(B, H, L, d, "f32", 123)
    ro, rl = oracle.path_fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], None, 0.5)
    g = _dev(x)
    kc = torch.zeros(B, H, L, d, device=DEV)
    vc = torch.zeros(B, H, L, d, device=DEV)
    for t in range(L):
        o, lse = pa.path_decode_step(g["q"][:, :, t].contiguous(), g["k"][:, :, t].contiguous(),
                                     g["v"][:, :, t].contiguous(), g["w"][:, :, t].contiguous(),
                                     g["beta"][:, :, t].contiguous(), kc, vc, t, scale=0.5)
        assert np.max(np.abs(_np(o) - ro[:, :, t])) <= 1e-4
        assert np.max(np.abs(_np(lse) - rl[:, :, t])) <= 1e-4
