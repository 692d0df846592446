"""GPU checks of the bf16 forward at the edges of the input range that
include/path_attn.h states for PATH_BF16, against the fp64 oracle on the same
stored values:

  * values: |v| up to 1e5 everywhere; single entries of +-6e4 and +-1e5 in a
    few blocks (blocks at different power-of-two scales within one head); one
    block of values near 1e30 beside ordinary ones;
  * queries and keys: q and k scaled by 1e3 (logits near 1e6; |k|_2 <= 2^15
    and scale |q|_2 <= 2^14 still hold) and by 1e-4 (logits near 0).

Bars, as the header states them (per head): |do| <= 2e-2 + 2^-8 max_j |v_j|;
|dlse_i| <= 1e-3 + 2^-18 max_j |s_ij|; every output finite.
"""
import numpy as np
import pytest
import torch

import dependent_position_encoding_fwd_amd as pa
import oracle
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _v_large_all(x):
    x["v"] = (x["v"].float() * 2.5e4).to(torch.bfloat16)


def _v_edges(x):
    v = x["v"].float()
    v[:, :, 10, 3], v[:, :, 11, 4] = 6e4, -6e4          # block 0: 2^15 <= |v| < 2^16
    v[:, :, 130, 0], v[:, :, 131, 1] = 1e5, -1e5        # block 2: 2^16 <= |v| < 2^17
    x["v"] = v.to(torch.bfloat16)


def _v_huge_block(x):
    v = x["v"].float()
    v[:, :, 64:128] *= 1e30                             # block 1 only
    x["v"] = v.to(torch.bfloat16)


def _qk_big(x):
    x["q"] = (x["q"].float() * 1e3).to(torch.bfloat16)
    x["k"] = (x["k"].float() * 1e3).to(torch.bfloat16)


def _qk_small(x):
    x["q"] = (x["q"].float() * 1e-4).to(torch.bfloat16)
    x["k"] = (x["k"].float() * 1e-4).to(torch.bfloat16)


CASES = {"v_large_all": _v_large_all, "v_edges": _v_edges, "v_huge_block": _v_huge_block,
         "qk_big": _qk_big, "qk_small": _qk_small}


@pytest.mark.parametrize("precision", ["auto", "accurate"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", sorted(CASES))
def test_bf16_range_edges(case, d, precision):
    L, H, scale = 300, 2, 0.125
    print(f"[range] {case} d={d} L={L} {precision}", flush=True)
    x = synthetic.fwd_inputs(1, H, L, d, "bf16", seed=500 + d + len(case))
    CASES[case](x)
    g = {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}
    o, lse = pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], None, scale=scale, precision=precision)
    torch.cuda.synchronize()
    on = o.float().cpu().numpy().astype(np.float64)
    ln = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln))
    for h in range(H):
        ro, rl, lg = oracle.path_fwd_head(x["q"][0, h], x["k"][0, h], x["v"][0, h], x["w"][0, h], x["beta"][0, h],
                                          None, scale, rows=np.arange(L), want_logits=True)
        vmax = float(x["v"][0, h].float().abs().max())
        smax = np.max(np.where(np.isfinite(lg), np.abs(lg), 0.0), axis=1)
        eo = np.abs(on[0, h] - ro)
        el = np.abs(ln[0, h] - rl)
        bo = 2e-2 + 2.0 ** -8 * vmax
        bl = 1e-3 + 2.0 ** -18 * smax
        print(f"    head {h}: max|v|={vmax:.3g} max|do|={eo.max():.3e} (bar {bo:.3g})  "
              f"max|dlse|={el.max():.3e} worst lse ratio {np.max(el / bl):.3f}", flush=True)
        assert eo.max() <= bo, (h, eo.max(), bo)
        assert np.all(el <= bl), (h, el.max())
