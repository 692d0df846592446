"""GPU check of path_decode_step_noalloc (the decode step whose scratch lives in
a static device array) against path_decode_step (caller workspace), through the
C ABI: two calls in a row, the second on a smaller input, each compared bit for
bit (o, lse and both caches) with the workspace entry point on its own copy of
the same inputs.  The two share their kernels, so the results must be identical."""
import pytest
import torch

import dependent_position_encoding_fwd_amd as pa
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pair(B, H, d, n, cap, dtype, seed):
    print(f"[noalloc] B={B} H={H} d={d} len={n} cap={cap} {dtype} seed={seed}", flush=True)
    x = synthetic.decode_inputs(B, H, d, n, cap, dtype, seed)
    a = {k: v.to(DEV) for k, v in x.items()}
    b = {k: v.to(DEV) for k, v in x.items()}
    o1, l1 = pa.path_decode_step(a["q_t"], a["k_t"], a["v_t"], a["w_t"], a["beta_t"], a["k_cache"], a["v_cache"],
                                 n, scale=0.7)
    o2, l2 = pa.path_decode_step_noalloc(b["q_t"], b["k_t"], b["v_t"], b["w_t"], b["beta_t"], b["k_cache"],
                                         b["v_cache"], n, scale=0.7)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
    assert torch.equal(a["k_cache"], b["k_cache"])
    assert torch.equal(a["v_cache"], b["v_cache"])
    assert bool(torch.isfinite(o2.float()).all())


def test_noalloc_matches_workspace_step_twice_second_smaller():
    _pair(8, 16, 64, 8192, 8200, "bf16", 71)   # 128 heads x 8 chunks of partials
    _pair(2, 3, 64, 700, 710, "bf16", 72)      # smaller: fewer heads, one chunk


def test_noalloc_d128_and_fp32():
    _pair(2, 4, 128, 3000, 3001, "f32", 73)
    _pair(1, 2, 128, 0, 1, "bf16", 74)         # empty cache: only the new key

