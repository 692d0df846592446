"""GPU parity of the paged, variable-length decode step (path_decode_step_paged,
through the C ABI) against the fp64 oracle's decode step on each sequence's
logically contiguous cache [PaTH summary (gist.science 2505.16381) §3
"Inferência"]: the page layout is storage only, so every (b, h) must give what
path_decode_head gives on its first cache_lens[b] keys, its pages must hold the
updated keys and the appended token, and no other slot may change.  Pages are
assigned in a seeded random order, with pages no sequence maps.
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


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _bf16_ulp(x):
    ax = np.maximum(np.abs(x), 1e-30)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def _paginate(kc, vc, lens, page, extra, seed):
    """Scatter [B,H,cap,d] caches into shuffled pages [NP,H,page,d]; sequence b
    maps ceil((lens[b] + 1) / page) pages (room for the appended token).  Slots
    outside the sequences hold seeded noise that must survive the step."""
    B, H, cap, d = kc.shape
    g = torch.Generator().manual_seed(seed)
    need = [(int(n) + page) // page for n in lens]
    MP = max(need)
    NP = sum(need) + extra
    perm = torch.randperm(NP, generator=g)
    table = torch.full((B, MP), -1, dtype=torch.int32)
    kp = torch.randn(NP, H, page, d, generator=g).to(kc.dtype)
    vp = torch.randn(NP, H, page, d, generator=g).to(kc.dtype)
    i = 0
    for b in range(B):
        for lp in range(need[b]):
            pg = int(perm[i])
            i += 1
            table[b, lp] = pg
            lo, hi = lp * page, min((lp + 1) * page, int(lens[b]))
            if hi > lo:
                kp[pg, :, : hi - lo] = kc[b, :, lo:hi]
                vp[pg, :, : hi - lo] = vc[b, :, lo:hi]
    return kp, vp, table


def _gather(pages, table, b, n, page):
    rows = [pages[int(table[b, j // page]), :, j % page] for j in range(n)]
    return torch.stack(rows, dim=1) if rows else pages.new_zeros(pages.shape[1], 0, pages.shape[3])


def _paginate_cum(cum, table, lens, page, num_pages, seed):
    """The gate-prefix cache [B,H,cap] in the key pages' layout [NP,H,page], with
    seeded noise in every slot no sequence owns."""
    B, H, _ = cum.shape
    g = torch.Generator().manual_seed(seed)
    cp = torch.randn(num_pages, H, page, generator=g)
    for b in range(B):
        for lp in range((int(lens[b]) + page) // page):
            lo, hi = lp * page, min((lp + 1) * page, int(lens[b]))
            if hi > lo:
                cp[int(table[b, lp]), :, : hi - lo] = cum[b, :, lo:hi]
    return cp


def _paged_case(B, H, d, lens, page, dtype, scale, seed, extra=3, heads=None, fox=False):
    print(f"[paged] B={B} H={H} d={d} lens={list(lens)} page={page} {dtype} seed={seed} fox={fox}", flush=True)
    cap = max(lens) + 1
    x = synthetic.decode_inputs(B, H, d, cap - 1, cap, dtype, seed, fox=fox)
    kp, vp, table = _paginate(x["k_cache"], x["v_cache"], lens, page, extra, seed + 1)
    kp0, vp0 = kp.clone(), vp.clone()
    g = {n: t.to(DEV) for n, t in x.items()}
    kd, vd, td = kp.to(DEV), vp.to(DEV), table.to(DEV)
    ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
    if fox:
        # the running gate prefixes c_j of each sequence's cached tokens (fp64 sums stored fp32)
        cum = torch.cumsum(x["log_f_cache"].double(), dim=-1).float()
        cp = _paginate_cum(cum, table, lens, page, kp.shape[0], seed + 2)
        cp0, cd = cp.clone(), cp.to(DEV)
        o, lse = pa.path_decode_step_paged_fox(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["log_f_t"],
                                               kd, vd, cd, td, ld, max(lens), scale=scale)
    else:
        o, lse = pa.path_decode_step_paged(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], kd, vd, td, ld,
                                           max(lens), scale=scale)
    torch.cuda.synchronize()
    kg, vg = kd.cpu(), vd.cpu()
    cg = cd.cpu() if fox else None
    touched = torch.zeros(kp.shape[0], H, page, dtype=torch.bool)
    for b in range(B):
        n = int(lens[b])
        for j in range(n + 1):
            touched[int(table[b, j // page]), :, j % page] = True
        if fox:
            # c_t = c_{n-1} + log f_t in fp32 (log f_t alone on an empty cache), at the new key's slot
            pg, sl = int(table[b, n // page]), n % page
            prev = cum[b, :, n - 1] if n > 0 else torch.zeros(H)
            assert torch.equal(cg[pg, :, sl], prev + x["log_f_t"][b]), b
        for h in range(H) if heads is None else [hh for bb, hh in heads if bb == b]:
            if fox:
                ro, rl, kupd, _ = oracle.path_decode_fox_head(
                    x["q_t"][b, h], x["k_t"][b, h], x["v_t"][b, h], x["w_t"][b, h], float(x["beta_t"][b, h]),
                    float(x["log_f_t"][b, h]), x["k_cache"][b, h, :n], x["v_cache"][b, h, :n], cum[b, h, :n], scale)
            else:
                ro, rl, kupd = oracle.path_decode_head(x["q_t"][b, h], x["k_t"][b, h], x["v_t"][b, h],
                                                       x["w_t"][b, h], float(x["beta_t"][b, h]),
                                                       x["k_cache"][b, h, :n], x["v_cache"][b, h, :n], scale)
            assert np.max(np.abs(_np(o[b, h]) - ro)) <= TOL_O[dtype], (b, h)
            assert abs(float(lse[b, h]) - rl) <= TOL_LSE, (b, h)
            got = _np(_gather(kg, table, b, n, page)[h])
            if dtype == "bf16":
                assert np.all(np.abs(got - kupd) <= 0.5 * _bf16_ulp(kupd) + 1e-5)
            else:
                assert np.all(np.abs(got - kupd) <= 1e-5)
            pg, sl = int(table[b, n // page]), n % page
            assert torch.equal(kg[pg, h, sl], x["k_t"][b, h]) and torch.equal(vg[pg, h, sl], x["v_t"][b, h])
            assert torch.equal(_gather(vg, table, b, n, page)[h], x["v_cache"][b, h, :n])
    # every slot no sequence owns (and every value slot but the appended ones) is untouched
    assert torch.equal(kg[~touched], kp0[~touched])
    assert torch.equal(vg[~touched], vp0[~touched])
    if fox:
        appended = torch.zeros_like(touched)
        for b in range(B):
            n = int(lens[b])
            appended[int(table[b, n // page]), :, n % page] = True
        assert torch.equal(cg[~appended], cp0[~appended])
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page", [16, 100])
def test_paged_small(dtype, d, page):
    _paged_case(3, 2, d, [0, 150, 1333], page, dtype, 1.0, seed=page + d)


def test_paged_page_boundaries():
    """Lengths that end on, just before and just after page boundaries."""
    _paged_case(4, 2, 64, [63, 64, 65, 128], 64, "bf16", 0.5, seed=9)


def test_paged_matches_contiguous_bitwise():
    """Equal lengths: the paged step is the contiguous step with another row map,
    so o, lse and the updated keys are bit-identical."""
    B, H, d, n, page = 2, 3, 64, 2100, 128
    x = synthetic.decode_inputs(B, H, d, n, n + 1, "bf16", 11)
    kp, vp, table = _paginate(x["k_cache"], x["v_cache"], [n] * B, page, 2, 12)
    g = {k: t.to(DEV) for k, t in x.items()}
    oc, lc = pa.path_decode_step(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["k_cache"], g["v_cache"], n)
    kd, vd = kp.to(DEV), vp.to(DEV)
    op, lp = pa.path_decode_step_paged(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], kd, vd, table.to(DEV),
                                       torch.full((B,), n, dtype=torch.int32, device=DEV), n)
    torch.cuda.synchronize()
    assert torch.equal(oc, op) and torch.equal(lc, lp)
    kg = kd.cpu()
    for b in range(B):
        assert torch.equal(_gather(kg, table, b, n + 1, page), g["k_cache"][b, :, : n + 1].cpu())


def test_paged_full_size():
    """Cache-8192 decode shapes (H=16, d=64, bf16) with lengths spread over 1..8192
    and 256-slot pages; every head of every sequence against the oracle."""
    B, H, d = 16, 16, 64
    lens = [int(v) for v in np.random.default_rng(3).integers(1, 8193, size=B)]
    _paged_case(B, H, d, lens, 256, "bf16", 1.0, seed=5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page", [16, 100])
def test_paged_fox_small(dtype, d, page):
    """Gated paged step: per sequence, the oracle's gated step on its logically
    contiguous cache and prefix cache; c_t lands at the new key's slot."""
    _paged_case(3, 2, d, [0, 150, 1333], page, dtype, 1.0, seed=page + d + 5, fox=True)


def test_paged_fox_page_boundaries():
    _paged_case(4, 2, 64, [63, 64, 65, 128], 64, "bf16", 0.5, seed=19, fox=True)


def test_paged_fox_matches_contiguous_fox_bitwise():
    """Equal lengths: the gated paged step is the gated contiguous step with
    another row map, so o, lse, the updated keys and c_t are bit-identical."""
    B, H, d, n, page = 2, 3, 64, 2100, 128
    x = synthetic.decode_inputs(B, H, d, n, n + 1, "bf16", 21, fox=True)
    cum = torch.cumsum(x["log_f_cache"].double(), dim=-1).float()
    kp, vp, table = _paginate(x["k_cache"], x["v_cache"], [n] * B, page, 2, 22)
    cp = _paginate_cum(cum, table, [n] * B, page, kp.shape[0], 23)
    g = {k: t.to(DEV) for k, t in x.items()}
    cc = cum.to(DEV)
    oc, lc = pa.path_decode_step_fox(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["log_f_t"],
                                     g["k_cache"], g["v_cache"], cc, n)
    kd, vd, cd = kp.to(DEV), vp.to(DEV), cp.to(DEV)
    op, lp = pa.path_decode_step_paged_fox(g["q_t"], g["k_t"], g["v_t"], g["w_t"], g["beta_t"], g["log_f_t"], kd,
                                           vd, cd, table.to(DEV), torch.full((B,), n, dtype=torch.int32, device=DEV),
                                           n)
    torch.cuda.synchronize()
    assert torch.equal(oc, op) and torch.equal(lc, lp)
    kg, cg = kd.cpu(), cd.cpu()
    for b in range(B):
        assert torch.equal(_gather(kg, table, b, n + 1, page), g["k_cache"][b, :, : n + 1].cpu())
        assert torch.equal(cg[int(table[b, n // page]), :, n % page], cc[b, :, n].cpu())


def test_paged_fox_full_size():
    """Cache-8192 decode shapes with forget gates, lengths spread over 1..8192,
    256-slot pages; every head of every sequence against the oracle."""
    B, H, d = 16, 16, 64
    lens = [int(v) for v in np.random.default_rng(4).integers(1, 8193, size=B)]
    _paged_case(B, H, d, lens, 256, "bf16", 1.0, seed=6, fox=True)
