"""Seeded synthetic inputs for PaTH attention workloads.

Shared by the tests, the smoke check and the benchmark; holds none of the
method's arithmetic (no transitions, no logits, no softmax).  Every head's
tensors come from their own seeded generator, so a subset of heads can be
regenerated alone, bit for bit, to feed the CPU oracle.

Distributions follow the workloads of the PaTH summary (gist.science
2505.16381): q, k, v standard normal; w Gaussian vectors normalised to unit
length; beta = 2 * sigmoid(z), z ~ N(0,1), so beta lies in (0,2) as §2
"Mecanismo Central" states; optional tokens with beta near 2 (z ~ N(6,0.5))
to exercise reflections with a negative eigenvalue; optional forget gates
f = sigmoid(N(3,1)) for PaTH-FoX (§2 "Extensões: PaTH-FoX").  They stand in
for the activations of the trained models the pages evaluate, which are not
available here.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _seed(*parts) -> int:
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(*parts) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(*parts))
    return g


@dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: str
    scale: float
    seed: int
    near2_frac: float = 0.0   # fraction of tokens (per batch row) with z ~ N(6, 0.5)
    fox: bool = False         # PaTH-FoX forget gates
    desc: str = ""


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    d: int
    cache_len: int
    capacity: int
    dtype: str
    scale: float
    seed: int
    desc: str = ""


# The five workloads.  Config 2's "q, k ~ N(0,1)/sqrt(d)" is read as the
# standard logit multiplier scale = 1/sqrt(64) = 0.125 on N(0,1) q and k.
CONFIGS = {
    1: FwdConfig("fp32_B1H1_L256_d64", 1, 1, 256, 64, "f32", 1.0, 1,
                 desc="PaTH forward fp32, B=1 H=1 L=256 d=64"),
    2: FwdConfig("bf16_B8H16_L4096_d64", 8, 16, 4096, 64, "bf16", 0.125, 2,
                 desc="PaTH forward bf16, B=8 H=16 L=4096 d=64, scale 1/sqrt(d)"),
    3: FwdConfig("bf16_B1H16_L16384_d64_near2", 1, 16, 16384, 64, "bf16", 1.0, 3, near2_frac=0.1,
                 desc="PaTH long-context forward bf16, B=1 H=16 L=16384 d=64, 10% tokens beta~2"),
    4: FwdConfig("bf16_B4H16_L8192_d128_fox", 4, 16, 8192, 128, "bf16", 1.0, 4, fox=True,
                 desc="PaTH-FoX forward bf16, B=4 H=16 L=8192 d=128"),
    5: DecodeConfig("bf16_B64H16_d64_cache8192", 64, 16, 64, 8192, 8193, "bf16", 1.0, 5,
                    desc="PaTH decode step bf16, B=64 H=16 d=64, cache 8192"),
}


def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def _unit(g: torch.Tensor) -> torch.Tensor:
    return g / torch.linalg.vector_norm(g, dim=-1, keepdim=True)


def fwd_inputs(B, H, L, d, dtype="bf16", seed=0, near2_frac=0.0, fox=False, heads=None):
    """Forward inputs on the CPU.

    Returns a dict with q, k, v, w ([N..., L, d] in `dtype`), beta and (if fox)
    log_forget ([..., L] fp32).  With heads=None the leading dims are [B, H];
    with a list of (b, h) pairs they are [len(heads)] and hold exactly those
    heads' values.
    """
    tdt = DTYPES[dtype]
    hl = _heads(B, H, heads)
    n_near = int(round(near2_frac * L))
    masks = {}
    out = {n: [] for n in ("q", "k", "v", "w", "beta", "log_forget")}
    for (b, h) in hl:
        for name in ("q", "k", "v"):
            out[name].append(torch.randn(L, d, generator=_gen(seed, name, b, h)))
        out["w"].append(_unit(torch.randn(L, d, generator=_gen(seed, "w", b, h))))
        z = torch.randn(L, generator=_gen(seed, "z", b, h))
        if n_near > 0:
            if b not in masks:
                masks[b] = torch.randperm(L, generator=_gen(seed, "mask", b))[:n_near]
            znear = 6.0 + 0.5 * torch.randn(n_near, generator=_gen(seed, "znear", b, h))
            z[masks[b]] = znear
        out["beta"].append(2.0 * torch.sigmoid(z))
        if fox:
            y = 3.0 + torch.randn(L, generator=_gen(seed, "forget", b, h))
            out["log_forget"].append(torch.nn.functional.logsigmoid(y))
    res = {}
    for name in ("q", "k", "v", "w"):
        t = torch.stack(out[name]).to(tdt)
        res[name] = t.view(B, H, L, d) if heads is None else t
    for name in ("beta", "log_forget"):
        if out[name]:
            t = torch.stack(out[name]).to(torch.float32)
            res[name] = t.view(B, H, L) if heads is None else t
    if not fox:
        res["log_forget"] = None
    return res


def decode_inputs(B, H, d, cache_len, capacity, dtype="bf16", seed=0, heads=None, fox=False):
    """Decode-step inputs on the CPU.

    q_t, k_t, v_t, w_t: [.., d] in `dtype`; beta_t: [..] fp32; k_cache, v_cache:
    [.., capacity, d] in `dtype` with slots >= cache_len zero.  With fox=True
    also the gates of the new token, log_f_t [..] fp32, and of the cached
    tokens, log_f_cache [.., capacity] fp32 (zero from slot cache_len on), drawn
    like the forward's forget gates; turning the latter into the prefix cache
    is left to the caller.
    """
    tdt = DTYPES[dtype]
    hl = _heads(B, H, heads)
    acc = {n: [] for n in ("q_t", "k_t", "v_t", "w_t", "beta_t", "k_cache", "v_cache")}
    for (b, h) in hl:
        for name in ("q_t", "k_t", "v_t"):
            acc[name].append(torch.randn(d, generator=_gen(seed, name, b, h)))
        acc["w_t"].append(_unit(torch.randn(d, generator=_gen(seed, "w_t", b, h))))
        acc["beta_t"].append(2.0 * torch.sigmoid(torch.randn(1, generator=_gen(seed, "z_t", b, h)))[0])
        for name in ("k_cache", "v_cache"):
            c = torch.zeros(capacity, d)
            c[:cache_len] = torch.randn(cache_len, d, generator=_gen(seed, name, b, h))
            acc[name].append(c)
    lead = (B, H) if heads is None else (len(hl),)
    res = {}
    for name in ("q_t", "k_t", "v_t", "w_t"):
        res[name] = torch.stack(acc[name]).to(tdt).view(*lead, d)
    res["beta_t"] = torch.stack(acc["beta_t"]).to(torch.float32).view(*lead)
    for name in ("k_cache", "v_cache"):
        res[name] = torch.stack(acc[name]).to(tdt).view(*lead, capacity, d)
    if fox:
        res.update(decode_gate_inputs(B, H, cache_len, capacity, seed, heads))
    return res


def decode_gate_inputs(B, H, cache_len, capacity, seed=0, heads=None):
    """The forget gates of a gated decode step alone (what decode_inputs adds
    with fox=True): log_f_t [..] and log_f_cache [.., capacity] fp32."""
    hl = _heads(B, H, heads)
    lft, lfc = [], []
    for (b, h) in hl:
        y = 3.0 + torch.randn(cache_len + 1, generator=_gen(seed, "forget", b, h))
        lf = torch.nn.functional.logsigmoid(y)
        c = torch.zeros(capacity)
        c[:cache_len] = lf[:cache_len]
        lfc.append(c)
        lft.append(lf[cache_len])
    lead = (B, H) if heads is None else (len(hl),)
    return {"log_f_t": torch.stack(lft).to(torch.float32).view(*lead),
            "log_f_cache": torch.stack(lfc).to(torch.float32).view(*lead, capacity)}


def config_inputs(cfg_id: int, heads=None, small=None):
    """Inputs of one of the five workloads (optionally a subset of heads)."""
    c = CONFIGS[cfg_id]
    if isinstance(c, DecodeConfig):
        return decode_inputs(c.B, c.H, c.d, c.cache_len, c.capacity, c.dtype, c.seed, heads)
    return fwd_inputs(c.B, c.H, c.L, c.d, c.dtype, c.seed, c.near2_frac, c.fox, heads)


def project_inputs(B: int, L: int, Dm: int, H: int, d: int, seed: int):
    """Inputs of the projection prologue: tokens x [B, L, Dm] ~ N(0,1) (bf16),
    per-head maps Ww [H, d, Dm] and gate vectors u [H, Dm] ~ N(0, 1/Dm) (bf16,
    so projections are O(1)), biases b [H] ~ N(0,1) (fp32).  Random weights
    stand in for trained ones."""
    x = torch.randn(B, L, Dm, generator=_gen("proj", seed, "x")).to(torch.bfloat16)
    Ww = (torch.randn(H, d, Dm, generator=_gen("proj", seed, "Ww")) / Dm ** 0.5).to(torch.bfloat16)
    u = (torch.randn(H, Dm, generator=_gen("proj", seed, "u")) / Dm ** 0.5).to(torch.bfloat16)
    bias = torch.randn(H, generator=_gen("proj", seed, "b"))
    return {"x": x, "Ww": Ww, "u": u, "b": bias}
