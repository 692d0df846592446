"""PaTH attention on MI355X (gfx950): thin Python binding of libpath_attn.so.

Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, allocates outputs and workspaces with torch, and passes
raw device pointers plus the current HIP stream through the C ABI declared in
include/path_attn.h.  There is no fallback: if the shared library is missing
the import of `lib()` raises.

Method: "PaTH Attention" (gist.science 2505.16381) - causal softmax attention
with logits k_j^T (H_{j+1}...H_i) q_i, H_s = I - beta_s w_s w_s^T (§2
"Mecanismo Central"), optional PaTH-FoX forget bias (§2 "Extensões"), UT block
transform and right-to-left block scan (§3), in-place key-cache decode (§3
"Inferência").
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpath_attn.so")

PATH_F32, PATH_BF16 = 0, 1
PRECISION = {"accurate": 0, "auto": 1}
STATUS = {0: "PATH_OK", 1: "PATH_ERR_NULL", 2: "PATH_ERR_SHAPE", 3: "PATH_ERR_UNSUPPORTED",
          4: "PATH_ERR_WORKSPACE", 5: "PATH_ERR_CAPACITY", 6: "PATH_ERR_HIP", 7: "PATH_ERR_SCRATCH"}
EXPORTS = ["path_status_string", "path_abi_version", "path_prepare", "path_fwd_workspace_bytes",
           "path_attn_fwd", "path_fwd_stage_prepare", "path_fwd_stage_scan",
           "path_decode_workspace_bytes", "path_decode_step", "path_decode_step_fox",
           "path_bwd_workspace_bytes", "path_attn_bwd", "path_project", "path_decode_step_paged",
           "path_decode_step_noalloc", "path_decode_noalloc_max_bytes", "path_decode_step_paged_fox"]

_lib = None
_I64, _INT, _F, _VP, _SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class PathError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load libpath_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m dependent_position_encoding_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.path_status_string.restype = ctypes.c_char_p
        L.path_status_string.argtypes = [_INT]
        L.path_abi_version.restype = _INT
        L.path_prepare.restype = _INT
        L.path_prepare.argtypes = [_I64, _I64, _I64, _I64, _INT] + [_VP] * 10 + [_VP]
        L.path_fwd_workspace_bytes.restype = _SZ
        L.path_fwd_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _INT, _INT]
        L.path_attn_fwd.restype = _INT
        L.path_attn_fwd.argtypes = [_I64, _I64, _I64, _I64, _INT, _F, _INT] + [_VP] * 8 + [_VP, _SZ, _VP]
        L.path_fwd_stage_prepare.restype = _INT
        L.path_fwd_stage_prepare.argtypes = [_I64, _I64, _I64, _I64, _INT, _F, _INT] + [_VP] * 6 + [_VP, _SZ, _VP]
        L.path_fwd_stage_scan.restype = _INT
        L.path_fwd_stage_scan.argtypes = [_I64, _I64, _I64, _I64, _INT, _F, _INT] + [_VP] * 8 + [_VP, _SZ, _VP]
        L.path_decode_workspace_bytes.restype = _SZ
        L.path_decode_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64]
        L.path_decode_step.restype = _INT
        L.path_decode_step.argtypes = ([_I64, _I64, _I64, _INT, _F] + [_VP] * 7 + [_I64, _I64] +
                                       [_VP, _VP, _VP, _SZ, _VP])
        L.path_bwd_workspace_bytes.restype = _SZ
        L.path_bwd_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _INT, _INT]
        L.path_attn_bwd.restype = _INT
        L.path_attn_bwd.argtypes = [_I64, _I64, _I64, _I64, _INT, _F] + [_VP] * 15 + [_VP, _SZ, _VP]
        L.path_decode_step_paged.restype = _INT
        L.path_decode_step_paged.argtypes = ([_I64, _I64, _I64, _INT, _F] + [_VP] * 7 + [_I64, _I64, _VP, _I64, _VP,
                                             _I64, _VP, _VP, _VP, _SZ, _VP])
        L.path_decode_step_paged_fox.restype = _INT
        L.path_decode_step_paged_fox.argtypes = ([_I64, _I64, _I64, _INT, _F] + [_VP] * 9 + [_I64, _I64, _VP, _I64,
                                                 _VP, _I64, _VP, _VP, _VP, _SZ, _VP])
        L.path_project.restype = _INT
        L.path_project.argtypes = [_I64] * 5 + [_VP] * 4 + [_F] + [_VP, _VP, _VP]
        L.path_decode_step_noalloc.restype = _INT
        L.path_decode_step_noalloc.argtypes = ([_I64, _I64, _I64, _INT, _F] + [_VP] * 7 + [_I64, _I64] +
                                               [_VP, _VP, _VP])
        L.path_decode_noalloc_max_bytes.restype = _SZ
        L.path_decode_noalloc_max_bytes.argtypes = []
        L.path_decode_step_fox.restype = _INT
        L.path_decode_step_fox.argtypes = ([_I64, _I64, _I64, _INT, _F] + [_VP] * 9 + [_I64, _I64] +
                                           [_VP, _VP, _VP, _SZ, _VP])
        _lib = L
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().path_status_string(int(status)).decode()
    except Exception:  # pragma: no cover
        return "?"


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PATH_F32
    if t.dtype == torch.bfloat16:
        return PATH_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (use float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _outputs(q, out):
    """(o, lse) for a forward on q: new tensors, or the caller's `out` after the
    checks the C side cannot make (it only sees raw pointers)."""
    B, H, L, d = q.shape
    if out is None:
        return torch.empty_like(q), torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    o, lse = out
    _check(o, "o", q.dtype, (B, H, L, d))
    _check(lse, "lse", torch.float32, (B, H, L))
    if o.device != q.device or lse.device != q.device:
        raise ValueError("o and lse must be on q's device")
    return o, lse


def _check_workspace(ws, q, nbytes=None):
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("workspace must be a 1-D torch.uint8 tensor")
    if ws.device != q.device:
        raise ValueError("workspace must be on the inputs' device")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if nbytes is not None and ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {nbytes} needed")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _raise(st: int, what: str):
    if st != 0:
        raise PathError(st, what)


def fwd_workspace_bytes(B, H, L, d, dtype_code, with_forget) -> int:
    return int(lib().path_fwd_workspace_bytes(B, H, L, d, dtype_code, int(bool(with_forget))))


def _fwd_args(q, k, v, w, beta, log_forget):
    B, H, L, d = q.shape
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("w", w)):
        _check(t, name, dt, (B, H, L, d))
    _check(beta, "beta", torch.float32, (B, H, L))
    if log_forget is not None:
        _check(log_forget, "log_forget", torch.float32, (B, H, L))
    return B, H, L, d, _dtype_code(q)


def fwd_workspace(q, log_forget=None) -> torch.Tensor:
    """A workspace tensor large enough for path_attn_fwd on inputs shaped like q."""
    B, H, L, d = q.shape
    nbytes = fwd_workspace_bytes(B, H, L, d, _dtype_code(q), log_forget is not None)
    if nbytes == 0:
        _raise(2, "path_fwd_workspace_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device)


def path_attn_fwd(q, k, v, w, beta, log_forget=None, scale=1.0, precision="auto", workspace=None,
                  out=None):
    """PaTH forward.  q,k,v,w [B,H,L,d] (fp32 or bf16, same dtype); beta, log_forget [B,H,L] fp32.

    Returns (o [B,H,L,d] in the input dtype, lse [B,H,L] fp32)."""
    B, H, L, d, code = _fwd_args(q, k, v, w, beta, log_forget)
    o, lse = _outputs(q, out)
    if workspace is None:
        workspace = fwd_workspace(q, log_forget)
    _check_workspace(workspace, q)
    st = lib().path_attn_fwd(B, H, L, d, code, float(scale), PRECISION[precision], _ptr(q), _ptr(k), _ptr(v),
                             _ptr(w), _ptr(beta), _ptr(log_forget), _ptr(o), _ptr(lse), _ptr(workspace),
                             int(workspace.numel()), _stream(q))
    _raise(st, "path_attn_fwd")
    return o, lse


def bwd_workspace_bytes(B, H, L, d, dtype_code, with_forget) -> int:
    return int(lib().path_bwd_workspace_bytes(B, H, L, d, dtype_code, int(bool(with_forget))))


def path_attn_bwd(q, k, v, w, beta, o, lse, do, log_forget=None, scale=1.0, workspace=None):
    """PaTH backward: gradients of sum(do * o) for the forward path_attn_fwd(q, k, v, w,
    beta, log_forget, scale) that returned (o, lse).

    Returns (dq, dk, dv, dw in the input dtype, dbeta fp32, dlog_forget fp32 or None)."""
    B, H, L, d, code = _fwd_args(q, k, v, w, beta, log_forget)
    _check(o, "o", q.dtype, (B, H, L, d))
    _check(do, "do", q.dtype, (B, H, L, d))
    _check(lse, "lse", torch.float32, (B, H, L))
    dq, dk, dv, dw = (torch.empty_like(q) for _ in range(4))
    dbeta = torch.empty_like(beta)
    dlf = torch.empty_like(log_forget) if log_forget is not None else None
    nbytes = bwd_workspace_bytes(B, H, L, d, code, log_forget is not None)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    st = lib().path_attn_bwd(B, H, L, d, code, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
                             _ptr(log_forget), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw),
                             _ptr(dbeta), _ptr(dlf), _ptr(workspace), int(workspace.numel()), _stream(q))
    _raise(st, "path_attn_bwd")
    return dq, dk, dv, dw, dbeta, dlf


def path_fwd_stage_prepare(q, k, v, w, beta, log_forget=None, scale=1.0, precision="auto", workspace=None):
    """First stage of path_attn_fwd: block UT data into `workspace` (returned)."""
    B, H, L, d, code = _fwd_args(q, k, v, w, beta, log_forget)
    if workspace is None:
        workspace = fwd_workspace(q, log_forget)
    _check_workspace(workspace, q)
    st = lib().path_fwd_stage_prepare(B, H, L, d, code, float(scale), PRECISION[precision], _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(w), _ptr(beta), _ptr(log_forget), _ptr(workspace),
                                      int(workspace.numel()), _stream(q))
    _raise(st, "path_fwd_stage_prepare")
    return workspace


def path_fwd_stage_scan(q, k, v, w, beta, workspace, log_forget=None, scale=1.0, precision="auto", out=None):
    """Second stage of path_attn_fwd: the right-to-left scan from a prepared workspace."""
    B, H, L, d, code = _fwd_args(q, k, v, w, beta, log_forget)
    o, lse = _outputs(q, out)
    _check_workspace(workspace, q)
    st = lib().path_fwd_stage_scan(B, H, L, d, code, float(scale), PRECISION[precision], _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(w), _ptr(beta), _ptr(log_forget), _ptr(o), _ptr(lse),
                                   _ptr(workspace), int(workspace.numel()), _stream(q))
    _raise(st, "path_fwd_stage_scan")
    return o, lse


def path_prepare(q, k, w, beta, log_forget=None):
    """Per-block UT transform.  Returns dict of fp32 tensors tinv [B,H,Nb,64,64],
    qhat/khat [B,H,L,d], pT [B,H,Nb,d,d] and (with log_forget) cum [B,H,L]."""
    B, H, L, d = q.shape
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("w", w)):
        _check(t, name, dt, (B, H, L, d))
    _check(beta, "beta", torch.float32, (B, H, L))
    Nb = (L + 63) // 64
    f32 = dict(dtype=torch.float32, device=q.device)
    out = {"tinv": torch.empty((B, H, Nb, 64, 64), **f32), "qhat": torch.empty((B, H, L, d), **f32),
           "khat": torch.empty((B, H, L, d), **f32), "pT": torch.empty((B, H, Nb, d, d), **f32)}
    if log_forget is not None:
        _check(log_forget, "log_forget", torch.float32, (B, H, L))
        out["cum"] = torch.empty((B, H, L), **f32)
    st = lib().path_prepare(B, H, L, d, _dtype_code(q), _ptr(q), _ptr(k), _ptr(w), _ptr(beta), _ptr(log_forget),
                            _ptr(out["tinv"]), _ptr(out["qhat"]), _ptr(out["khat"]), _ptr(out["pT"]),
                            _ptr(out.get("cum")), _stream(q))
    _raise(st, "path_prepare")
    return out


def decode_workspace_bytes(B, H, d, cache_len) -> int:
    return int(lib().path_decode_workspace_bytes(B, H, d, cache_len))


def path_decode_step(q_t, k_t, v_t, w_t, beta_t, k_cache, v_cache, cache_len, scale=1.0, workspace=None):
    """One decode step.  q_t,k_t,v_t,w_t [B,H,d]; beta_t [B,H] fp32; caches [B,H,capacity,d].

    Updates k_cache[:, :, :cache_len] in place, writes k_t, v_t at slot cache_len,
    returns (o [B,H,d], lse [B,H] fp32)."""
    return _decode(q_t, k_t, v_t, w_t, beta_t, None, k_cache, v_cache, None, cache_len, scale, workspace)


def path_decode_step_noalloc(q_t, k_t, v_t, w_t, beta_t, k_cache, v_cache, cache_len, scale=1.0):
    """path_decode_step without a workspace: the library's static device scratch
    (path_decode_noalloc_max_bytes() per GPU) holds the step's partials.  Calls
    that overlap in time on one GPU race.  Returns (o [B,H,d], lse [B,H] fp32)."""
    B, H, d = q_t.shape
    cap = k_cache.shape[2]
    dt = q_t.dtype
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _check(t, name, dt, (B, H, d))
    _check(beta_t, "beta_t", torch.float32, (B, H))
    _check(k_cache, "k_cache", dt, (B, H, cap, d))
    _check(v_cache, "v_cache", dt, (B, H, cap, d))
    o = torch.empty_like(q_t)
    lse = torch.empty((B, H), dtype=torch.float32, device=q_t.device)
    st = lib().path_decode_step_noalloc(B, H, d, _dtype_code(q_t), float(scale), _ptr(q_t), _ptr(k_t), _ptr(v_t),
                                        _ptr(w_t), _ptr(beta_t), _ptr(k_cache), _ptr(v_cache), int(cache_len),
                                        int(cap), _ptr(o), _ptr(lse), _stream(q_t))
    _raise(st, "path_decode_step_noalloc")
    return o, lse


def decode_noalloc_max_bytes() -> int:
    return int(lib().path_decode_noalloc_max_bytes())


def path_decode_step_fox(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache, v_cache, cum_cache, cache_len,
                         scale=1.0, workspace=None):
    """One PaTH-FoX decode step: path_decode_step plus log_f_t [B,H] fp32 and the
    gate-prefix cache cum_cache [B,H,capacity] fp32 (slots < cache_len hold c_j;
    the step writes c_t at slot cache_len)."""
    return _decode(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache, v_cache, cum_cache, cache_len, scale, workspace)


def _decode(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache, v_cache, cum_cache, cache_len, scale, workspace):
    B, H, d = q_t.shape
    cap = k_cache.shape[2]
    dt = q_t.dtype
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _check(t, name, dt, (B, H, d))
    _check(beta_t, "beta_t", torch.float32, (B, H))
    _check(k_cache, "k_cache", dt, (B, H, cap, d))
    _check(v_cache, "v_cache", dt, (B, H, cap, d))
    fox = log_f_t is not None
    if fox:
        _check(log_f_t, "log_f_t", torch.float32, (B, H))
        _check(cum_cache, "cum_cache", torch.float32, (B, H, cap))
    o = torch.empty_like(q_t)
    lse = torch.empty((B, H), dtype=torch.float32, device=q_t.device)
    nbytes = decode_workspace_bytes(B, H, d, cache_len)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q_t.device)
    _check_workspace(workspace, q_t)
    head = (B, H, d, _dtype_code(q_t), float(scale), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(w_t), _ptr(beta_t))
    tail = (int(cache_len), int(cap), _ptr(o), _ptr(lse), _ptr(workspace), int(workspace.numel()), _stream(q_t))
    if fox:
        st = lib().path_decode_step_fox(*head, _ptr(log_f_t), _ptr(k_cache), _ptr(v_cache), _ptr(cum_cache), *tail)
        _raise(st, "path_decode_step_fox")
    else:
        st = lib().path_decode_step(*head, _ptr(k_cache), _ptr(v_cache), *tail)
        _raise(st, "path_decode_step")
    return o, lse


def path_project(x, Ww, u, bias, beta_max=None, out=None):
    """Projection prologue: x [B,L,Dm], Ww [H,d,Dm], u [H,Dm] (bf16), bias [H] fp32.

    Returns (w [B,H,L,d] bf16, unit length per (b,h,l); beta [B,H,L] fp32 =
    2 sigmoid(u_h . x + bias_h), capped at beta_max when given)."""
    B, L, Dm = x.shape
    H, d, _ = Ww.shape
    _check(x, "x", torch.bfloat16, (B, L, Dm))
    _check(Ww, "Ww", torch.bfloat16, (H, d, Dm))
    _check(u, "u", torch.bfloat16, (H, Dm))
    _check(bias, "bias", torch.float32, (H,))
    w, beta = out if out is not None else (torch.empty((B, H, L, d), dtype=torch.bfloat16, device=x.device),
                                           torch.empty((B, H, L), dtype=torch.float32, device=x.device))
    _check(w, "w", torch.bfloat16, (B, H, L, d))
    _check(beta, "beta", torch.float32, (B, H, L))
    bm = 0.0 if beta_max is None else float(beta_max)
    st = lib().path_project(B, L, Dm, H, d, _ptr(x), _ptr(Ww), _ptr(u), _ptr(bias), bm, _ptr(w), _ptr(beta),
                            _stream(x))
    _raise(st, "path_project")
    return w, beta


def path_decode_step_paged(q_t, k_t, v_t, w_t, beta_t, k_pages, v_pages, page_table, cache_lens, max_cache_len,
                           scale=1.0, workspace=None):
    """Decode step over a paged cache.  q_t, k_t, v_t, w_t [B,H,d]; beta_t [B,H] fp32;
    k_pages, v_pages [num_pages,H,page_size,d] (updated in place, new token appended);
    page_table [B,max_pages] int32 and cache_lens [B] int32 on the device; max_cache_len
    (host int) bounds every cache_lens[b].  Returns (o [B,H,d], lse [B,H] fp32)."""
    return _paged(q_t, k_t, v_t, w_t, beta_t, None, k_pages, v_pages, None, page_table, cache_lens, max_cache_len,
                  scale, workspace)


def path_decode_step_paged_fox(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_pages, v_pages, cum_pages, page_table,
                               cache_lens, max_cache_len, scale=1.0, workspace=None):
    """Gated (PaTH-FoX) decode step over a paged cache: path_decode_step_paged plus
    log_f_t [B,H] fp32 and the gate-prefix pages cum_pages [num_pages,H,page_size]
    fp32 (c_j at key j's slot; the step writes c_t at the new key's slot)."""
    return _paged(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_pages, v_pages, cum_pages, page_table, cache_lens,
                  max_cache_len, scale, workspace)


def _paged(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_pages, v_pages, cum_pages, page_table, cache_lens, max_cache_len,
           scale, workspace):
    B, H, d = q_t.shape
    num_pages, _, page_size, _ = k_pages.shape
    max_pages = page_table.shape[1]
    dt = q_t.dtype
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _check(t, name, dt, (B, H, d))
    _check(beta_t, "beta_t", torch.float32, (B, H))
    _check(k_pages, "k_pages", dt, (num_pages, H, page_size, d))
    _check(v_pages, "v_pages", dt, (num_pages, H, page_size, d))
    _check(page_table, "page_table", torch.int32, (B, max_pages))
    _check(cache_lens, "cache_lens", torch.int32, (B,))
    fox = log_f_t is not None
    if fox:
        _check(log_f_t, "log_f_t", torch.float32, (B, H))
        _check(cum_pages, "cum_pages", torch.float32, (num_pages, H, page_size))
    o = torch.empty_like(q_t)
    lse = torch.empty((B, H), dtype=torch.float32, device=q_t.device)
    nbytes = decode_workspace_bytes(B, H, d, max_cache_len)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q_t.device)
    _check_workspace(workspace, q_t)
    head = (B, H, d, _dtype_code(q_t), float(scale), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(w_t), _ptr(beta_t))
    tail = (int(num_pages), int(page_size), _ptr(page_table), int(max_pages), _ptr(cache_lens), int(max_cache_len),
            _ptr(o), _ptr(lse), _ptr(workspace), int(workspace.numel()), _stream(q_t))
    if fox:
        st = lib().path_decode_step_paged_fox(*head, _ptr(log_f_t), _ptr(k_pages), _ptr(v_pages), _ptr(cum_pages),
                                              *tail)
        _raise(st, "path_decode_step_paged_fox")
    else:
        st = lib().path_decode_step_paged(*head, _ptr(k_pages), _ptr(v_pages), *tail)
        _raise(st, "path_decode_step_paged")
    return o, lse
