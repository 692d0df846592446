"""fp64 CPU oracle for PaTH attention.  TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The HIP library never does, and this
package never imports the library: the two share no code.

The arithmetic lives in `path_oracle.c` (plain C, fp64, OpenMP over query
rows; it also holds the hand-written reverse mode of the defining loop for
the gradients), for tiny explicit-matrix cross-checks in `tiny.py`, and for
gradients in `grad.py` as well (float64 torch.autograd of the defining loop,
the small-size reference the C reverse mode is pinned against).  This module
only compiles the C file with the host compiler and marshals numpy arrays.

Source pages: "PaTH Attention" technical summary (gist.science 2505.16381),
§2 "Mecanismo Central", §2 "Extensões: PaTH-FoX", §3 "Representação de
Transformação UT", §3 "Algoritmo Estilo FlashAttention", §3 "Inferência".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "path_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


# ORACLE_SANITIZE=1 selects a build of the same source under AddressSanitizer
# and UndefinedBehaviorSanitizer (the process must then be started with the
# sanitizer runtimes preloaded; tests/test_oracle_sanitized.py does that).
_SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
if _SANITIZE:
    _LIB_PATH = os.path.join(_OUT_DIR, "liboracle_asan_ubsan.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = False) -> str:
    """Compile path_oracle.c into oracle/_build/liboracle.so (gcc -O2 -fopenmp)."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *(_SAN_FLAGS if _SANITIZE else []), _SRC,
               "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_path_fwd.argtypes = [_I64, _I64, _D, _D, _D, _D, _D, _D, ctypes.c_double,
                                            _I64, ctypes.POINTER(_I64), _D, _D, _D]
            lib.oracle_path_decode.argtypes = [_I64, _I64, _D, _D, _D, _D, ctypes.c_double, _D, _D,
                                               ctypes.c_double, _D, _D]
            lib.oracle_path_decode_fox.argtypes = [_I64, _I64, _D, _D, _D, _D, ctypes.c_double,
                                                   ctypes.c_double, _D, _D, _D, ctypes.c_double, _D, _D, _D]
            lib.oracle_ut_tinv.argtypes = [_I64, _I64, _D, _D, _D]
            lib.oracle_block_adjust.argtypes = [_I64, _I64, _D, _D, _D, _D, _D, _D, _D]
            lib.oracle_prefix_sum.argtypes = [_I64, _D, _D]
            lib.oracle_path_bwd.argtypes = [_I64, _I64, _D, _D, _D, _D, _D, _D, ctypes.c_double, _D,
                                            _D, _D, _D, _D, _D, _D]
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact upcast of the stored values (bf16/fp32 tensors or arrays) to fp64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def path_fwd_head(q, k, v, w, beta, log_forget=None, scale=1.0, rows=None, want_logits=False):
    """One head: q,k,v,w [L,d]; beta, log_forget [L].  Returns (o, lse[, logits])."""
    lib = _load()
    q, k, v, w, beta = (_f64(x) for x in (q, k, v, w, beta))
    L, d = q.shape
    lf = _f64(log_forget) if log_forget is not None else None
    if rows is None:
        n = L
        rows_p = ctypes.POINTER(_I64)()
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.shape[0]
        rows_p = rows_arr.ctypes.data_as(ctypes.POINTER(_I64))
    o = np.zeros((n, d))
    lse = np.zeros((n,))
    lg = np.zeros((n, L)) if want_logits else None
    lib.oracle_path_fwd(L, d, _p(q), _p(k), _p(v), _p(w), _p(beta), _p(lf) if lf is not None else _D(),
                        float(scale), n, rows_p, _p(o), _p(lse), _p(lg) if lg is not None else _D())
    return (o, lse, lg) if want_logits else (o, lse)


def path_fwd(q, k, v, w, beta, log_forget=None, scale=1.0):
    """Batched [B,H,L,d] forward; returns fp64 (o [B,H,L,d], lse [B,H,L])."""
    q, k, v, w, beta = (_f64(x) for x in (q, k, v, w, beta))
    lf = _f64(log_forget) if log_forget is not None else None
    B, H, L, d = q.shape
    o = np.zeros((B, H, L, d))
    lse = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = path_fwd_head(q[b, h], k[b, h], v[b, h], w[b, h], beta[b, h],
                                               None if lf is None else lf[b, h], scale)
    return o, lse


def path_bwd_head(q, k, v, w, beta, log_forget, scale, do):
    """Gradients of <do, o> for one head by the C reverse mode of the defining
    loop: dict dq, dk, dv, dw [L,d], dbeta [L], dlog_forget [L] (None without
    gates), float64 numpy (the same layout as oracle.grad.path_bwd_head)."""
    lib = _load()
    q, k, v, w, beta, do = (_f64(x) for x in (q, k, v, w, beta, do))
    L, d = q.shape
    lf = _f64(log_forget) if log_forget is not None else None
    out = {n: np.zeros((L, d)) for n in ("dq", "dk", "dv", "dw")}
    out["dbeta"] = np.zeros((L,))
    dlf = np.zeros((L,)) if lf is not None else None
    lib.oracle_path_bwd(L, d, _p(q), _p(k), _p(v), _p(w), _p(beta), _p(lf) if lf is not None else _D(),
                        float(scale), _p(do), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dw"]),
                        _p(out["dbeta"]), _p(dlf) if dlf is not None else _D())
    out["dlog_forget"] = dlf
    return out


def path_logits(q, k, w, beta, log_forget=None, scale=1.0):
    """Full [L,L] logits of one head (entries j > i are -inf)."""
    q = _f64(q)
    v = np.zeros_like(q)
    _, _, lg = path_fwd_head(q, k, v, w, beta, log_forget, scale, rows=np.arange(q.shape[0]),
                             want_logits=True)
    return lg


def path_decode_head(q_t, k_t, v_t, w_t, beta_t, k_cache, v_cache, scale=1.0):
    """One decode step of one head.  Returns (o [d], lse, updated k_cache [len,d])."""
    lib = _load()
    q_t, k_t, v_t, w_t = (_f64(x) for x in (q_t, k_t, v_t, w_t))
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache)
    n, d = kc.shape
    o = np.zeros((d,))
    lse = np.zeros((1,))
    lib.oracle_path_decode(n, d, _p(q_t), _p(k_t), _p(v_t), _p(w_t), float(beta_t), _p(kc), _p(vc),
                           float(scale), _p(o), _p(lse))
    return o, float(lse[0]), kc


def path_decode_fox_head(q_t, k_t, v_t, w_t, beta_t, log_f_t, k_cache, v_cache, cum_cache, scale=1.0):
    """One PaTH-FoX decode step of one head; cum_cache [len] holds the gate
    prefixes of the cached keys.  Returns (o [d], lse, updated k_cache, c_t)."""
    lib = _load()
    q_t, k_t, v_t, w_t = (_f64(x) for x in (q_t, k_t, v_t, w_t))
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache)
    cc = _f64(cum_cache)
    n, d = kc.shape
    assert cc.shape == (n,)
    o = np.zeros((d,))
    lse = np.zeros((1,))
    ct = np.zeros((1,))
    lib.oracle_path_decode_fox(n, d, _p(q_t), _p(k_t), _p(v_t), _p(w_t), float(beta_t), float(log_f_t),
                               _p(kc), _p(vc), _p(cc), float(scale), _p(o), _p(lse), _p(ct))
    return o, float(lse[0]), kc, float(ct[0])


def ut_tinv(w, beta):
    """T^{-1} of one block (upper triangular n x n) by back substitution."""
    lib = _load()
    w, beta = _f64(w), _f64(beta)
    n, d = w.shape
    t = np.zeros((n, n))
    lib.oracle_ut_tinv(n, d, _p(w), _p(beta), _p(t))
    return t


def block_adjust(q, k, w, beta):
    """(qhat [n,d], khat [n,d], pT [d,d]) of one block, one H at a time."""
    lib = _load()
    q, k, w, beta = (_f64(x) for x in (q, k, w, beta))
    n, d = q.shape
    qh, kh, pt = np.zeros((n, d)), np.zeros((n, d)), np.zeros((d, d))
    lib.oracle_block_adjust(n, d, _p(q), _p(k), _p(w), _p(beta), _p(qh), _p(kh), _p(pt))
    return qh, kh, pt


def prefix_sum(x):
    lib = _load()
    x = _f64(x)
    c = np.zeros_like(x)
    lib.oracle_prefix_sum(x.shape[0], _p(x), _p(c))
    return c
