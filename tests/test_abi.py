"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU (every call
here fails validation, so nothing is ever enqueued)."""
import ctypes
import os
import re

import pytest

import dependent_position_encoding_fwd_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "path_attn.h")

OK, NULL, SHAPE, UNSUP, WS, CAP = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(path_[a-z_0-9]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    L = pa.lib()
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(pa.EXPORTS) == names


def test_status_strings_and_version():
    L = pa.lib()
    assert L.path_abi_version() == 1
    for st in range(8):
        assert len(L.path_status_string(st)) > 0
    assert L.path_status_string(99) == b"unknown status"


def _fwd(B=1, H=1, Lq=128, d=64, dtype=1, prec=1, ptr=FAKE, ws=FAKE, wsb=1 << 40, lf=None, o=FAKE):
    return pa.lib().path_attn_fwd(B, H, Lq, d, dtype, 1.0, prec, ptr, ptr, ptr, ptr, ptr, lf, o, ptr, ws, wsb, None)


def test_fwd_validation():
    assert _fwd(d=96) == UNSUP
    assert _fwd(d=32) == UNSUP
    assert _fwd(dtype=7) == UNSUP
    assert _fwd(prec=5) == UNSUP
    assert _fwd(B=0) == SHAPE
    assert _fwd(Lq=0) == SHAPE
    assert _fwd(H=-3) == SHAPE
    assert _fwd(B=1 << 40, H=1 << 20) == SHAPE   # element count overflow
    assert _fwd(ptr=None) == NULL
    assert _fwd(o=None) == NULL
    assert _fwd(ws=None) == WS
    assert _fwd(wsb=16) == WS
    assert _fwd(ws=ctypes.c_void_p(0x1010)) == WS  # not 256-byte aligned
    odd = ctypes.c_void_p(0x1008)  # 8-byte but not 16-byte aligned
    assert _fwd(ptr=odd) == UNSUP                  # bf16 rows move in 16-byte pieces
    assert _fwd(o=odd) == UNSUP
    assert _fwd(dtype=0, ptr=odd, ws=None) == WS   # fp32 has no such rule: next check fails


def _bwd(B=1, H=1, Lq=128, d=64, dtype=1, ptr=FAKE, lf=None, dlf=None, ws=FAKE, wsb=1 << 40, dq=FAKE,
         dout=FAKE):
    return pa.lib().path_attn_bwd(B, H, Lq, d, dtype, 1.0, ptr, ptr, ptr, ptr, ptr, lf, ptr, ptr, dout, dq, ptr,
                                  ptr, ptr, ptr, dlf, ws, wsb, None)


def test_bwd_validation():
    assert _bwd(d=96) == UNSUP
    assert _bwd(dtype=7) == UNSUP
    assert _bwd(Lq=0) == SHAPE
    assert _bwd(ptr=None) == NULL
    assert _bwd(lf=FAKE) == NULL                   # gates given without their gradient
    assert _bwd(ws=None) == WS
    assert _bwd(ws=ctypes.c_void_p(0x1010)) == WS  # not 256-byte aligned
    odd = ctypes.c_void_p(0x1008)
    assert _bwd(dq=odd) == UNSUP                   # bf16 tensors start on 16 bytes
    assert _bwd(dout=odd) == UNSUP
    assert _bwd(dtype=0, dq=odd, ws=None) == WS    # fp32 has no such rule


def test_workspace_sizes():
    L = pa.lib()
    assert L.path_fwd_workspace_bytes(1, 1, 64, 96, 1, 0) == 0
    a = L.path_fwd_workspace_bytes(2, 3, 200, 64, 1, 0)
    b = L.path_fwd_workspace_bytes(2, 3, 200, 64, 1, 1)
    assert a > 0 and b > a and a % 256 == 0 and b % 256 == 0
    assert L.path_decode_workspace_bytes(1, 1, 64, 0) >= 256
    assert L.path_decode_workspace_bytes(1, 1, 48, 10) == 0


def test_prepare_validation():
    L = pa.lib()
    assert L.path_prepare(1, 1, 64, 64, 1, FAKE, FAKE, None, FAKE, None, FAKE, None, None, None, None, None) == NULL
    assert L.path_prepare(1, 1, 64, 64, 1, None, FAKE, FAKE, FAKE, None, None, FAKE, None, None, None, None) == NULL
    assert L.path_prepare(1, 1, 64, 64, 1, FAKE, FAKE, FAKE, FAKE, None, None, None, None, None, FAKE, None) == NULL
    assert L.path_prepare(1, 1, 64, 80, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None, None, None) == UNSUP
    # nothing requested: valid no-op, no launch
    assert L.path_prepare(1, 1, 64, 64, 1, FAKE, FAKE, FAKE, FAKE, None, None, None, None, None, None, None) == OK


def _dec(cache_len=10, capacity=11, d=64, dtype=1, ptr=FAKE, ws=FAKE, wsb=1 << 30):
    return pa.lib().path_decode_step(2, 2, d, dtype, 1.0, ptr, ptr, ptr, ptr, ptr, ptr, ptr, cache_len, capacity,
                                     ptr, ptr, ws, wsb, None)


def test_decode_validation():
    assert _dec(cache_len=11, capacity=11) == CAP
    assert _dec(cache_len=20, capacity=11) == CAP
    assert _dec(cache_len=-1) == SHAPE
    assert _dec(capacity=0, cache_len=0) == SHAPE
    assert _dec(d=100) == UNSUP
    assert _dec(dtype=3) == UNSUP
    assert _dec(ptr=None) == NULL
    assert _dec(ws=None) == WS
    assert _dec(wsb=8) == WS


def _dec_fox(cache_len=10, capacity=11, lf=FAKE, cum=FAKE, ptr=FAKE, ws=FAKE, wsb=1 << 30):
    return pa.lib().path_decode_step_fox(2, 2, 64, 1, 1.0, ptr, ptr, ptr, ptr, ptr, lf, ptr, ptr, cum, cache_len,
                                         capacity, ptr, ptr, ws, wsb, None)


def test_decode_fox_validation():
    assert _dec_fox(lf=None) == NULL
    assert _dec_fox(cum=None) == NULL
    assert _dec_fox(ptr=None) == NULL
    assert _dec_fox(cache_len=11, capacity=11) == CAP
    assert _dec_fox(cache_len=-1) == SHAPE
    assert _dec_fox(ws=None) == WS


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    b = torch.zeros(1, 1, 64)
    with pytest.raises(ValueError):
        pa.path_attn_fwd(x, x, x, x, b)


def _proj(B=1, L=128, Dm=256, H=2, d=64, ptr=FAKE, x=None, bias=FAKE, w=None):
    xp = ptr if x is None else x
    wp = ptr if w is None else w
    return pa.lib().path_project(B, L, Dm, H, d, xp, ptr, ptr, bias, 0.0, wp, ptr, None)


def test_project_validation():
    assert _proj(d=96) == UNSUP
    assert _proj(Dm=96) == SHAPE          # not a multiple of 64
    assert _proj(Dm=0) == SHAPE
    assert _proj(B=0) == SHAPE
    assert _proj(H=0) == SHAPE
    assert _proj(B=1 << 40, L=1 << 20) == SHAPE
    assert _proj(ptr=None) == NULL
    assert _proj(bias=None) == NULL
    assert _proj(x=ctypes.c_void_p(0x1008)) == UNSUP   # not 16-byte aligned
    assert _proj(w=ctypes.c_void_p(0x1008)) == UNSUP   # w is written in 16-byte segments


def _paged(B=2, H=2, d=64, dtype=1, npages=8, page=16, mp=4, maxlen=20, ptr=FAKE, ws=FAKE, wsb=1 << 30,
           table=FAKE):
    return pa.lib().path_decode_step_paged(B, H, d, dtype, 1.0, ptr, ptr, ptr, ptr, ptr, ptr, ptr, npages, page,
                                           table, mp, ptr, maxlen, ptr, ptr, ws, wsb, None)


def test_decode_paged_validation():
    assert _paged(d=80) == UNSUP
    assert _paged(dtype=4) == UNSUP
    assert _paged(page=0) == SHAPE
    assert _paged(npages=0) == SHAPE
    assert _paged(mp=0) == SHAPE
    assert _paged(maxlen=-1) == SHAPE
    assert _paged(maxlen=64) == CAP         # 4 pages of 16 slots hold keys 0..63, the new key needs slot maxlen
    assert _paged(ptr=None) == NULL
    assert _paged(table=None) == NULL
    assert _paged(ws=None) == WS
    assert _paged(wsb=8) == WS


def _noalloc(B=2, H=2, d=64, dtype=1, cache_len=10, capacity=11, ptr=FAKE):
    return pa.lib().path_decode_step_noalloc(B, H, d, dtype, 1.0, ptr, ptr, ptr, ptr, ptr, ptr, ptr, cache_len,
                                             capacity, ptr, ptr, None)


def test_decode_noalloc_validation():
    """Every failing check returns before the static scratch is looked up."""
    SCRATCH = 7
    assert pa.lib().path_decode_noalloc_max_bytes() == 8 << 20
    assert _noalloc(d=100) == UNSUP
    assert _noalloc(dtype=3) == UNSUP
    assert _noalloc(cache_len=-1) == SHAPE
    assert _noalloc(cache_len=11, capacity=11) == CAP
    assert _noalloc(ptr=None) == NULL
    # 64 x 16 heads x 64 chunks x 66 floats = 17.3 MB of partials > 8 MiB
    assert _noalloc(B=64, H=16, cache_len=65536, capacity=65537) == SCRATCH
    # the cache-8192 workload step fits: 1024 heads x 8 chunks x 66 floats + 512 B = 2.2 MB
    assert pa.lib().path_decode_workspace_bytes(64, 16, 64, 8192) <= 8 << 20


def _paged_fox(lf=FAKE, cum=FAKE, d=64, maxlen=20, ptr=FAKE, ws=FAKE):
    # B=2 H=2 bf16, 8 pages of 16 slots, 4 logical pages per sequence
    return pa.lib().path_decode_step_paged_fox(2, 2, d, 1, 1.0, ptr, ptr, ptr, ptr, ptr, lf, ptr, ptr, cum,
                                               8, 16, FAKE, 4, ptr, maxlen, ptr, ptr, ws, 1 << 30, None)


def test_decode_paged_fox_validation():
    assert _paged_fox(lf=None) == NULL
    assert _paged_fox(cum=None) == NULL
    assert _paged_fox(ptr=None) == NULL
    assert _paged_fox(d=80) == UNSUP
    assert _paged_fox(maxlen=64) == CAP
    assert _paged_fox(ws=None) == WS
