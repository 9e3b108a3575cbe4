"""Thin ctypes binding of liboscar (include/oscar.h): argument marshalling only.

Every computation runs in the C/HIP library; this module turns torch tensors
(device memory, streams) and NumPy arrays (host calibration data) into the
pointers and sizes the C ABI takes, and raises ``OscarError`` on a non-OK
status.  If the library has not been built, importing works but any call
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboscar.so")

OSCAR_OK = 0
STATUS_NAMES = {0: "OSCAR_OK", 1: "OSCAR_ERR_INVALID_ARG", 2: "OSCAR_ERR_UNSUPPORTED", 3: "OSCAR_ERR_NUMERIC",
                4: "OSCAR_ERR_WORKSPACE", 5: "OSCAR_ERR_HIP"}

# Every symbol include/oscar.h declares.
EXPORTS = [
    "oscar_status_string", "oscar_last_error", "oscar_version", "oscar_build_rotation",
    "oscar_build_fixed_rotation", "oscar_int2_page_bytes", "oscar_bf16_page_bytes", "oscar_quantize_append",
    "oscar_write_bf16", "oscar_decode_step_update", "oscar_decode_workspace_bytes", "oscar_calib_gram",
    "oscar_build_rotation_from_targets", "oscar_decode_workspace_init", "oscar_paged_decode_attn",
    "oscar_paged_decode_attn_bf16", "oscar_bw_probe_read", "oscar_paged_decode_attn_noalloc",
    "oscar_int4_page_bytes", "oscar_quantize_append_int4", "oscar_extend_workspace_bytes",
    "oscar_paged_extend_attn", "oscar_decode_int4_workspace_bytes", "oscar_paged_decode_attn_int4",
    "oscar_decode_step",
]


class OscarError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


class OscarCache(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_recent", ctypes.c_int32), ("int2_pool", ctypes.c_void_p), ("n_int2_pages", ctypes.c_int64),
                ("bf16_pool", ctypes.c_void_p), ("n_bf16_pages", ctypes.c_int64)]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_F64 = ctypes.c_double
_SZ = ctypes.c_size_t
_STATUS = ctypes.c_int


def load(path: str = LIB_PATH):
    """Load liboscar.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OscarError(5, f"{path} not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    sig = {
        "oscar_status_string": (ctypes.c_char_p, [_STATUS]),
        "oscar_last_error": (ctypes.c_char_p, []),
        "oscar_version": (_I32, []),
        "oscar_build_rotation": (_STATUS, [_I32, _I32, _I32, _I64, _P, _P, _P, _P, _F64, _I32, _I32,
                                           _P, _P, _P, _P, _P, _P]),
        "oscar_build_fixed_rotation": (_STATUS, [_I32, _I32, _I32, _I64, _P, _P, _F64, _I32, _P, _P, _P, _P]),
        "oscar_calib_gram": (_STATUS, [_P, _I64, _I32, _I32, _I32, _P, _P]),
        "oscar_build_rotation_from_targets": (_STATUS, [_I32, _I32, _P, _P, _I64, _P, _P, _F64, _I32, _I32,
                                                        _P, _P, _P, _P, _P, _P]),
        "oscar_int2_page_bytes": (_SZ, [_I32, _I32]),
        "oscar_bf16_page_bytes": (_SZ, [_I32, _I32]),
        "oscar_quantize_append": (_STATUS, [ctypes.POINTER(OscarCache), _P, _P, _I64, _P, _P, _P, _I32, _P, _P,
                                            _F32, _F32, _P]),
        "oscar_write_bf16": (_STATUS, [ctypes.POINTER(OscarCache), _P, _P, _I64, _P, _P, _P, _I32, _P]),
        "oscar_decode_step_update": (_STATUS, [ctypes.POINTER(OscarCache), _P, _P, _I32, _P, _P, _P, _I32, _P, _P,
                                               _F32, _F32, _P]),
        "oscar_decode_workspace_bytes": (_STATUS, [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
        "oscar_decode_workspace_init": (_STATUS, [_P, _SZ, _P]),
        "oscar_paged_decode_attn": (_STATUS, [ctypes.POINTER(OscarCache), _P, _I32, _I32, _P, _I32, _P, _P, _I32,
                                              _P, _P, _F32, _I32, _P, _SZ, _P, _P]),
        "oscar_paged_decode_attn_bf16": (_STATUS, [ctypes.POINTER(OscarCache), _P, _I32, _I32, _P, _I32, _P, _I32,
                                                   _F32, _I32, _P, _SZ, _P, _P]),
        "oscar_bw_probe_read": (_STATUS, [_P, _SZ, _P, _P]),
        "oscar_int4_page_bytes": (_SZ, [_I32, _I32]),
        "oscar_decode_step": (_STATUS, [ctypes.POINTER(OscarCache), _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _I32,
                                        _P, _P, _F32, _F32, _F32, _I32, _P, _SZ, _P, _P]),
        "oscar_quantize_append_int4": (_STATUS, [ctypes.POINTER(OscarCache), _P, _P, _I64, _P, _P, _P, _I32, _P, _P,
                                                 _F32, _F32, _P]),
        "oscar_extend_workspace_bytes": (_STATUS, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   ctypes.POINTER(_SZ)]),
        "oscar_paged_extend_attn": (_STATUS, [ctypes.POINTER(OscarCache), _I32, _P, _P, _P, _I32, _I32, _P, _P, _I32,
                                              _I32, _P, _P, _I32, _P, _P, _F32, _I32, _P, _SZ, _P, _P]),
        "oscar_decode_int4_workspace_bytes": (_STATUS, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                        ctypes.POINTER(_SZ)]),
        "oscar_paged_decode_attn_int4": (_STATUS, [ctypes.POINTER(OscarCache), _P, _I32, _I32, _P, _I32, _P, _P, _I32,
                                                   _P, _P, _F32, _I32, _P, _SZ, _P, _P]),
        "oscar_paged_decode_attn_noalloc": (_STATUS, [ctypes.POINTER(OscarCache), _P, _I32, _I32, _P, _I32, _P, _P,
                                                      _I32, _P, _P, _F32, _I32, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != OSCAR_OK:
        raise OscarError(status, load().oscar_last_error().decode())


def version() -> int:
    return load().oscar_version()


def int2_page_bytes(d: int, n_kv_heads: int) -> int:
    return load().oscar_int2_page_bytes(d, n_kv_heads)


def bf16_page_bytes(d: int, n_kv_heads: int) -> int:
    return load().oscar_bf16_page_bytes(d, n_kv_heads)


# ------------------------------------------------------------ host calls ---


def _host_f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def build_rotation(q_calib, k_calib, v_calib, group_q: int, clip_quantile: float = 0.999,
                   o_calib=None, max_sweeps: int = 0, n_threads: int = 0) -> dict:
    """Host calibration (oscar_build_rotation).  Arrays are [N, heads, d]."""
    q = _host_f32(q_calib); k = _host_f32(k_calib); v = _host_f32(v_calib)
    o = _host_f32(o_calib) if o_calib is not None else None
    n, hkv, d = k.shape
    rk = np.zeros((hkv, d, d)); rv = np.zeros((hkv, d, d))
    ek = np.zeros((hkv, d)); ev = np.zeros((hkv, d))
    tk = ctypes.c_double(); tv = ctypes.c_double()
    ptr = lambda a: a.ctypes.data_as(_P) if a is not None else None  # noqa: E731
    _check(load().oscar_build_rotation(d, hkv, group_q, n, ptr(q), ptr(k), ptr(v), ptr(o), clip_quantile,
                                       max_sweeps, n_threads, ptr(rk), ptr(rv), ctypes.byref(tk),
                                       ctypes.byref(tv), ptr(ek), ptr(ev)))
    return dict(r_k=rk, r_v=rv, tau_k=tk.value, tau_v=tv.value, eig_k=ek, eig_v=ev)


def build_rotation_from_targets(c_q, c_s, k_calib, v_calib, clip_quantile: float = 0.999, max_sweeps: int = 0,
                                n_threads: int = 0) -> dict:
    """Steps 2-4 of the calibration from given targets (oscar_build_rotation_from_targets).
    c_q, c_s float64 [H_kv, d, d]; k_calib, v_calib [N, H_kv, d]."""
    cq = np.ascontiguousarray(c_q, dtype=np.float64); cs = np.ascontiguousarray(c_s, dtype=np.float64)
    k = _host_f32(k_calib); v = _host_f32(v_calib)
    n, hkv, d = k.shape
    rk = np.zeros((hkv, d, d)); rv = np.zeros((hkv, d, d))
    ek = np.zeros((hkv, d)); ev = np.zeros((hkv, d))
    tk = ctypes.c_double(); tv = ctypes.c_double()
    ptr = lambda a: a.ctypes.data_as(_P)  # noqa: E731
    _check(load().oscar_build_rotation_from_targets(d, hkv, ptr(cq), ptr(cs), n, ptr(k), ptr(v), clip_quantile,
                                                    max_sweeps, n_threads, ptr(rk), ptr(rv), ctypes.byref(tk),
                                                    ctypes.byref(tv), ptr(ek), ptr(ev)))
    return dict(r_k=rk, r_v=rv, tau_k=tk.value, tau_v=tv.value, eig_k=ek, eig_v=ev)


ROTATION_HADAMARD = 1
ROTATION_IDENTITY = 2


def build_fixed_rotation(variant: int, k_calib, v_calib, clip_quantile: float = 0.999, n_threads: int = 0) -> dict:
    """Comparison rotations (oscar_build_fixed_rotation).  Arrays are [N, H_kv, d]."""
    k = _host_f32(k_calib); v = _host_f32(v_calib)
    n, hkv, d = k.shape
    rk = np.zeros((hkv, d, d)); rv = np.zeros((hkv, d, d))
    tk = ctypes.c_double(); tv = ctypes.c_double()
    ptr = lambda a: a.ctypes.data_as(_P)  # noqa: E731
    _check(load().oscar_build_fixed_rotation(int(variant), d, hkv, n, ptr(k), ptr(v), clip_quantile, n_threads,
                                             ptr(rk), ptr(rv), ctypes.byref(tk), ctypes.byref(tv)))
    return dict(r_k=rk, r_v=rv, tau_k=tk.value, tau_v=tv.value)


# ---------------------------------------------------------- device calls ---


def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise OscarError(1, "expected a device tensor")
    if not t.is_contiguous():
        raise OscarError(1, "expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def int4_page_bytes(d: int, n_kv_heads: int) -> int:
    return load().oscar_int4_page_bytes(d, n_kv_heads)


def make_cache(d: int, n_kv_heads: int, n_sink: int, n_recent: int, int2_pool=None, bf16_pool=None,
               code_bits: int = 2) -> OscarCache:
    """The cache description; with code_bits = 4 the quantized pool is an INT4 pool."""
    c = OscarCache()
    c.d, c.n_kv_heads, c.n_sink, c.n_recent = d, n_kv_heads, n_sink, n_recent
    if int2_pool is not None:
        c.int2_pool = _dptr(int2_pool)
        pb = int2_page_bytes(d, n_kv_heads) if code_bits == 2 else int4_page_bytes(d, n_kv_heads)
        c.n_int2_pages = int2_pool.numel() * int2_pool.element_size() // pb
    if bf16_pool is not None:
        c.bf16_pool = _dptr(bf16_pool)
        c.n_bf16_pages = bf16_pool.numel() * bf16_pool.element_size() // bf16_page_bytes(d, n_kv_heads)
    return c


def quantize_append(cache: OscarCache, k_new, v_new, row_seq, row_pos, bt_q, r_k, r_v, tau_k: float, tau_v: float,
                    stream=None):
    """k_new/v_new bf16 [n, H_kv, d]; row_seq/row_pos int32 [n]; bt_q int32 [B, max_pages]; r_* fp32 [H_kv, d, d]."""
    n = k_new.shape[0]
    _check(load().oscar_quantize_append(ctypes.byref(cache), _dptr(k_new), _dptr(v_new), n, _dptr(row_seq),
                                        _dptr(row_pos), _dptr(bt_q), bt_q.shape[1], _dptr(r_k), _dptr(r_v),
                                        float(tau_k), float(tau_v), _stream(stream)))


def quantize_append_int4(cache: OscarCache, k_new, v_new, row_seq, row_pos, bt_q, r_k, r_v, tau_k: float,
                         tau_v: float, stream=None):
    """As quantize_append, into INT4 pages."""
    n = k_new.shape[0]
    _check(load().oscar_quantize_append_int4(ctypes.byref(cache), _dptr(k_new), _dptr(v_new), n, _dptr(row_seq),
                                             _dptr(row_pos), _dptr(bt_q), bt_q.shape[1], _dptr(r_k), _dptr(r_v),
                                             float(tau_k), float(tau_v), _stream(stream)))


def write_bf16(cache: OscarCache, k_new, v_new, row_seq, row_pos, bt_h, stream=None):
    n = k_new.shape[0]
    _check(load().oscar_write_bf16(ctypes.byref(cache), _dptr(k_new), _dptr(v_new), n, _dptr(row_seq),
                                   _dptr(row_pos), _dptr(bt_h), bt_h.shape[1], _stream(stream)))


def decode_step_update(cache: OscarCache, k_new, v_new, seq_lens, bt_q, bt_h, r_k, r_v, tau_k: float, tau_v: float,
                       stream=None):
    """k_new/v_new bf16 [B, H_kv, d] (the new tokens); seq_lens int32 [B] (lengths with them)."""
    b = k_new.shape[0]
    _check(load().oscar_decode_step_update(ctypes.byref(cache), _dptr(k_new), _dptr(v_new), b, _dptr(seq_lens),
                                           _dptr(bt_q), _dptr(bt_h), bt_q.shape[1], _dptr(r_k), _dptr(r_v),
                                           float(tau_k), float(tau_v), _stream(stream)))


def calib_gram(x, n_kv_heads: int, out=None, stream=None):
    """x device bf16 [N, H_x, d] -> device float64 [H_kv, d, d] (oscar_calib_gram)."""
    import torch
    n, hx, d = x.shape
    if out is None:
        out = torch.empty((n_kv_heads, d, d), dtype=torch.float64, device=x.device)
    _check(load().oscar_calib_gram(_dptr(x), n, hx, n_kv_heads, d, _dptr(out), _stream(stream)))
    return out


def decode_workspace_bytes(batch: int, n_kv_heads: int, n_q_heads: int, d: int, max_seq_len: int,
                           split_pages: int = 0) -> int:
    out = _SZ()
    _check(load().oscar_decode_workspace_bytes(batch, n_kv_heads, n_q_heads, d, max_seq_len, split_pages,
                                               ctypes.byref(out)))
    return out.value


def decode_workspace_init(ws, stream=None):
    _check(load().oscar_decode_workspace_init(_dptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def paged_decode_attn(cache: OscarCache, q, seq_lens, max_seq_len: int, bt_q, bt_h, r_k, r_v, out, workspace,
                      sm_scale: Optional[float] = None, split_pages: int = 0, stream=None):
    """q bf16 [B, H_q, d] -> out bf16 [B, H_q, d]."""
    B, hq, d = q.shape
    sc = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    _check(load().oscar_paged_decode_attn(ctypes.byref(cache), _dptr(q), B, hq, _dptr(seq_lens), max_seq_len,
                                          _dptr(bt_q), _dptr(bt_h), bt_h.shape[1], _dptr(r_k), _dptr(r_v), sc,
                                          split_pages, _dptr(workspace),
                                          workspace.numel() * workspace.element_size(), _dptr(out),
                                          _stream(stream)))


def paged_decode_attn_bf16(cache: OscarCache, q, seq_lens, max_seq_len: int, bt_h, out, workspace,
                           sm_scale: Optional[float] = None, split_pages: int = 0, stream=None):
    B, hq, d = q.shape
    sc = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    _check(load().oscar_paged_decode_attn_bf16(ctypes.byref(cache), _dptr(q), B, hq, _dptr(seq_lens), max_seq_len,
                                               _dptr(bt_h), bt_h.shape[1], sc, split_pages, _dptr(workspace),
                                               workspace.numel() * workspace.element_size(), _dptr(out),
                                               _stream(stream)))


def paged_decode_attn_noalloc(cache: OscarCache, q, seq_lens, max_seq_len: int, bt_q, bt_h, r_k, r_v, out,
                              sm_scale: Optional[float] = None, split_pages: int = 0, stream=None):
    """As paged_decode_attn, with the library's built-in device scratch instead of a workspace."""
    B, hq, d = q.shape
    sc = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    _check(load().oscar_paged_decode_attn_noalloc(ctypes.byref(cache), _dptr(q), B, hq, _dptr(seq_lens),
                                                  max_seq_len, _dptr(bt_q), _dptr(bt_h), bt_h.shape[1], _dptr(r_k),
                                                  _dptr(r_v), sc, split_pages, _dptr(out), _stream(stream)))


def bw_probe_read(buf, sink, stream=None):
    """One streaming read of the device tensor ``buf`` (nothing written back)."""
    _check(load().oscar_bw_probe_read(_dptr(buf), buf.numel() * buf.element_size(), _dptr(sink), _stream(stream)))


def extend_workspace_bytes(batch: int, n_kv_heads: int, n_q_heads: int, d: int, n_sink: int, n_recent: int,
                           max_cache_len: int, max_new: int, split_steps: int = 0) -> int:
    out = _SZ()
    _check(load().oscar_extend_workspace_bytes(batch, n_kv_heads, n_q_heads, d, n_sink, n_recent, max_cache_len,
                                               max_new, split_steps, ctypes.byref(out)))
    return out.value


def paged_extend_attn(cache: OscarCache, code_bits: int, q, k_new, v_new, cu_rows, cache_lens, max_cache_len: int,
                      max_new: int, bt_q, bt_h, r_k, r_v, out, workspace=None, sm_scale: Optional[float] = None,
                      split_steps: int = 0, stream=None):
    """q bf16 [T, H_q, d], k_new/v_new bf16 [T, H_kv, d], cu_rows int32 [B + 1], cache_lens int32 [B]."""
    B = cache_lens.shape[0]
    hq, d = q.shape[1], q.shape[2]
    sc = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    ws = _dptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().oscar_paged_extend_attn(ctypes.byref(cache), code_bits, _dptr(q), _dptr(k_new), _dptr(v_new), B, hq,
                                          _dptr(cu_rows), _dptr(cache_lens), max_cache_len, max_new, _dptr(bt_q),
                                          _dptr(bt_h), bt_h.shape[1], _dptr(r_k), _dptr(r_v), sc, split_steps, ws, wsb,
                                          _dptr(out), _stream(stream)))


def decode_int4_workspace_bytes(batch: int, n_kv_heads: int, n_q_heads: int, d: int, n_sink: int, n_recent: int,
                                max_seq_len: int, split_steps: int = 0) -> int:
    out = _SZ()
    _check(load().oscar_decode_int4_workspace_bytes(batch, n_kv_heads, n_q_heads, d, n_sink, n_recent, max_seq_len,
                                                    split_steps, ctypes.byref(out)))
    return out.value


def paged_decode_attn_int4(cache: OscarCache, q, seq_lens, max_seq_len: int, bt_q, bt_h, r_k, r_v, out,
                           workspace=None, sm_scale: Optional[float] = None, split_steps: int = 0, stream=None):
    B, hq, d = q.shape
    sc = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    ws = _dptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().oscar_paged_decode_attn_int4(ctypes.byref(cache), _dptr(q), B, hq, _dptr(seq_lens), max_seq_len,
                                               _dptr(bt_q), _dptr(bt_h), bt_h.shape[1], _dptr(r_k), _dptr(r_v), sc,
                                               split_steps, ws, wsb, _dptr(out), _stream(stream)))


def decode_step(cache: OscarCache, k_new, v_new, q, seq_lens, max_seq_len: int, bt_q, bt_h, r_k, r_v, tau_k: float,
                tau_v: float, out, workspace, sm_scale: Optional[float] = None, split_pages: int = 0, stream=None):
    """The step's cache update and the decode in one launch (oscar_decode_step)."""
    B, hq, d = q.shape
    sc = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    _check(load().oscar_decode_step(ctypes.byref(cache), _dptr(k_new), _dptr(v_new), _dptr(q), B, hq, _dptr(seq_lens),
                                    max_seq_len, _dptr(bt_q), _dptr(bt_h), bt_h.shape[1], _dptr(r_k), _dptr(r_v),
                                    float(tau_k), float(tau_v), sc, split_pages, _dptr(workspace),
                                    workspace.numel() * workspace.element_size(), _dptr(out), _stream(stream)))
