"""The C-ABI library (CPU side): it loads, exports every symbol the header
declares, and rejects bad host-visible arguments before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from int2_rotated_kv_oscar_amd import lib

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "oscar.h")


def _declared():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(lib.EXPORTS)
    L = lib.load()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_geometry():
    L = lib.load()
    assert L.oscar_status_string(0) == b"OSCAR_OK"
    assert L.oscar_status_string(4) == b"OSCAR_ERR_WORKSPACE"
    assert lib.version() == 1
    assert lib.int2_page_bytes(128, 8) == 8 * 1536 and lib.int2_page_bytes(64, 1) == 768
    assert lib.bf16_page_bytes(128, 8) == 8 * 16 * 128 * 2 * 2
    assert lib.int2_page_bytes(96, 1) == 0


def test_workspace_planning():
    # split_pages = 64: per (sequence, KV head) one BF16 item and ceil(2048 / 64)
    # INT2 items of 64 pages, one record each
    b = lib.decode_workspace_bytes(1, 8, 32, 128, 32768, 64)
    rec = (2 * 4 + 4 * 128 + 1 + 3) // 4 * 4
    assert b == 256 + 8 * (1 + 2048 // 64) * rec * 4
    assert lib.decode_workspace_bytes(0, 8, 32, 128, 0) == 0
    for bad, status in (((1, 8, 30, 128, 100, 0), 1), ((1, 1, 17, 128, 100, 0), 2), ((1, 1, 4, 96, 100, 0), 2),
                        ((1, 1, 4, 128, 100, 12), 1), ((-1, 1, 4, 128, 100, 0), 1),
                        ((1, 1, 4, 128, 32768, 8), 2),  # 2048 pages in 8-page items: more than 256 records
                        ((16, 1, 4, 128, 2 ** 31 - 1, 0), 2)):  # 2^31 pages of work or more in one call
        with pytest.raises(lib.OscarError) as e:
            lib.decode_workspace_bytes(*bad)
        assert e.value.status == status


def test_attention_chunk_planning():
    # chunks of split_steps 32-token steps: the quantized page pairs in chunks
    # of their own, then the raw steps (and new-row tiles); one record of
    # 4 + 2d floats per column (16 per decode tile, 256 per extend tile at d = 128)
    rec = (4 + 2 * 128) * 4
    # a 32k sequence, 8 KV heads, S = 4, W = 128: 1025 quantized steps, 6 raw
    assert lib.decode_int4_workspace_bytes(1, 8, 32, 128, 4, 128, 32768, 16) == 8 * (65 + 1) * 16 * rec
    # automatic (256 CUs here and on the MI355X): at most three workgroups per CU
    auto = lib.decode_int4_workspace_bytes(1, 8, 32, 128, 4, 128, 32768) // (8 * 16 * rec)
    assert auto == 95 and 8 * auto <= 3 * 256
    auto4 = lib.decode_int4_workspace_bytes(4, 8, 64, 128, 4, 128, 131072) // (32 * 16 * rec)
    assert 32 * auto4 <= 3 * 256 and auto4 >= 16
    # one chunk suffices: no workspace
    assert lib.decode_int4_workspace_bytes(1, 1, 4, 64, 4, 32, 100, 64) == 0
    # extend: 512 new rows x 4 heads = 8 column tiles of 256; 6 raw steps + 16
    # new-row tiles in 3 chunks of 8, the 1025 quantized steps in 129
    assert lib.extend_workspace_bytes(1, 1, 4, 128, 4, 128, 32768, 512, 8) == 8 * (129 + 3) * 256 * rec
    for bad, status in (((1, 8, 30, 128, 4, 128, 100, 0), 1), ((1, 1, 4, 96, 4, 128, 100, 0), 2),
                        ((1, 1, 4, 128, 4, 128, 100, -1), 1), ((1, 1, 4, 128, 4, 128, 2 ** 20, 1), 2)):
        with pytest.raises(lib.OscarError) as e:
            lib.decode_int4_workspace_bytes(*bad)
        assert e.value.status == status


def test_device_calls_validate_before_launch():
    L = lib.load()
    c = lib.OscarCache()
    c.d, c.n_kv_heads = 96, 1
    assert L.oscar_quantize_append(ctypes.byref(c), None, None, 1, None, None, None, 1, None, None, 1.0, 1.0, None) == 2
    c.d = 128
    assert L.oscar_quantize_append(ctypes.byref(c), None, None, 1, None, None, None, 1, None, None, 1.0, 1.0, None) == 1
    assert L.oscar_quantize_append(None, None, None, 1, None, None, None, 1, None, None, 1.0, 1.0, None) == 1
    assert b"cache is NULL" in L.oscar_last_error()
    c.int2_pool, c.n_int2_pages = 16, 1   # never dereferenced: validation fails first
    assert L.oscar_quantize_append(ctypes.byref(c), None, None, 0, None, None, None, 1, None, None, 1.0, 1.0, None) == 0
    assert L.oscar_quantize_append(ctypes.byref(c), None, None, -1, None, None, None, 1, None, None, 1.0, 1.0, None) == 1
    c.bf16_pool, c.n_bf16_pages = 16, 1
    # batch 0 is a no-op; a missing workspace is reported before any launch
    assert L.oscar_paged_decode_attn(ctypes.byref(c), None, 0, 4, None, 0, None, None, 1, None, None, 0.1, 0,
                                     None, 0, None, None) == 0
    assert L.oscar_paged_decode_attn(ctypes.byref(c), 16, 1, 4, 16, 32, 16, 16, 2, 16, 16, 0.1, 0,
                                     None, 0, 16, None) == 4
    assert L.oscar_paged_decode_attn(ctypes.byref(c), 16, 1, 4, 16, 33, 16, 16, 2, 16, 16, 0.1, 0,
                                     16, 1 << 20, 16, None) == 1   # max_seq_len > 16 * max_pages
    # decode-step update: both pools required, batch 0 a no-op, then pointers and clips
    c2 = lib.OscarCache()
    c2.d, c2.n_kv_heads, c2.n_recent = 128, 1, 4
    c2.int2_pool, c2.n_int2_pages = 16, 1
    assert L.oscar_decode_step_update(ctypes.byref(c2), 16, 16, 1, 16, 16, 16, 1, 16, 16, 1.0, 1.0, None) == 1
    assert b"BF16 pool missing" in L.oscar_last_error()
    c2.bf16_pool, c2.n_bf16_pages = 16, 1
    assert L.oscar_decode_step_update(ctypes.byref(c2), None, None, 0, None, None, None, 1, None, None, 1.0, 1.0,
                                      None) == 0
    assert L.oscar_decode_step_update(ctypes.byref(c2), 16, 16, -1, 16, 16, 16, 1, 16, 16, 1.0, 1.0, None) == 1
    assert L.oscar_decode_step_update(ctypes.byref(c2), 16, 16, 1, 16, None, 16, 1, 16, 16, 1.0, 1.0, None) == 1
    assert L.oscar_decode_step_update(ctypes.byref(c2), 16, 16, 1, 16, 16, 16, 1, 16, 16, 0.0, 1.0, None) == 1
    # calibration Gram: validated before any launch
    assert L.oscar_calib_gram(None, 8, 4, 1, 128, 16, None) == 1
    assert L.oscar_calib_gram(16, 8, 4, 1, 96, 16, None) == 2
    assert L.oscar_calib_gram(16, 8, 6, 4, 128, 16, None) == 1     # 6 heads over 4 KV heads
    assert L.oscar_calib_gram(24, 8, 4, 1, 128, 16, None) == 1     # not 16-byte aligned
    assert b"aligned" in L.oscar_last_error()
    assert L.oscar_calib_gram(16, 0, 4, 1, 128, 16, None) == 1
    assert L.oscar_calib_gram(16, 8, 17, 1, 128, 16, None) == 2    # 17 heads per KV group
    assert L.oscar_decode_workspace_init(None, 64, None) == 4


def test_build_rotation_validation():
    q = np.zeros((4, 2, 64), np.float32); k = np.zeros((4, 1, 64), np.float32)
    with pytest.raises(lib.OscarError) as e:
        lib.build_rotation(q, k, k, 2, clip_quantile=1.5)
    assert e.value.status == 1
    bad = k.copy(); bad[0, 0, 0] = np.nan
    with pytest.raises(lib.OscarError) as e:
        lib.build_rotation(q, bad, k, 2)
    assert e.value.status == 3
    with pytest.raises(lib.OscarError) as e:
        lib.build_rotation(np.zeros((4, 1, 96), np.float32), np.zeros((4, 1, 96), np.float32),
                           np.zeros((4, 1, 96), np.float32), 1)
    assert e.value.status == 2
