"""Pins of oracle.layout: hand-derived positions, bijectivity, an exhaustive
byte round trip, slot-local writes."""
import os

import numpy as np
import pytest

from oracle import layout

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(kind):
    out = []
    with open(os.path.join(GOLD, "layout_positions.txt")) as f:
        for line in f:
            if line.startswith(kind + " "):
                out.append([int(v) for v in line.split()[1:]])
    return out


def test_hand_derived_positions():
    for d, m, c, word, bit in _rows("KC"):
        assert layout.kc_position(m, c, d) == (word, bit)
    for d, t, c, word, bit in _rows("VC"):
        assert layout.vc_position(t, c, d) == (word, bit)
    for d, t, g, idx in _rows("VSZ"):
        assert layout.vsz_index(t, g, d) == idx
    for d, *offs in _rows("AREAS"):
        assert list(layout.area_offsets(d)) + [layout.int2_head_bytes(d)] == offs


@pytest.mark.parametrize("d", [64, 128])
def test_positions_are_a_bijection(d):
    for fn in (layout.kc_position, layout.vc_position):
        seen = set()
        for m in range(16):
            for c in range(d):
                w, b = fn(m, c, d)
                assert 0 <= w < d and b % 2 == 0 and 0 <= b < 32
                seen.add((w, b))
        assert len(seen) == 16 * d  # every 2-bit field of the d words used once


@pytest.mark.parametrize("d", [64, 128])
def test_exhaustive_byte_round_trip(d):
    # O8: each of the 256 byte values, placed in every byte of the code areas,
    # reads back as its four 2-bit codes and is rebuilt by writing them.
    pool = layout.Int2Pool(1, 1, d)
    kw, kb, vw, vb, _, _ = layout.position_tables(d)
    for area, wt, bt in ((0, kw, kb), (1, vw, vb)):
        inv = {}
        for m in range(16):
            for c in range(d):
                inv[(int(wt[m, c]), int(bt[m, c]))] = (m, c)
        off = layout.area_offsets(d)[area]
        for byte_idx in range(0, 4 * d, 7):
            word, sub = divmod(byte_idx, 4)
            for val in range(256):
                pool.data[...] = 0
                pool.data[0, 0, off + byte_idx] = val
                got = pool.read(np.zeros(16, np.int64), np.arange(16), 0)[area]
                for k in range(4):
                    m, c = inv[(word, 8 * sub + 2 * k)]
                    assert got[m, c] == (val >> (2 * k)) & 3
                # write the codes back into a zeroed pool -> same byte image
                codes = got.copy()
                pool.data[...] = 0
                zeros16 = np.zeros((16, d // 32), np.float16)
                args = [codes, np.zeros_like(codes)] if area == 0 else [np.zeros_like(codes), codes]
                pool.write(np.zeros(16, np.int64), np.arange(16), 0, *args, zeros16, zeros16, zeros16, zeros16)
                assert pool.data[0, 0, off + byte_idx] == val
                assert int(pool.data[0, 0, off:off + 4 * d].astype(np.int64).sum()) == val


def test_writes_touch_only_their_slot_and_head():
    d = 128
    rng = np.random.default_rng(0)
    pool = layout.Int2Pool(3, 2, d)
    pool.data[...] = rng.integers(0, 256, size=pool.data.shape, dtype=np.uint8)
    before = pool.data.copy()
    codes = rng.integers(0, 4, size=(1, d), dtype=np.uint8)
    f = rng.standard_normal((1, 4)).astype(np.float16)
    pool.write(np.array([1]), np.array([6]), 1, codes, codes[:, ::-1].copy(), f, f * 2, f * 3, f * 4)
    got = pool.read(np.array([1]), np.array([6]), 1)
    assert np.array_equal(got[0], codes) and np.array_equal(got[1], codes[:, ::-1])
    assert np.array_equal(got[2], f) and np.array_equal(got[5], f * 4)
    # every other slot of every head and page reads as before
    other = layout.Int2Pool(3, 2, d, before)
    for p in range(3):
        for h in range(2):
            slots = np.array([s for s in range(16) if not (p == 1 and h == 1 and s == 6)])
            a = pool.read(np.full(len(slots), p), slots, h)
            b = other.read(np.full(len(slots), p), slots, h)
            for x, y in zip(a, b):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_bf16_pool_layout():
    d = 64
    pool = layout.Bf16Pool(2, 2, d)
    k = np.arange(d, dtype=np.uint16)[None, :] + 1000
    v = np.arange(d, dtype=np.uint16)[None, :] + 2000
    pool.write(np.array([1]), np.array([5]), 1, k, v)
    base = (1 * 2 + 1) * 32 * d
    flat = pool.data.reshape(-1)
    assert flat[base + 5 * d + 7] == 1007          # K token-major [slot][d]
    assert flat[base + 16 * d + 7 * 16 + 5] == 2007  # V channel-major [d][slot]
    rk, rv = pool.read(np.array([1]), np.array([5]), 1)
    assert np.array_equal(rk, k) and np.array_equal(rv, v)
