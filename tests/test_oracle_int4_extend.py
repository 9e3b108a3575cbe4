"""Pins of the INT4 cache variant (16-level quantizer, INT4 page images) and
of the chunked-prefill ("extend") attention over the mixed cache ([TS] 2.2.B
"Kernel Integration": paged, prefix-cache compatible; [TS] 4 "Scalability":
the INT4 KV baseline)."""
import os

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import cache as oc
from oracle import layout, quant

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "int4_layout_positions.txt")


def _orth(rng, d):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


# ------------------------------------------------------------- INT4 ------


def test_int4_nearest_level_brute_force():
    # every code is the nearest of the 16 levels z16 + c s16 (ties only at
    # exact midpoints), the extremes of a group map to 0 and 15
    rng = np.random.default_rng(3)
    y = rng.standard_normal((50, 64)) * rng.choice([0.01, 1, 30], size=(50, 1))
    qr = quant.quantize_rotated(y, bits=4)
    s = qr.s16.astype(np.float64).repeat(32, axis=1)
    z = qr.z16.astype(np.float64).repeat(32, axis=1)
    lv = z[..., None] + np.arange(16)[None, None, :] * s[..., None]
    dist = np.abs(y[..., None] - lv)
    best = dist.min(axis=2)
    got = np.take_along_axis(dist, qr.codes[..., None].astype(np.int64), axis=2)[..., 0]
    near_tie = quant.boundary_distance(qr.t, bits=4) < 1e-9
    assert np.all((got <= best + 1e-12) | near_tie)
    assert qr.codes.max() <= 15


def test_int4_hand_group_and_grid():
    # a group on the grid z + c s with f16-exact s and z decodes exactly, and
    # its codes are 0..15; the range/15 scale: (8.5 - 1) / 15 = 0.5
    y = np.concatenate([1.0 + 0.5 * np.arange(16), 1.0 + 0.5 * np.arange(16)[::-1]])[None]
    qr = quant.quantize_rotated(y, bits=4)
    assert float(qr.s16[0, 0]) == 0.5 and float(qr.z16[0, 0]) == 1.0
    assert qr.codes[0].tolist() == list(range(16)) + list(range(15, -1, -1))
    np.testing.assert_array_equal(quant.dequantize(qr.codes, qr.s16, qr.z16), y)
    # a constant group: scale 0, every code 0, decodes to the f16 zero
    qc = quant.quantize_rotated(np.full((1, 32), 0.3), bits=4)
    assert float(qc.s16[0, 0]) == 0.0 and qc.codes.max() == 0


def test_int4_exhaustive_nibble_round_trip():
    # all 256 byte values <-> all 16 x 16 code pairs, in K and V areas, every slot
    d = 64
    pool = layout.Int4Pool(2, 1, d)
    pairs = np.array([(a, b) for a in range(16) for b in range(16)], np.uint8)  # 256 pairs
    codes = np.concatenate([pairs.reshape(8, 64), pairs[::-1].reshape(8, 64)])
    zs = np.zeros((16, 2), np.float16)
    pool.write(np.zeros(16, np.int64), np.arange(16), 0, codes, codes[::-1], zs, zs, zs, zs)
    ck, cv, *_ = pool.read(np.zeros(16, np.int64), np.arange(16), 0)
    np.testing.assert_array_equal(ck, codes)
    np.testing.assert_array_equal(cv, codes[::-1])
    # the bytes hold exactly low | high << 4
    kb = pool.data[0, 0, :16 * 32].reshape(16, 32)
    np.testing.assert_array_equal(kb, codes[:, 0::2] | (codes[:, 1::2] << 4))
    assert sorted(set(kb.reshape(-1).tolist())) == list(range(256))


def test_int4_hand_derived_positions():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        d, area = int(f[0]), f[1]
        ng = d // 32
        pool = layout.Int4Pool(1, 1, d)
        zc = np.zeros((1, d), np.uint8)
        zs = np.zeros((1, ng), np.float16)
        if area in ("K", "V"):
            m, c, byte, shift = map(int, f[2:])
            code = zc.copy(); code[0, c] = 9
            pool.write([0], [m], 0, code if area == "K" else zc, code if area == "V" else zc, zs, zs, zs, zs)
            nz = np.nonzero(pool.data[0, 0])[0]
            assert nz.tolist() == [byte] and pool.data[0, 0, byte] == 9 << shift, line
        else:
            m, g, byte = map(int, f[2:])
            v = zs.copy(); v[0, g] = np.float16(1.5)  # bits 0x3E00: the high byte is nonzero
            args = [v if area == a else zs for a in ("KS", "KZ", "VS", "VZ")]
            pool.write([0], [m], 0, zc, zc, *args)
            assert pool.data[0, 0].view(np.uint16)[byte // 2] == 0x3E00 and np.count_nonzero(pool.data) == 1, line


def test_int4_fill_through_cache_helpers():
    # the bits-aware cache fill writes decodable INT4 rows: dequantized rows
    # are within half a step of the rotated, clipped rows
    rng = np.random.default_rng(5)
    d, n = 64, 40
    r = _orth(rng, d)[None]
    xb = (rng.standard_normal((n, 1, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pool = layout.Int4Pool(3, 1, d)
    res = oc.quantize_append(pool, xb, xb, np.zeros(n), np.arange(n), np.arange(3)[None], r, r, 3.0, 3.0,
                             layout.bf16_to_f64, bits=4)
    ck, cv, ks, kz, vs, vz = pool.read(np.arange(n) // 16, np.arange(n) % 16, 0)
    yk = quant.dequantize(ck, ks, kz)
    step = ks.astype(np.float64).repeat(32, axis=1)
    assert np.all(np.abs(yk - res.k[0].y) <= 0.5 * step + 1e-3 * step + 1e-12)


# ----------------------------------------------------------- extend ------


def _cache(rng, d, hkv, P, S, W, bits):
    """A one-sequence cache of length P built by the oracle's fill, identity tables."""
    rk = np.stack([_orth(rng, d) for _ in range(hkv)])
    rv = np.stack([_orth(rng, d) for _ in range(hkv)])
    n_pages = max(1, (P + 15) // 16)
    k = rng.standard_normal((max(P, 1), hkv, d)); k[:, :, 3] *= 10
    v = rng.standard_normal((max(P, 1), hkv, d))
    kb = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pool = (layout.Int2Pool if bits == 2 else layout.Int4Pool)(n_pages + 2, hkv, d)
    bf = layout.Bf16Pool(n_pages + 2, hkv, d)
    bt = np.arange(n_pages + 2, dtype=np.int64)[None]
    (ms, mp), (hs, hp) = oc.fill_rows([P], S, W)
    if len(ms):
        oc.quantize_append(pool, kb[mp], vb[mp], ms, mp, bt, rk, rv, 50.0, 50.0, layout.bf16_to_f64, bits)
    if len(hs):
        oc.write_bf16(bf, kb[hp], vb[hp], hs, hp, bt)
    return pool, bf, bt, rk, rv


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("P,S,W", [(150, 4, 32), (40, 4, 32), (0, 4, 32), (77, 0, 0), (200, 16, 0)])
def test_extend_equals_decode_with_the_window_widened(bits, P, S, W):
    # row i of the extend (position P + i) equals a decode at length P + i + 1
    # whose recent window also holds the new rows 0..i in BF16 pages: the
    # regions of that cache are the prefix's, plus the new tokens as raw rows
    rng = np.random.default_rng(P + S + W + bits)
    d, hkv, G, n = 64, 2, 3, 9
    pool, bf, bt, rk, rv = _cache(rng, d, hkv, P, S, W, bits)
    q = rng.standard_normal((n, hkv * G, d))
    kn = rng.standard_normal((n, hkv, d)); vn = rng.standard_normal((n, hkv, d))
    knb = (kn.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vnb = (vn.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kn64, vn64 = layout.bf16_to_f64(knb), layout.bf16_to_f64(vnb)
    got = att.extend_attention(q, kn64, vn64, pool, bf, [0, n], [P], bt, bt, rk, rv, S, W)
    bf2 = layout.Bf16Pool(bf.n_pages, hkv, d, bf.data.copy())
    for i in range(n):
        oc.write_bf16(bf2, knb[i:i + 1], vnb[i:i + 1], [0], [P + i], bt)
        ref = att.decode_attention(q[i:i + 1], pool, bf2, [P + i + 1], bt, bt, rk, rv, S, W + i + 1)
        np.testing.assert_allclose(got[i], ref[0], rtol=1e-12, atol=1e-12)


def test_extend_without_prefix_is_causal_sdpa():
    # P = 0: causal attention of the new rows alone, as torch's SDPA computes it
    rng = np.random.default_rng(8)
    d, n, hkv, G = 64, 23, 1, 4
    pool = layout.Int2Pool(1, hkv, d); bf = layout.Bf16Pool(1, hkv, d)
    q = rng.standard_normal((n, hkv * G, d)); kn = rng.standard_normal((n, hkv, d)); vn = rng.standard_normal((n, hkv, d))
    got = att.extend_attention(q, kn, vn, pool, bf, [0, n], [0], np.zeros((1, 1), np.int64), np.zeros((1, 1), np.int64),
                               np.eye(d)[None], np.eye(d)[None], 4, 32)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q).permute(1, 0, 2), torch.tensor(kn[:, 0])[None].expand(G, n, d),
        torch.tensor(vn[:, 0])[None].expand(G, n, d), is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_extend_brute_force_small():
    # scalar loops over one short case: decode every cached token from its
    # codes, rotate middle rows back by hand, explicit exp sums
    rng = np.random.default_rng(13)
    d, hkv, G, n, P, S, W = 64, 1, 2, 3, 21, 2, 3
    pool, bf, bt, rk, rv = _cache(rng, d, hkv, P, S, W, 2)
    q = rng.standard_normal((n, G, d)); kn = rng.standard_normal((n, 1, d)); vn = rng.standard_normal((n, 1, d))
    got = att.extend_attention(q, kn, vn, pool, bf, [0, n], [P], bt, bt, rk, rv, S, W)
    keys, vals = [], []
    for t in range(P):
        if t < S or t >= P - W:
            kb, vb = bf.read([t // 16], [t % 16], 0)
            keys.append(layout.bf16_to_f64(kb)[0]); vals.append(layout.bf16_to_f64(vb)[0])
        else:
            ck, cv, ks, kz, vs, vz = pool.read([t // 16], [t % 16], 0)
            kh = [int(ck[0, c]) * float(ks[0, c // 32]) + float(kz[0, c // 32]) for c in range(d)]
            vh = [int(cv[0, c]) * float(vs[0, c // 32]) + float(vz[0, c // 32]) for c in range(d)]
            keys.append(np.array([sum(kh[j] * rk[0][c, j] for j in range(d)) for c in range(d)]))
            vals.append(np.array([sum(vh[j] * rv[0][c, j] for j in range(d)) for c in range(d)]))
    for i in range(n):
        ks_ = keys + [kn[j, 0] for j in range(i + 1)]
        vs_ = vals + [vn[j, 0] for j in range(i + 1)]
        for g in range(G):
            lg = [sum(q[i, g, c] * kk[c] for c in range(d)) / 8.0 for kk in ks_]
            mx = max(lg)
            e = [np.exp(x - mx) for x in lg]
            o = sum(ei * vv for ei, vv in zip(e, vs_)) / sum(e)
            np.testing.assert_allclose(got[i, g], o, rtol=1e-11, atol=1e-12)


def test_extend_row_subset_equals_full_rows():
    rng = np.random.default_rng(21)
    d, hkv, G, n, P = 64, 1, 2, 12, 90
    pool, bf, bt, rk, rv = _cache(rng, d, hkv, P, 4, 32, 2)
    q = rng.standard_normal((n, G, d)); kn = rng.standard_normal((n, 1, d)); vn = rng.standard_normal((n, 1, d))
    full = att.extend_attention(q, kn, vn, pool, bf, [0, n], [P], bt, bt, rk, rv, 4, 32)
    sub = att.extend_attention(q, kn, vn, pool, bf, [0, n], [P], bt, bt, rk, rv, 4, 32, rows={3, 11})
    np.testing.assert_array_equal(sub[[3, 11]], full[[3, 11]])
    assert not sub[[0, 1, 2, 4, 10]].any()
