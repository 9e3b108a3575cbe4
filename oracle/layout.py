"""Page images of the paged mixed-precision cache, written from the prose
definition of the layout (INT2 pages: codes, f16 scales and zeros per slot;
BF16 pages: raw K token-major, raw V channel-major).

[TS] 2.2.B: sink/recent tokens in BF16 pages, the middle history in INT2
pages, paged and compatible with prefix caching.  The byte and bit positions
are this build's own choice; this module restates them independently of the
HIP library so that a mismatch in either shows up as a parity failure.
"""
from __future__ import annotations

import numpy as np

PAGE = 16
GROUP = 32


def int2_head_bytes(d: int) -> int:
    return 12 * d


def bf16_head_elems(d: int) -> int:
    return 32 * d


def area_offsets(d: int):
    """Byte offsets of KC, VC, KS, KZ, VS, VZ inside one page-head."""
    ng = d // GROUP
    kc = 0
    vc = kc + 4 * d
    ks = vc + 4 * d
    kz = ks + 2 * PAGE * ng
    vs = kz + 2 * PAGE * ng
    vz = vs + 2 * PAGE * ng
    return kc, vc, ks, kz, vs, vz


def kc_position(m: int, c: int, d: int):
    """(word, bit) of the K code of slot m, channel c."""
    n_w = d // 64
    g, hb, quad, r = c // 32, (c // 16) % 2, (c // 4) % 4, c % 4
    w = g // 2
    return (quad * 16 + m) * n_w + w, 16 * (r % 2) + 8 * (g % 2) + 4 * hb + 2 * (r // 2)


def vc_position(t: int, c: int, d: int):
    """(word, bit) of the V code of slot t, channel c."""
    n_w = d // 64
    q, r = t // 4, t % 4
    c16, blk = c % 16, c // 16
    w, bb = blk // 4, blk % 4
    return (q * 16 + c16) * n_w + w, 16 * (r % 2) + 8 * (r // 2) + 2 * bb


def vsz_index(t: int, g: int, d: int) -> int:
    """f16 index of the V scale/zero of slot t, group g."""
    ng = d // GROUP
    return ((t // 4) * ng + g) * 4 + t % 4


def position_tables(d: int):
    """Arrays [16, d] of (word, bit) for KC and VC, and [16, n_g] f16 indices."""
    ng = d // GROUP
    kw = np.zeros((PAGE, d), np.int64); kb = np.zeros((PAGE, d), np.int64)
    vw = np.zeros((PAGE, d), np.int64); vb = np.zeros((PAGE, d), np.int64)
    for m in range(PAGE):
        for c in range(d):
            kw[m, c], kb[m, c] = kc_position(m, c, d)
            vw[m, c], vb[m, c] = vc_position(m, c, d)
    ksi = np.array([[m * ng + g for g in range(ng)] for m in range(PAGE)])
    vsi = np.array([[vsz_index(m, g, d) for g in range(ng)] for m in range(PAGE)])
    return kw, kb, vw, vb, ksi, vsi


class Int2Pool:
    """uint8 [n_pages, H_kv, 12 d] with slot-level writes and reads."""

    def __init__(self, n_pages: int, n_kv_heads: int, d: int, data: np.ndarray | None = None):
        self.d, self.hkv, self.n_pages = d, n_kv_heads, n_pages
        nb = int2_head_bytes(d)
        if data is None:
            data = np.zeros((n_pages, n_kv_heads, nb), np.uint8)
        self.data = np.ascontiguousarray(data, dtype=np.uint8).reshape(n_pages, n_kv_heads, nb)
        self.tab = position_tables(d)
        self.off = area_offsets(d)

    def _words(self, area: int) -> np.ndarray:
        o = self.off[area]
        return self.data[:, :, o:o + 4 * self.d].view(np.uint32)  # [P, H, d]

    def _halves(self, area: int) -> np.ndarray:
        ng = self.d // GROUP
        o = self.off[area]
        return self.data[:, :, o:o + 2 * PAGE * ng].view(np.float16)  # [P, H, 16 ng]

    def write(self, page: np.ndarray, slot: np.ndarray, head: int, codes_k, codes_v, ks, kz, vs, vz):
        """Store rows (one per (page, slot)) for one head; codes uint8 [n, d], f16 [n, n_g]."""
        kw, kb, vw, vb, ksi, vsi = self.tab
        page = np.asarray(page, np.int64); slot = np.asarray(slot, np.int64)
        for area, wt, bt, codes in ((0, kw, kb, codes_k), (1, vw, vb, codes_v)):
            words = self._words(area)
            wi = wt[slot]                      # [n, d]
            bi = bt[slot].astype(np.uint32)
            pg = np.broadcast_to(page[:, None], wi.shape)
            clear = ~(np.uint32(3) << bi)
            setv = (np.asarray(codes, np.uint32) & 3) << bi
            np.bitwise_and.at(words, (pg, head, wi), clear)
            np.bitwise_or.at(words, (pg, head, wi), setv)
        for area, it, vals in ((2, ksi, ks), (3, ksi, kz), (4, vsi, vs), (5, vsi, vz)):
            halves = self._halves(area)
            halves[page[:, None], head, it[slot]] = np.asarray(vals, np.float16)

    def read(self, page: np.ndarray, slot: np.ndarray, head: int):
        """(codes_k, codes_v uint8 [n, d], ks, kz, vs, vz f16 [n, n_g]) of rows."""
        kw, kb, vw, vb, ksi, vsi = self.tab
        page = np.asarray(page, np.int64); slot = np.asarray(slot, np.int64)
        out = []
        for area, wt, bt in ((0, kw, kb), (1, vw, vb)):
            words = self._words(area)
            w = words[page[:, None], head, wt[slot]]
            out.append(((w >> bt[slot].astype(np.uint32)) & 3).astype(np.uint8))
        for area, it in ((2, ksi), (3, ksi), (4, vsi), (5, vsi)):
            out.append(self._halves(area)[page[:, None], head, it[slot]].copy())
        return tuple(out)


def int4_head_bytes(d: int) -> int:
    return 20 * d


class Int4Pool:
    """INT4 page images, uint8 [n_pages, H_kv, 20 d].  One page-head holds,
    one after the other: K codes [16 slots][d/2] bytes, V codes [16][d/2]
    (channel 2i in the low nibble of byte i, channel 2i + 1 in the high
    nibble), then f16 K scales [16][n_g], K zeros [16][n_g], V scales
    [16][n_g], V zeros [16][n_g].  Every slot owns its bytes."""

    def __init__(self, n_pages: int, n_kv_heads: int, d: int, data: np.ndarray | None = None):
        self.d, self.hkv, self.n_pages = d, n_kv_heads, n_pages
        nb = int4_head_bytes(d)
        if data is None:
            data = np.zeros((n_pages, n_kv_heads, nb), np.uint8)
        self.data = np.ascontiguousarray(data, dtype=np.uint8).reshape(n_pages, n_kv_heads, nb)
        ng = d // GROUP
        self.off_codes = (0, PAGE * d // 2)
        base = PAGE * d
        self.off_sz = tuple(base + 2 * PAGE * ng * i for i in range(4))

    def _codes(self, area: int) -> np.ndarray:
        o = self.off_codes[area]
        return self.data[:, :, o:o + PAGE * self.d // 2].reshape(self.n_pages, self.hkv, PAGE, self.d // 2)

    def _halves(self, area: int) -> np.ndarray:
        ng = self.d // GROUP
        o = self.off_sz[area]
        return self.data[:, :, o:o + 2 * PAGE * ng].view(np.float16).reshape(self.n_pages, self.hkv, PAGE, ng)

    def write(self, page, slot, head: int, codes_k, codes_v, ks, kz, vs, vz):
        page = np.asarray(page, np.int64); slot = np.asarray(slot, np.int64)
        for area, codes in ((0, codes_k), (1, codes_v)):
            c = np.asarray(codes, np.uint8) & 15
            self._codes(area)[page, head, slot] = c[:, 0::2] | (c[:, 1::2] << 4)
        for area, vals in ((0, ks), (1, kz), (2, vs), (3, vz)):
            self._halves(area)[page, head, slot] = np.asarray(vals, np.float16)

    def read(self, page, slot, head: int):
        page = np.asarray(page, np.int64); slot = np.asarray(slot, np.int64)
        out = []
        for area in (0, 1):
            b = self._codes(area)[page, head, slot]
            c = np.empty((len(page), self.d), np.uint8)
            c[:, 0::2] = b & 15
            c[:, 1::2] = b >> 4
            out.append(c)
        for area in range(4):
            out.append(self._halves(area)[page, head, slot].copy())
        return tuple(out)


class Bf16Pool:
    """uint16 (bf16 bits) [n_pages, H_kv, 32 d]: K [16][d] then V [d][16]."""

    def __init__(self, n_pages: int, n_kv_heads: int, d: int, data: np.ndarray | None = None):
        self.d, self.hkv, self.n_pages = d, n_kv_heads, n_pages
        if data is None:
            data = np.zeros((n_pages, n_kv_heads, bf16_head_elems(d)), np.uint16)
        self.data = np.ascontiguousarray(data, dtype=np.uint16).reshape(n_pages, n_kv_heads, 32 * d)

    def write(self, page, slot, head: int, k_bits, v_bits):
        d = self.d
        page = np.asarray(page, np.int64); slot = np.asarray(slot, np.int64)
        self.data[page[:, None], head, slot[:, None] * d + np.arange(d)[None, :]] = k_bits
        self.data[page[:, None], head, 16 * d + np.arange(d)[None, :] * 16 + slot[:, None]] = v_bits

    def read(self, page, slot, head: int):
        d = self.d
        page = np.asarray(page, np.int64); slot = np.asarray(slot, np.int64)
        k = self.data[page[:, None], head, slot[:, None] * d + np.arange(d)[None, :]]
        v = self.data[page[:, None], head, 16 * d + np.arange(d)[None, :] * 16 + slot[:, None]]
        return k.copy(), v.copy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
