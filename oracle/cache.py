"""Fill oracle page images from raw rows: the reference for quantize-append and
the BF16 store ([TS] 2.2.B), slot by slot, per KV head, for K and V."""
from __future__ import annotations

import dataclasses

import numpy as np

from .attention import regions
from .layout import Bf16Pool, Int2Pool, Int4Pool, bf16_to_f64
from .quant import QuantRows, quantize_rows

PAGE = 16


@dataclasses.dataclass
class AppendResult:
    """Per (tensor, head) quantization record of the appended rows."""
    k: list  # QuantRows per head
    v: list


def quantize_append(pool, k_bits: np.ndarray, v_bits: np.ndarray, row_seq, row_pos, bt_q,
                    r_k, r_v, tau_k: float, tau_v: float, bf16_to_f64, bits: int = 2) -> AppendResult:
    """Quantize rows (bf16 bits [n, H_kv, d]) and store them in their slots
    (an Int2Pool with bits = 2, an Int4Pool with bits = 4)."""
    row_seq = np.asarray(row_seq, np.int64)
    row_pos = np.asarray(row_pos, np.int64)
    page = np.asarray(bt_q)[row_seq, row_pos // PAGE]
    slot = row_pos % PAGE
    kr, vr = [], []
    for h in range(pool.hkv):
        qk = quantize_rows(bf16_to_f64(k_bits[:, h, :]), np.asarray(r_k[h], np.float64), float(tau_k), bits)
        qv = quantize_rows(bf16_to_f64(v_bits[:, h, :]), np.asarray(r_v[h], np.float64), float(tau_v), bits)
        pool.write(page, slot, h, qk.codes, qv.codes, qk.s16, qk.z16, qv.s16, qv.z16)
        kr.append(qk)
        vr.append(qv)
    return AppendResult(kr, vr)


def write_bf16(pool: Bf16Pool, k_bits: np.ndarray, v_bits: np.ndarray, row_seq, row_pos, bt_h):
    row_seq = np.asarray(row_seq, np.int64)
    row_pos = np.asarray(row_pos, np.int64)
    page = np.asarray(bt_h)[row_seq, row_pos // PAGE]
    for h in range(pool.hkv):
        pool.write(page, row_pos % PAGE, h, k_bits[:, h, :], v_bits[:, h, :])


def fill_rows(seq_lens, n_sink: int, n_recent: int, shared_prefix: int = 0):
    """Which token of which sequence goes where when a decode batch's cache is
    filled at once ([TS] 2.2.B "Mixed-Precision Layout": sink and recent tokens
    stay BF16, the middle history is INT2), each physical slot once: tokens
    below ``shared_prefix`` live on pages every sequence aliases, so only
    sequence 0 writes them.

    Returns ((seq, pos) of the middle tokens, (seq, pos) of the sink and recent
    tokens), int64 arrays, sequence-major and ascending in position.
    """
    ms, mp, hs, hp = [], [], [], []
    for b, L in enumerate(np.asarray(seq_lens, np.int64)):
        sink, mid, rec = regions(int(L), n_sink, n_recent)
        lo = shared_prefix if (b > 0 and shared_prefix) else 0
        t_mid = np.arange(max(mid[0], lo), mid[1], dtype=np.int64)
        t_raw = np.concatenate([np.arange(*sink), np.arange(*rec)]).astype(np.int64)
        t_raw = t_raw[t_raw >= lo]
        ms.append(np.full(len(t_mid), b, np.int64)); mp.append(t_mid)
        hs.append(np.full(len(t_raw), b, np.int64)); hp.append(t_raw)
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return (cat(ms), cat(mp)), (cat(hs), cat(hp))


def build_from_inputs(inp, r_k, r_v, tau_k: float, tau_v: float, bits: int = 2):
    """Oracle page images for a generated decode batch: every middle row
    quantized into its INT2 slot, every sink/recent row stored in its BF16
    slot (the split into regions taken here, by ``fill_rows``).  Returns
    (int2 pool, bf16 pool, AppendResult, middle row triple (seq, pos, row))."""
    w = inp.w
    int2 = (Int2Pool if bits == 2 else Int4Pool)(inp.n_int2_pages, w.n_kv_heads, w.d)
    bf = Bf16Pool(inp.n_bf16_pages, w.n_kv_heads, w.d)
    (ms, mp), (hs, hp) = fill_rows(inp.seq_lens, w.n_sink, w.n_recent, w.shared_prefix)
    mr = np.array([inp.row_of[b][t] for b, t in zip(ms, mp)], np.int64)
    hr = np.array([inp.row_of[b][t] for b, t in zip(hs, hp)], np.int64)
    res = quantize_append(int2, inp.k_rows[mr], inp.v_rows[mr], ms, mp, inp.bt_q, r_k, r_v, tau_k, tau_v,
                          bf16_to_f64, bits)
    write_bf16(bf, inp.k_rows[hr], inp.v_rows[hr], hs, hp, inp.bt_h)
    return int2, bf, res, (ms, mp, mr)


def decode_step_update(int2: Int2Pool, bf: Bf16Pool, k_new: np.ndarray, v_new: np.ndarray, seq_lens, bt_q, bt_h,
                       n_sink: int, n_recent: int, r_k, r_v, tau_k: float, tau_v: float, bf16_to_f64):
    """One decode step's cache writes under the mixed-precision layout
    ([TS] 2.2.B: sink and recent tokens in BF16, the middle history in INT2).

    For sequence b of length L (its new token at L - 1 included): the new
    token goes to its BF16 slot if it is a sink or recent token; the token
    that enters the middle history at this length (L - 1 - W, the one leaving
    the recent window; L - 1 itself when W = 0) is quantized into its INT2
    slot, its raw row taken from its BF16 slot (W >= 1) or from the new row.
    Returns (AppendResult of the quantized rows, their (seq, pos) arrays).
    """
    rows_k, rows_v, seqs, poss = [], [], [], []
    new_seq, new_pos = [], []
    bt_q = np.asarray(bt_q); bt_h = np.asarray(bt_h)
    for b, L in enumerate(np.asarray(seq_lens, np.int64)):
        if L < 1:
            continue
        p = int(L) - 1
        t = p - n_recent if n_recent >= 1 else p
        if t >= n_sink:
            if n_recent >= 1:
                pg, sl = bt_h[b, t // PAGE], t % PAGE
                kv = [bf.read(np.array([pg]), np.array([sl]), h) for h in range(bf.hkv)]
                rows_k.append(np.stack([x[0][0] for x in kv]))
                rows_v.append(np.stack([x[1][0] for x in kv]))
            else:
                rows_k.append(k_new[b]); rows_v.append(v_new[b])
            seqs.append(b); poss.append(t)
        if n_recent >= 1 or p < n_sink:
            new_seq.append(b); new_pos.append(p)
    res = None
    if seqs:
        res = quantize_append(int2, np.stack(rows_k), np.stack(rows_v), seqs, poss, bt_q, r_k, r_v, tau_k, tau_v,
                              bf16_to_f64)
    if new_seq:
        write_bf16(bf, k_new[new_seq], v_new[new_seq], new_seq, new_pos, bt_h)
    return res, (np.array(seqs, np.int64), np.array(poss, np.int64))
