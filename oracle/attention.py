"""Decode attention over the mixed paged cache (fp64), and its building blocks.

[TS] 2.2.B "kernel integration": unpacking, dequantization, inverse rotation
and attention for the INT2 history, with BF16 sink and recent tokens; [AB].
The method reaches exactly softmax attention over the decoded cache mapped
back to the original basis.  Because R is orthogonal,
  (q R_K) . kh = q . (kh R_K^T)   and   (sum p vh) R_V^T = sum p (vh R_V^T),
so this module computes the output the direct way (decode each middle key and
value, rotate it back with R^T, then plain softmax attention) in
``decode_attention``; ``decode_attention_rotated`` takes the rotated-space
route that a fused kernel takes, and the tests check the two agree.

Readings: scale 1/sqrt(d) unless given; query head i reads KV head i // G;
regions sink = [0, min(S, L)), recent = [max(S, L - W), L), middle = the rest.
"""
from __future__ import annotations

import numpy as np

from .layout import Bf16Pool, Int2Pool, bf16_to_f64
from .quant import dequantize

PAGE = 16


def regions(L: int, S: int, W: int):
    sink = (0, min(S, L))
    rec = (max(S, L - W), L)
    mid = (S, L - W) if L - W > S else (S, S)
    return sink, mid, rec


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q k^T scale) v for q [G, d], k/v [L, d]; the textbook definition."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def sequence_kv(int2: Int2Pool, bf16: Bf16Pool, bt_q_row, bt_h_row, L: int, S: int, W: int, h: int):
    """Decoded cache of one (sequence, KV head).

    Returns (raw_idx, k_raw, v_raw, mid_idx, k_rot, v_rot): token positions and
    float64 rows of the BF16 regions (raw) and of the middle (rotated, decoded).
    """
    sink, mid, rec = regions(L, S, W)
    raw_idx = np.concatenate([np.arange(*sink), np.arange(*rec)]).astype(np.int64)
    mid_idx = np.arange(*mid, dtype=np.int64)
    d = int2.d
    if raw_idx.size:
        kb, vb = bf16.read(np.asarray(bt_h_row)[raw_idx // PAGE], raw_idx % PAGE, h)
        k_raw, v_raw = bf16_to_f64(kb), bf16_to_f64(vb)
    else:
        k_raw = v_raw = np.zeros((0, d))
    if mid_idx.size:
        ck, cv, ks, kz, vs, vz = int2.read(np.asarray(bt_q_row)[mid_idx // PAGE], mid_idx % PAGE, h)
        k_rot, v_rot = dequantize(ck, ks, kz), dequantize(cv, vs, vz)
    else:
        k_rot = v_rot = np.zeros((0, d))
    return raw_idx, k_raw, v_raw, mid_idx, k_rot, v_rot


def extend_attention(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, pool, bf16: Bf16Pool, cu, cache_lens,
                     bt_q, bt_h, r_k: np.ndarray, r_v: np.ndarray, S: int, W: int,
                     scale: float | None = None, rows=None) -> np.ndarray:
    """Chunked-prefill ("extend") attention over the mixed paged cache, fp64.

    [TS] 2.2.B "Kernel Integration" (paged attention with prefix caching) and
    [TS] 3: a request whose prefix is already cached prefills only its new
    tokens, which attend the cached prefix through its pages.  Reading: the
    new rows of sequence b (rows cu[b] .. cu[b+1] - 1 of q, k_new, v_new) sit
    at positions P + i, P = cache_lens[b]; row i attends the cached prefix
    [0, P), whose regions are those of a length-P cache (sink and recent raw
    from BF16 pages, the middle decoded from the quantized pages and rotated
    back), and the new rows 0..i (causal), raw.  ``pool`` is an Int2Pool or an
    Int4Pool.  q float64 [T, H_q, d]; k_new, v_new float64 [T, H_kv, d];
    returns float64 [T, H_q, d].  ``rows``: if given, only these global rows
    are computed (the others stay zero).
    """
    T, hq, d = q.shape
    hkv = k_new.shape[1]
    G = hq // hkv
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((T, hq, d))
    cu = np.asarray(cu, np.int64)
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        P = int(cache_lens[b])
        for h in range(hkv):
            if P > 0:
                _, k_raw, v_raw, _, k_rot, v_rot = sequence_kv(pool, bf16, bt_q[b], bt_h[b], P, S, W, h)
                kc = np.concatenate([k_raw, k_rot @ np.asarray(r_k[h], np.float64).T])
                vc = np.concatenate([v_raw, v_rot @ np.asarray(r_v[h], np.float64).T])
            else:
                kc = vc = np.zeros((0, d))
            for i in range(r1 - r0):
                if rows is not None and r0 + i not in rows:
                    continue
                k = np.concatenate([kc, np.asarray(k_new[r0:r0 + i + 1, h], np.float64)])
                v = np.concatenate([vc, np.asarray(v_new[r0:r0 + i + 1, h], np.float64)])
                out[r0 + i, h * G:(h + 1) * G] = softmax_attention(np.asarray(q[r0 + i, h * G:(h + 1) * G], np.float64),
                                                                   k, v, sc)
    return out


def decode_attention(q: np.ndarray, int2: Int2Pool, bf16: Bf16Pool, seq_lens, bt_q, bt_h,
                     r_k: np.ndarray, r_v: np.ndarray, S: int, W: int, scale: float | None = None) -> np.ndarray:
    """Output [B, H_q, d] float64: plain attention over the decoded cache with
    middle keys/values rotated back (kh R_K^T, vh R_V^T)."""
    B, hq, d = q.shape
    hkv = int2.hkv
    G = hq // hkv
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((B, hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for h in range(hkv):
            raw_idx, k_raw, v_raw, mid_idx, k_rot, v_rot = sequence_kv(int2, bf16, bt_q[b], bt_h[b], L, S, W, h)
            k = np.concatenate([k_raw, k_rot @ np.asarray(r_k[h], np.float64).T])
            v = np.concatenate([v_raw, v_rot @ np.asarray(r_v[h], np.float64).T])
            out[b, h * G:(h + 1) * G] = softmax_attention(np.asarray(q[b, h * G:(h + 1) * G], np.float64), k, v, sc)
    return out


def partial_state(qraw: np.ndarray, qrot: np.ndarray, k_raw, v_raw, k_rot, v_rot, scale: float):
    """(m, l, acc_raw, acc_rot) of one chunk: running max, sum of exp, and the
    unnormalised value sums in the raw and the rotated basis."""
    G = qraw.shape[0]
    d = qraw.shape[1]
    s = np.concatenate([(qraw @ k_raw.T) * scale, (qrot @ k_rot.T) * scale], axis=1)
    if s.shape[1] == 0:
        return np.full(G, -np.inf), np.zeros(G), np.zeros((G, d)), np.zeros((G, d))
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    nr = k_raw.shape[0]
    return m, p.sum(axis=1), p[:, :nr] @ v_raw, p[:, nr:] @ v_rot


def merge_states(states, r_v_h: np.ndarray) -> np.ndarray:
    """Log-sum-exp merge of chunk states, then the output rotation by R_V^T."""
    ms = np.stack([s[0] for s in states])            # [C, G]
    M = ms.max(axis=0)
    wgt = np.where(np.isfinite(ms), np.exp(ms - M[None, :]), 0.0)
    l = sum(w * s[1] for w, s in zip(wgt, states))
    raw = sum(w[:, None] * s[2] for w, s in zip(wgt, states))
    rot = sum(w[:, None] * s[3] for w, s in zip(wgt, states))
    return (raw + rot @ np.asarray(r_v_h, np.float64).T) / l[:, None]


def decode_attention_rotated(q: np.ndarray, int2: Int2Pool, bf16: Bf16Pool, seq_lens, bt_q, bt_h,
                             r_k, r_v, S: int, W: int, scale: float | None = None,
                             chunk_tokens: int | None = None) -> np.ndarray:
    """The rotated-space route: q~ = q R_K for middle logits, two value sums,
    chunks of ``chunk_tokens`` positions merged by log-sum-exp, R_V^T applied
    once after the merge."""
    B, hq, d = q.shape
    hkv = int2.hkv
    G = hq // hkv
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((B, hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        ct = L if chunk_tokens is None else chunk_tokens
        for h in range(hkv):
            raw_idx, k_raw, v_raw, mid_idx, k_rot, v_rot = sequence_kv(int2, bf16, bt_q[b], bt_h[b], L, S, W, h)
            qh = np.asarray(q[b, h * G:(h + 1) * G], np.float64)
            qt = qh @ np.asarray(r_k[h], np.float64)
            states = []
            for t0 in range(0, L, ct):
                rs = (raw_idx >= t0) & (raw_idx < t0 + ct)
                ms = (mid_idx >= t0) & (mid_idx < t0 + ct)
                states.append(partial_state(qh, qt, k_raw[rs], v_raw[rs], k_rot[ms], v_rot[ms], sc))
            out[b, h * G:(h + 1) * G] = merge_states(states, r_v[h])
    return out
