"""Offline calibration: targets, eigenbases and the composite rotation (fp64).

Follows [TS] section 2.1 (the key target is the query covariance, the value
target is V^T S^T S V) and section 2.2.A (steps 1-4: empirical targets, eigen-
decomposition, R = U . H_Had . P_br, per-layer clip thresholds from rotated
calibration activations).  Readings taken where the pages are silent are
listed in each docstring.
"""
from __future__ import annotations

import numpy as np


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d with integer entries (H_1 = [1])."""
    assert d >= 1 and d & (d - 1) == 0
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def bit_reverse(j: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (j & 1)
        j >>= 1
    return r


def bitrev_perm(d: int) -> np.ndarray:
    """P_br with P[r, c] = 1 iff r is the log2(d)-bit reversal of c ([TS] 2.2.A step 3)."""
    bits = d.bit_length() - 1
    p = np.zeros((d, d), dtype=np.int64)
    for c in range(d):
        p[bit_reverse(c, bits), c] = 1
    return p


def causal_attention_out(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int = 1024) -> np.ndarray:
    """O = S V with S = row-softmax(q k^T / sqrt(d) + causal mask); q, k, v [N, d].

    Reading: calibration row r attends to rows 0..r (the scores a causal
    decoder produces on the calibration sequence).
    """
    n, d = q.shape
    out = np.empty((n, d))
    scale = 1.0 / np.sqrt(d)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        s = (q[r0:r1] @ k[:r1].T) * scale
        mask = np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]
        s[mask] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r1] = p @ v[:r1]
    return out


def calibration_targets(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, group_q: int,
                        oc: np.ndarray | None = None):
    """C_Q(h) and C_S(h) per KV head ([TS] 2.1; 2.2.A step 1).

    qc [N, H_q, d], kc/vc [N, H_kv, d] (float64).  C_Q = (1/N) sum_n q_n^T q_n
    with q_n a row vector (the garbled sum on the summary page read as the
    outer product, matching "Q^T Q"), pooled over the G query heads of the
    group; C_S = V^T S^T S V / N = O^T O / N with O = S V, pooled likewise.
    Both are normalised by N G.
    """
    n, hq, d = qc.shape
    hkv = kc.shape[1]
    cq = np.zeros((hkv, d, d))
    cs = np.zeros((hkv, d, d))
    for h in range(hkv):
        for i in range(h * group_q, (h + 1) * group_q):
            qi = qc[:, i, :]
            cq[h] += qi.T @ qi
            o = oc[:, i, :] if oc is not None else causal_attention_out(qi, kc[:, h, :], vc[:, h, :])
            cs[h] += o.T @ o
    cq /= n * group_q
    cs /= n * group_q
    return cq, cs


def eig_desc(c: np.ndarray):
    """Eigenvalues (descending) and eigenvectors of a symmetric matrix ([TS] 2.2.A step 2).

    Reading: columns ordered by descending eigenvalue, each negated if needed
    so that its largest-magnitude entry is positive (lowest index on ties).
    """
    w, u = np.linalg.eigh(c)
    order = np.argsort(-w, kind="stable")
    w, u = w[order], u[:, order].copy()
    for j in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, j])))
        if u[i, j] < 0:
            u[:, j] = -u[:, j]
    return w, u


def composite_rotation(u: np.ndarray) -> np.ndarray:
    """R = U . (H_d / sqrt(d)) . P_br ([TS] 2.2.A step 3), acting as y = x . R."""
    d = u.shape[0]
    return u @ (hadamard(d) / np.sqrt(d)) @ bitrev_perm(d)


def linear_quantile(values: np.ndarray, q: float) -> float:
    """Quantile with linear interpolation between order statistics.

    Sorted ascending a[0..M-1], rr = q (M - 1), result
    a[floor(rr)] + (rr - floor(rr)) (a[floor(rr)+1] - a[floor(rr)]).
    """
    a = np.sort(np.asarray(values, dtype=np.float64).ravel())
    m = a.size
    rr = q * (m - 1)
    lo = int(np.floor(rr))
    hi = min(lo + 1, m - 1)
    return float(a[lo] + (rr - lo) * (a[hi] - a[lo]))


def clip_threshold(x: np.ndarray, r: np.ndarray, q: float) -> float:
    """Per-layer clip ([TS] 2.2.A step 4): quantile q of |x_h . R(h)| pooled
    over rows, heads and channels (one threshold per layer, symmetric)."""
    ys = [np.abs(x[:, h, :] @ r[h]) for h in range(x.shape[1])]
    return linear_quantile(np.concatenate([y.ravel() for y in ys]), q)


def build_rotation(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, group_q: int,
                   clip_quantile: float = 0.999, oc: np.ndarray | None = None) -> dict:
    """Everything the offline phase produces for one layer ([TS] 2.2.A)."""
    qc, kc, vc = (np.asarray(a, dtype=np.float64) for a in (qc, kc, vc))
    if oc is not None:
        oc = np.asarray(oc, dtype=np.float64)
    cq, cs = calibration_targets(qc, kc, vc, group_q, oc)
    hkv, d = kc.shape[1], kc.shape[2]
    rk = np.empty((hkv, d, d))
    rv = np.empty((hkv, d, d))
    ek = np.empty((hkv, d))
    ev = np.empty((hkv, d))
    for h in range(hkv):
        ek[h], uq = eig_desc(cq[h])
        ev[h], us = eig_desc(cs[h])
        rk[h] = composite_rotation(uq)
        rv[h] = composite_rotation(us)
    return dict(r_k=rk, r_v=rv, eig_k=ek, eig_v=ev, c_q=cq, c_s=cs,
                tau_k=clip_threshold(kc, rk, clip_quantile),
                tau_v=clip_threshold(vc, rv, clip_quantile))


HADAMARD_ONLY = 1
IDENTITY = 2


def fixed_rotation(variant: int, kc: np.ndarray, vc: np.ndarray, clip_quantile: float = 0.999) -> dict:
    """The pages' comparison rotations ([TS] 1: Hadamard transforms, the
    data-oblivious rotations; [TS] 4 "Accuracy Preservation": naive INT2 and
    Hadamard-only baselines), for every KV head and both K and V:
    Hadamard-only R = (H_d / sqrt(d)) . P_br, the composite rotation with the
    eigenbasis left out; naive R = I.  Clip thresholds as in step 4.
    """
    kc, vc = (np.asarray(a, dtype=np.float64) for a in (kc, vc))
    hkv, d = kc.shape[1], kc.shape[2]
    if variant == HADAMARD_ONLY:
        r = (hadamard(d) / np.sqrt(d)) @ bitrev_perm(d)
    elif variant == IDENTITY:
        r = np.eye(d)
    else:
        raise ValueError(f"unknown rotation variant {variant}")
    rr = np.broadcast_to(r, (hkv, d, d)).copy()
    return dict(r_k=rr, r_v=rr.copy(), tau_k=clip_threshold(kc, rr, clip_quantile),
                tau_v=clip_threshold(vc, rr, clip_quantile))
