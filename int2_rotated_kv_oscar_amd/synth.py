"""Seeded synthetic inputs shared by the GPU path, the tests and the bench.

This module only draws and lays out inputs; it contains none of the method's
arithmetic (no rotation, clipping, quantization or attention).  Every stream
is ``numpy.random.Generator(PCG64(SeedSequence([260517757, cfg_id, role])))``
so each (workload, role) pair is reproducible on any machine.

Roles: 1 outlier-channel choice, 2 calibration Q/K/V rows, 3 query mixing
matrices, 4 decode-history K/V rows, 5 decode queries, 6 context lengths,
7 physical-page permutation, 8 prefill-chunk rows.

The workloads stand in for the activations of the models and benchmarks the
OSCAR pages evaluate on (Qwen3-8B/32B-shaped layers, reasoning traces up to
32k tokens, RULER-style 128k contexts, 28 concurrent long requests): keys and
values are Gaussian (Student-t for the frontier-scale layer) with a few
channels scaled up to reproduce channel-wise outliers, and queries are a
Gaussian mixed by a matrix with singular values 1/i.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

ROOT_SEED = 260517757
PAGE = 16

# ---------------------------------------------------------------- bf16 ----


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-half-to-even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 draws -> float32 (RNE) -> bfloat16 (RNE) bits."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


# ------------------------------------------------------------- configs ----


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d: int
    n_sink: int
    n_recent: int
    calib_rows: int
    ctx: Tuple[str, int, int]          # ("fixed", L, L) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    k_noise: str = "normal"            # "normal" | "t3"
    q_scale: float = 1.0               # singular values q_scale / i
    shared_prefix: int = 0             # tokens shared (aliased pages) by all sequences
    k_outliers: Tuple[int, float] = (3, 15.0)
    v_outliers: Tuple[int, float] = (2, 8.0)

    @property
    def group_q(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 4, 1, 64, 4, 32, 2048, ("fixed", 512, 512)),
    "qwen3-8b-b1-32k": Workload("qwen3-8b-b1-32k", 2, 1, 32, 8, 128, 4, 128, 8192,
                                ("fixed", 32768, 32768)),
    "qwen3-8b-b28-ragged": Workload("qwen3-8b-b28-ragged", 3, 28, 32, 8, 128, 4, 128, 8192,
                                    ("uniform", 4096, 32768), shared_prefix=1024),
    "qwen3-32b-b1-128k": Workload("qwen3-32b-b1-128k", 4, 1, 64, 8, 128, 4, 128, 8192,
                                  ("fixed", 131072, 131072)),
    "qwen3-32b-b4-128k": Workload("qwen3-32b-b4-128k", 4, 4, 64, 8, 128, 4, 128, 8192,
                                  ("fixed", 131072, 131072)),
    "gqa96-b64-ragged": Workload("gqa96-b64-ragged", 5, 64, 96, 8, 128, 4, 128, 8192,
                                 ("loguniform", 4096, 65536), k_noise="t3"),
}


def rng_for(cfg_id: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg_id, role])))


# ------------------------------------------------------------ draws -------


def outlier_channels(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Per KV head, distinct outlier channels for K and for V (role 1)."""
    rng = rng_for(w.cfg_id, 1)
    kc = np.stack([rng.choice(w.d, size=w.k_outliers[0], replace=False) for _ in range(w.n_kv_heads)])
    vc = np.stack([rng.choice(w.d, size=w.v_outliers[0], replace=False) for _ in range(w.n_kv_heads)])
    return kc, vc


def _haar(rng: np.random.Generator, d: int) -> np.ndarray:
    z = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(z)
    return qm * np.sign(np.diag(rm))[None, :]


def query_mixers(w: Workload, q_scale: Optional[float] = None) -> np.ndarray:
    """A_i = U_i diag(c / j) W_i^T per query head (role 3); [H_q, d, d]."""
    c = w.q_scale if q_scale is None else q_scale
    rng = rng_for(w.cfg_id, 3)
    sv = c / np.arange(1, w.d + 1, dtype=np.float64)
    out = np.empty((w.n_q_heads, w.d, w.d))
    for i in range(w.n_q_heads):
        u = _haar(rng, w.d)
        v = _haar(rng, w.d)
        out[i] = (u * sv[None, :]) @ v.T
    return out


def _kv_draw(rng: np.random.Generator, n: int, w: Workload, chans: np.ndarray, scale: float,
             noise: str) -> np.ndarray:
    if noise == "t3":
        x = rng.standard_t(3.0, size=(n, w.n_kv_heads, w.d))
    else:
        x = rng.standard_normal((n, w.n_kv_heads, w.d))
    for h in range(w.n_kv_heads):
        x[:, h, chans[h]] *= scale
    return x


def kv_rows(rng: np.random.Generator, n: int, w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """n rows of K and V, bf16 bits [n, H_kv, d] each."""
    kc, vc = outlier_channels(w)
    k = _kv_draw(rng, n, w, kc, w.k_outliers[1], w.k_noise)
    v = _kv_draw(rng, n, w, vc, w.v_outliers[1], "normal")
    return to_bf16_bits(k), to_bf16_bits(v)


def q_rows(rng: np.random.Generator, n: int, w: Workload, mixers: np.ndarray) -> np.ndarray:
    """n query rows per query head, bf16 bits [n, H_q, d]."""
    z = rng.standard_normal((n, w.n_q_heads, w.d))
    q = np.einsum("nik,ikc->nic", z, mixers)
    return to_bf16_bits(q)


@dataclasses.dataclass
class CalibSet:
    q: np.ndarray  # float32 (bf16-exact) [N, H_q, d]
    k: np.ndarray  # float32 [N, H_kv, d]
    v: np.ndarray  # float32 [N, H_kv, d]


def calibration_set(w: Workload, n_rows: Optional[int] = None,
                    q_scale: Optional[float] = None) -> CalibSet:
    n = w.calib_rows if n_rows is None else n_rows
    rng = rng_for(w.cfg_id, 2)
    k, v = kv_rows(rng, n, w)
    q = q_rows(rng, n, w, query_mixers(w, q_scale))
    return CalibSet(bf16_bits_to_f32(q), bf16_bits_to_f32(k), bf16_bits_to_f32(v))


def context_lengths(w: Workload) -> np.ndarray:
    kind, lo, hi = w.ctx
    if kind == "fixed":
        return np.full(w.batch, lo, dtype=np.int32)
    rng = rng_for(w.cfg_id, 6)
    if kind == "uniform":
        return rng.integers(lo, hi, size=w.batch, endpoint=True).astype(np.int32)
    u = rng.uniform(math.log(lo), math.log(hi), size=w.batch)
    return np.round(np.exp(u)).astype(np.int32)


# ------------------------------------------------------ cache layout ------


def regions(L: int, S: int, W: int) -> Tuple[Tuple[int, int], Tuple[int, int], Tuple[int, int]]:
    """(sink, middle, recent) half-open token ranges of a length-L sequence."""
    sink = (0, min(S, L))
    rec = (max(S, L - W), L)
    mid = (S, L - W) if L - W > S else (S, S)
    return sink, mid, rec


@dataclasses.dataclass
class DecodeInputs:
    """A decode batch over a paged cache: raw rows, tables and queries.

    ``row_of[b][t]`` is the index into ``k_rows``/``v_rows`` of token t of
    sequence b (shared-prefix tokens map to the same rows).  Physical pages are
    a seeded permutation of the pool (role 7), shared prefix pages are named by
    every sequence's table.
    """
    w: Workload
    seq_lens: np.ndarray          # int32 [B]
    k_rows: np.ndarray            # uint16 bf16 [R, H_kv, d]
    v_rows: np.ndarray
    row_of: List[np.ndarray]      # per sequence, int64 [L_b]
    q: np.ndarray                 # uint16 bf16 [B, H_q, d]
    bt_q: np.ndarray              # int32 [B, max_pages]
    bt_h: np.ndarray              # int32 [B, max_pages]
    n_int2_pages: int
    n_bf16_pages: int
    max_pages: int

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0


def _page_flags(L: int, S: int, W: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per logical page: does it hold a middle token / a sink or recent token."""
    n_pages = (L + PAGE - 1) // PAGE
    sink, mid, rec = regions(L, S, W)
    a = np.arange(n_pages, dtype=np.int64) * PAGE
    b = np.minimum(a + PAGE, L)

    def overlaps(r):
        return np.maximum(a, r[0]) < np.minimum(b, r[1])
    return overlaps(mid), overlaps(sink) | overlaps(rec)


def _history_rng(cfg_id: int, part: int) -> np.random.Generator:
    """K/V history stream (role 4): part 0 the shared prefix, part b + 1 the
    own rows of sequence b, so any subset of sequences can be drawn alone."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg_id, 4, part])))


def decode_inputs(w: Workload, seq_lens: Optional[np.ndarray] = None, q_scale: Optional[float] = None,
                  shuffle: bool = True, spare_pages: int = 0,
                  draw_seqs: Optional[Sequence[int]] = None) -> DecodeInputs:
    """Raw K/V history, block tables and one decode query per sequence.

    ``draw_seqs`` limits the drawn history to those sequences (and the shared
    prefix); the own rows of the other sequences are left zero.  Drawn values
    do not depend on the subset."""
    lens = context_lengths(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    B = len(lens)
    S, W = w.n_sink, w.n_recent
    pre = w.shared_prefix
    if pre:
        assert pre % PAGE == 0 and all(L >= pre + W + PAGE for L in lens)
    n_rows = pre + int(sum(int(L) - pre for L in lens))
    k_rows = np.zeros((n_rows, w.n_kv_heads, w.d), np.uint16)
    v_rows = np.zeros((n_rows, w.n_kv_heads, w.d), np.uint16)
    if pre:
        k_rows[:pre], v_rows[:pre] = kv_rows(_history_rng(w.cfg_id, 0), pre, w)
    drawn = set(range(B)) if draw_seqs is None else {int(b) for b in draw_seqs}
    row_of = []
    nxt = pre
    for b, L in enumerate(lens):
        n_own = int(L) - pre
        own = np.arange(nxt, nxt + n_own, dtype=np.int64)
        row_of.append(np.concatenate([np.arange(pre, dtype=np.int64), own]))
        if b in drawn and n_own > 0:
            k_rows[nxt:nxt + n_own], v_rows[nxt:nxt + n_own] = kv_rows(_history_rng(w.cfg_id, b + 1), n_own, w)
        nxt += n_own
    max_pages = max(1, (int(lens.max()) + PAGE - 1) // PAGE) if B else 1
    pre_pages = pre // PAGE
    # logical -> "virtual" page ids (shared prefix pages once), then a seeded
    # permutation of each pool
    bt_q = np.full((B, max_pages), -1, np.int64)
    bt_h = np.full((B, max_pages), -1, np.int64)
    counters = [0, 0]
    shared = [None, None]
    for b, L in enumerate(lens):
        flags = _page_flags(int(L), S, W)
        for which, (tab, fl) in enumerate(((bt_q, flags[0]), (bt_h, flags[1]))):
            pages = np.nonzero(fl)[0]
            own = pages[pages >= pre_pages] if pre_pages else pages
            if pre_pages:
                pp = pages[pages < pre_pages]
                if shared[which] is None:
                    shared[which] = {int(p): counters[which] + i for i, p in enumerate(pp)}
                    counters[which] += len(pp)
                tab[b, pp] = [shared[which][int(p)] for p in pp]
            tab[b, own] = counters[which] + np.arange(len(own))
            counters[which] += len(own)
    nq = counters[0] + spare_pages
    nh = counters[1] + spare_pages
    prng = rng_for(w.cfg_id, 7)
    perm_q = prng.permutation(nq) if shuffle else np.arange(nq)
    perm_h = prng.permutation(nh) if shuffle else np.arange(nh)
    bt_q = np.where(bt_q >= 0, perm_q[np.maximum(bt_q, 0)] if nq else -1, -1).astype(np.int32)
    bt_h = np.where(bt_h >= 0, perm_h[np.maximum(bt_h, 0)] if nh else -1, -1).astype(np.int32)
    q = q_rows(rng_for(w.cfg_id, 5), B, w, query_mixers(w, q_scale))
    return DecodeInputs(w, lens, k_rows, v_rows, row_of, q, bt_q, bt_h, max(nq, 1), max(nh, 1), max_pages)


def middle_rows(inp: DecodeInputs) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(row_seq, row_pos, row index) of every middle token, each physical slot once."""
    S, W = inp.w.n_sink, inp.w.n_recent
    pre = inp.w.shared_prefix
    seqs, poss, rows = [], [], []
    for b, L in enumerate(inp.seq_lens):
        _, mid, _ = regions(int(L), S, W)
        lo = mid[0] if (b == 0 or pre == 0) else max(mid[0], pre)
        t = np.arange(lo, mid[1], dtype=np.int64)
        seqs.append(np.full(len(t), b, np.int32)); poss.append(t.astype(np.int32)); rows.append(inp.row_of[b][t])
    return np.concatenate(seqs), np.concatenate(poss), np.concatenate(rows)


def bf16_rows(inp: DecodeInputs) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(row_seq, row_pos, row index) of every sink/recent token, each physical slot once."""
    S, W = inp.w.n_sink, inp.w.n_recent
    pre = inp.w.shared_prefix
    seqs, poss, rows = [], [], []
    for b, L in enumerate(inp.seq_lens):
        sink, _, rec = regions(int(L), S, W)
        t = np.concatenate([np.arange(*sink), np.arange(*rec)]).astype(np.int64)
        if b > 0 and pre:
            t = t[t >= pre]
        seqs.append(np.full(len(t), b, np.int32)); poss.append(t.astype(np.int32)); rows.append(inp.row_of[b][t])
    return np.concatenate(seqs), np.concatenate(poss), np.concatenate(rows)


def prefill_rows(w: Workload, n_seqs: int, chunk: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """A prefill chunk of ``chunk`` consecutive positions per sequence (role 8).

    Returns (k bits, v bits [n, H_kv, d], row_seq, row_pos) with rows ordered by
    sequence then position, i.e. whole pages back to back.
    """
    rng = rng_for(w.cfg_id, 8)
    k, v = kv_rows(rng, n_seqs * chunk, w)
    row_seq = np.repeat(np.arange(n_seqs, dtype=np.int32), chunk)
    row_pos = np.tile(np.arange(chunk, dtype=np.int32), n_seqs)
    return k, v, row_seq, row_pos
