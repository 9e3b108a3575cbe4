"""Pins of oracle.rotation against textbook values, closed forms and brute force.

[TS] 2.1 (targets Q^T Q and V^T S^T S V), 2.2.A steps 1-4 (eigenbases,
R = U H_Had P_br, per-layer clip).
"""
import os

import numpy as np
import pytest

from oracle import rotation as rot
from int2_rotated_kv_oscar_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name, key):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            if line.startswith(key + " "):
                rows.append([int(v) for v in line.split()[1:]])
    return rows


def test_hadamard_textbook_and_orthogonality():
    # O2: textbook H_4 and H H^T = d I exactly in integers
    assert np.array_equal(rot.hadamard(4), np.array(_golden_rows("hadamard_bitrev.txt", "H4")))
    for d in (1, 2, 4, 8, 16, 32, 64, 128):
        h = rot.hadamard(d)
        assert h.dtype.kind == "i"
        assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
        assert np.array_equal(h, h.T)


def test_bit_reversal_textbook_and_involution():
    # O3
    assert [rot.bit_reverse(j, 3) for j in range(8)] == _golden_rows("hadamard_bitrev.txt", "BR8")[0]
    assert [rot.bit_reverse(j, 4) for j in range(16)] == _golden_rows("hadamard_bitrev.txt", "BR16")[0]
    for d in (2, 4, 64, 128):
        p = rot.bitrev_perm(d)
        assert np.array_equal(p @ p, np.eye(d, dtype=np.int64))
        assert np.array_equal(p, p.T)
        bits = d.bit_length() - 1
        assert all(rot.bit_reverse(rot.bit_reverse(j, bits), bits) == j for j in range(d))
        # P applied to a row vector: (x P)[c] = x[br(c)]
        x = np.arange(d, dtype=np.int64)
        assert list(x @ p) == [rot.bit_reverse(c, bits) for c in range(d)]


def test_eig_recovers_planted_spectrum():
    # O4/O5 without LAPACK deciding the outcome: plant C = U0 diag(l0) U0^T with known
    # distinct eigenvalues and check they come back, descending, with columns
    # equal to the planted ones up to the documented sign rule.
    rng = np.random.default_rng(7)
    d = 64
    u0, _ = np.linalg.qr(rng.standard_normal((d, d)))
    l0 = np.linspace(10.0, 0.5, d)
    c = (u0 * l0) @ u0.T
    w, u = rot.eig_desc(c)
    assert np.allclose(w, l0, rtol=0, atol=1e-12 * l0[0])
    for j in range(d):
        col = u0[:, j] * np.sign(u0[np.argmax(np.abs(u0[:, j])), j])
        assert np.allclose(u[:, j], col, atol=1e-10)
    assert np.all(np.diff(w) <= 0)


def test_eig_invariants_on_calibration_targets():
    # O4: U^T C U = diag(lambda), U orthogonal, lambda descending, sign rule
    w = synth.WORKLOADS["tiny"]
    cal = synth.calibration_set(w, n_rows=256)
    cq, cs = rot.calibration_targets(cal.q.astype(np.float64), cal.k.astype(np.float64),
                                     cal.v.astype(np.float64), w.group_q)
    for c in (cq[0], cs[0]):
        lam, u = rot.eig_desc(c)
        assert np.abs(u.T @ c @ u - np.diag(lam)).max() <= 1e-10 * np.abs(c).max()
        assert np.abs(u.T @ u - np.eye(c.shape[0])).max() <= 1e-12
        assert np.all(np.diff(lam) <= 1e-14 * lam[0])
        assert abs(lam.sum() - np.trace(c)) <= 1e-10 * abs(np.trace(c))
        for j in range(u.shape[1]):
            assert u[np.argmax(np.abs(u[:, j])), j] > 0


def test_calibration_targets_brute_force():
    # C_Q and C_S against scalar loops on a tiny input, including the causal
    # softmax written out element by element.
    rng = np.random.default_rng(3)
    N, G, hkv, d = 6, 2, 2, 4
    q = rng.standard_normal((N, G * hkv, d))
    k = rng.standard_normal((N, hkv, d))
    v = rng.standard_normal((N, hkv, d))
    cq, cs = rot.calibration_targets(q, k, v, G)
    for h in range(hkv):
        bq = np.zeros((d, d))
        bs = np.zeros((d, d))
        for i in range(h * G, h * G + G):
            for n in range(N):
                for a in range(d):
                    for b in range(d):
                        bq[a, b] += q[n, i, a] * q[n, i, b]
            o = np.zeros((N, d))
            for r in range(N):
                sc = [sum(q[r, i, a] * k[j, h, a] for a in range(d)) / np.sqrt(d) for j in range(r + 1)]
                mx = max(sc)
                e = [np.exp(s - mx) for s in sc]
                tot = sum(e)
                for j in range(r + 1):
                    o[r] += e[j] / tot * v[j, h]
            for n in range(N):
                for a in range(d):
                    for b in range(d):
                        bs[a, b] += o[n, a] * o[n, b]
        np.testing.assert_allclose(cq[h], bq / (N * G), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(cs[h], bs / (N * G), rtol=1e-12, atol=1e-13)


def test_value_target_is_VtStSV_over_N():
    # [TS] 2.1: for one query head the value target equals V^T S^T S V / N with
    # S the explicit (causal) score matrix.
    rng = np.random.default_rng(11)
    N, d = 9, 8
    q = rng.standard_normal((N, 1, d))
    k = rng.standard_normal((N, 1, d))
    v = rng.standard_normal((N, 1, d))
    _, cs = rot.calibration_targets(q, k, v, 1)
    s = np.zeros((N, N))
    for r in range(N):
        l = q[r, 0] @ k[: r + 1, 0].T / np.sqrt(d)
        e = np.exp(l - l.max())
        s[r, : r + 1] = e / e.sum()
    V = v[:, 0]
    np.testing.assert_allclose(cs[0], V.T @ s.T @ s @ V / N, rtol=1e-12, atol=1e-14)


def test_supplied_attention_output_is_used():
    rng = np.random.default_rng(5)
    N, d = 7, 4
    q = rng.standard_normal((N, 2, d)); k = rng.standard_normal((N, 1, d)); v = rng.standard_normal((N, 1, d))
    o = rng.standard_normal((N, 2, d))
    _, cs = rot.calibration_targets(q, k, v, 2, o)
    np.testing.assert_allclose(cs[0], (o[:, 0].T @ o[:, 0] + o[:, 1].T @ o[:, 1]) / (2 * N), rtol=1e-13)


@pytest.mark.parametrize("name", ["tiny"])
def test_rotation_orthogonal_and_equalizes_importance(name):
    # O1: R^T R = I;  O6: diag(R^T C R) = tr(C)/d (the Hadamard "equalizes the
    # importance metric across channels", [TS] 2.2.A step 3) for R_K with C_Q
    # and R_V with C_S.
    w = synth.WORKLOADS[name]
    cal = synth.calibration_set(w, n_rows=512)
    out = rot.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    d = w.d
    for h in range(w.n_kv_heads):
        for r, c in ((out["r_k"][h], out["c_q"][h]), (out["r_v"][h], out["c_s"][h])):
            assert np.abs(r.T @ r - np.eye(d)).max() <= 1e-10
            dg = np.diag(r.T @ c @ r)
            np.testing.assert_allclose(dg, np.full(d, np.trace(c) / d), rtol=1e-10)


def test_composite_rotation_structure():
    # R = U H P: with U = I, R[k, c] = H[k, br(c)] / sqrt(d)
    d = 16
    r = rot.composite_rotation(np.eye(d))
    h = rot.hadamard(d)
    for k in range(d):
        for c in range(d):
            assert r[k, c] == h[k, rot.bit_reverse(c, 4)] / np.sqrt(d)


def test_linear_quantile_brute_force():
    # O7: hand values and numpy's linear percentile (an independent routine)
    vals = np.arange(1001, dtype=np.float64)[::-1]
    assert rot.linear_quantile(vals, 0.999) == 999.0
    assert rot.linear_quantile(vals, 0.9995) == 999.5
    assert rot.linear_quantile([3.0, 1.0, 2.0], 1.0) == 3.0
    assert rot.linear_quantile([5.0], 0.999) == 5.0
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10007)
    for q in (0.5, 0.9, 0.999, 1.0):
        assert rot.linear_quantile(x, q) == pytest.approx(np.percentile(x, 100 * q, method="linear"), rel=1e-15)


def test_clip_threshold_pools_heads_and_channels():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 3, 8))
    r = np.stack([np.linalg.qr(rng.standard_normal((8, 8)))[0] for _ in range(3)])
    pooled = []
    for n in range(50):
        for h in range(3):
            for c in range(8):
                pooled.append(abs(sum(x[n, h, k] * r[h, k, c] for k in range(8))))
    pooled.sort()
    rr = 0.9 * (len(pooled) - 1)
    lo = int(rr)
    expect = pooled[lo] + (rr - lo) * (pooled[lo + 1] - pooled[lo])
    assert rot.clip_threshold(x, r, 0.9) == pytest.approx(expect, rel=1e-12)


def test_fixed_rotation_hadamard_only_pins():
    # [TS] 1 / 4: the Hadamard-only baseline is the composite rotation without
    # the eigenbasis.  d = 4 from the textbook H_4 with the columns taken in
    # 2-bit reversed order (0, 2, 1, 3), halved.
    h4 = np.array(_golden_rows("hadamard_bitrev.txt", "H4"), dtype=np.float64)
    kc = np.random.default_rng(3).standard_normal((9, 2, 4))
    r = rot.fixed_rotation(rot.HADAMARD_ONLY, kc, kc)
    assert np.array_equal(r["r_k"][0], h4[:, [0, 2, 1, 3]] / 2.0)
    assert np.array_equal(r["r_k"][1], r["r_k"][0]) and np.array_equal(r["r_v"], r["r_k"])
    for d in (64, 128):
        x = np.zeros((d, 1, d))
        a = 3.0
        for j in range(d):
            x[j, 0, j] = a  # one spike per row: the rotation spreads it evenly
        r = rot.fixed_rotation(rot.HADAMARD_ONLY, x, x)
        rk = r["r_k"][0]
        assert np.array_equal(np.abs(rk), np.full((d, d), 1.0 / np.sqrt(d)))
        assert np.abs(rk.T @ rk - np.eye(d)).max() <= 1e-14
        np.testing.assert_allclose(r["tau_k"], a / np.sqrt(d), rtol=1e-14)


def test_fixed_rotation_identity_pins():
    # naive INT2: no rotation; tau is the plain order statistic of |x|
    rng = np.random.default_rng(4)
    kc = rng.standard_normal((50, 3, 64))
    vc = rng.standard_normal((50, 3, 64)) * 2.0
    r = rot.fixed_rotation(rot.IDENTITY, kc, vc, clip_quantile=0.9)
    assert np.array_equal(r["r_k"], np.broadcast_to(np.eye(64), (3, 64, 64)))
    for key, x in (("tau_k", kc), ("tau_v", vc)):
        a = sorted(abs(float(t)) for t in x.ravel())
        rr = 0.9 * (len(a) - 1)
        lo = int(rr)
        assert r[key] == pytest.approx(a[lo] + (rr - lo) * (a[lo + 1] - a[lo]), rel=1e-15)
    with pytest.raises(ValueError):
        rot.fixed_rotation(7, kc, vc)
