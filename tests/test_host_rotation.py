"""oscar_build_rotation (host C++, float64) against the oracle and the
invariants of the method ([TS] 2.1, 2.2.A)."""
import numpy as np
import pytest

from int2_rotated_kv_oscar_amd import lib, synth
from oracle import rotation as orot


@pytest.mark.parametrize("name,n_rows", [("tiny", 2048), ("qwen3-8b-b1-32k", 384)])
def test_matches_oracle(name, n_rows):
    w = synth.WORKLOADS[name]
    cal = synth.calibration_set(w, n_rows=n_rows)
    got = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    ref = orot.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    d = w.d
    for key in ("eig_k", "eig_v"):
        np.testing.assert_allclose(got[key], ref[key], rtol=0, atol=1e-10 * np.abs(ref[key]).max())
    for h in range(w.n_kv_heads):
        for rk, c, lam in ((got["r_k"][h], ref["c_q"][h], ref["eig_k"][h]), (got["r_v"][h], ref["c_s"][h], ref["eig_v"][h])):
            assert np.abs(rk.T @ rk - np.eye(d)).max() <= 1e-10                         # O1
            np.testing.assert_allclose(np.diag(rk.T @ c @ rk), np.trace(c) / d, rtol=1e-9)  # O6
        # columns of R agree wherever the eigenvalue gap is wide (signs are canonical)
        for key, ek in (("r_k", ref["eig_k"][h]), ("r_v", ref["eig_v"][h])):
            gap = np.minimum(np.r_[np.inf, -np.diff(ek)], np.r_[-np.diff(ek), np.inf]) / ek[0]
            u_got = got[key][h] @ orot.bitrev_perm(d) @ (orot.hadamard(d) / np.sqrt(d)).T
            u_ref = ref[key][h] @ orot.bitrev_perm(d) @ (orot.hadamard(d) / np.sqrt(d)).T
            wide = gap > 1e-3
            assert np.abs(u_got[:, wide] - u_ref[:, wide]).max() <= 1e-8
    # tau depends on R, which is unique only up to rotations inside
    # near-degenerate eigenspaces, so it agrees to the eigensolver's accuracy
    assert got["tau_k"] == pytest.approx(ref["tau_k"], rel=1e-9)
    assert got["tau_v"] == pytest.approx(ref["tau_v"], rel=1e-9)


def test_supplied_attention_output_and_threads():
    w = synth.WORKLOADS["tiny"]
    cal = synth.calibration_set(w, n_rows=300)
    o = np.random.default_rng(1).standard_normal(cal.q.shape).astype(np.float32)
    got = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q, o_calib=o, n_threads=3)
    ref = orot.build_rotation(cal.q, cal.k, cal.v, w.group_q, oc=o)
    np.testing.assert_allclose(got["eig_v"], ref["eig_v"], rtol=0, atol=1e-10 * ref["eig_v"].max())
    one = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q, n_threads=1)
    many = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q, n_threads=8)
    assert np.array_equal(one["r_k"], many["r_k"]) and np.array_equal(one["r_v"], many["r_v"])


def test_jacobi_non_convergence_is_reported():
    w = synth.WORKLOADS["tiny"]
    cal = synth.calibration_set(w, n_rows=64)
    with pytest.raises(lib.OscarError) as e:
        lib.build_rotation(cal.q, cal.k, cal.v, w.group_q, max_sweeps=1)
    assert e.value.status == 3


@pytest.mark.parametrize("variant", [lib.ROTATION_HADAMARD, lib.ROTATION_IDENTITY])
def test_fixed_rotation_matches_oracle(variant):
    w = synth.WORKLOADS["qwen3-8b-b1-32k"]
    cal = synth.calibration_set(w, n_rows=256)
    got = lib.build_fixed_rotation(variant, cal.k, cal.v, n_threads=3)
    ref = orot.fixed_rotation(variant, cal.k, cal.v)
    assert np.array_equal(got["r_k"], ref["r_k"]) and np.array_equal(got["r_v"], ref["r_v"])
    assert got["tau_k"] == pytest.approx(ref["tau_k"], rel=1e-13)
    assert got["tau_v"] == pytest.approx(ref["tau_v"], rel=1e-13)


def test_fixed_rotation_validation():
    k = np.zeros((4, 1, 64), np.float32)
    with pytest.raises(lib.OscarError) as e:
        lib.build_fixed_rotation(5, k, k)
    assert e.value.status == 1
    with pytest.raises(lib.OscarError) as e:
        lib.build_fixed_rotation(lib.ROTATION_IDENTITY, np.zeros((4, 1, 96), np.float32),
                                 np.zeros((4, 1, 96), np.float32))
    assert e.value.status == 2
    bad = k.copy(); bad[1, 0, 3] = np.inf
    with pytest.raises(lib.OscarError) as e:
        lib.build_fixed_rotation(lib.ROTATION_HADAMARD, bad, k)
    assert e.value.status == 3


def test_rotation_from_targets_matches_build_rotation():
    # steps 2-4 from the oracle's targets reproduce the full host calibration
    w = synth.WORKLOADS["tiny"]
    cal = synth.calibration_set(w, n_rows=600)
    o = np.random.default_rng(2).standard_normal(cal.q.shape).astype(np.float32)
    full = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q, o_calib=o)
    cq, cs = orot.calibration_targets(np.asarray(cal.q, np.float32).astype(np.float64),
                                      np.asarray(cal.k, np.float32).astype(np.float64),
                                      np.asarray(cal.v, np.float32).astype(np.float64), w.group_q,
                                      oc=o.astype(np.float64))
    got = lib.build_rotation_from_targets(cq, cs, cal.k, cal.v, n_threads=2)
    for key in ("eig_k", "eig_v"):
        np.testing.assert_allclose(got[key], full[key], rtol=0, atol=1e-10 * np.abs(full[key]).max())
    for key in ("r_k", "r_v"):
        assert np.abs(got[key] - full[key]).max() <= 1e-6
    assert got["tau_k"] == pytest.approx(full["tau_k"], rel=1e-9)
    assert got["tau_v"] == pytest.approx(full["tau_v"], rel=1e-9)
    # the symmetric part is what counts
    skew = np.random.default_rng(3).standard_normal(cq.shape) * 1e-3
    got2 = lib.build_rotation_from_targets(cq + skew - skew.transpose(0, 2, 1), cs, cal.k, cal.v)
    np.testing.assert_allclose(got2["eig_k"], got["eig_k"], rtol=0, atol=1e-10 * np.abs(got["eig_k"]).max())
    bad = cq.copy(); bad[0, 1, 2] = np.nan
    with pytest.raises(lib.OscarError) as e:
        lib.build_rotation_from_targets(bad, cs, cal.k, cal.v)
    assert e.value.status == 3
