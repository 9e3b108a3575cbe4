"""Pins of oracle.quant: hand-worked groups, nearest-level brute force, grid
special cases, degenerate groups, f16 rounding ([TS] 2.2.B; readings in the
module docstring)."""
import os

import numpy as np
import pytest

from oracle import quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _examples():
    ex, cur = [], None
    with open(os.path.join(GOLD, "quant_groups.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            if key == "example":
                cur = {"name": vals[0]}
                ex.append(cur)
            else:
                cur[key] = [float(v) for v in vals]
    return ex


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"])
def test_hand_worked_groups(ex):
    x = np.array([ex["x"]])
    qr = quant.quantize_rows(x, np.eye(64), ex["tau"][0])
    assert qr.codes[0].tolist() == [int(c) for c in ex["codes"]]
    assert qr.s16[0].astype(np.float64).tolist() == ex["s16"]
    assert qr.z16[0].astype(np.float64).tolist() == ex["z16"]


def test_f16_round_half_even():
    vals = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2049.0, 2051.0, 65519.0, 65520.0, 2 ** -25, 3 * 2 ** -25])
    with np.errstate(over="ignore"):
        h = vals.astype(np.float16).astype(np.float64)
    assert h.tolist()[:5] == [1.0, 1 + 2 ** -9, 2048.0, 2052.0, 65504.0]
    assert np.isinf(h[5])
    assert h[6] == 0.0 and h[7] == 2 ** -23  # subnormal ties to even


def test_codes_are_nearest_level():
    # O9: every code minimises |y - (c s16 + z16)| over c in {0..3}; a tie only
    # at an exact midpoint.
    rng = np.random.default_rng(1)
    x = rng.standard_normal((400, 128)) * rng.uniform(0.01, 20, size=(400, 1))
    r, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    qr = quant.quantize_rows(x, r, 2.5)
    y = qr.y.reshape(400, 4, 32)
    s = qr.s16.astype(np.float64)[:, :, None]
    z = qr.z16.astype(np.float64)[:, :, None]
    lv = z[..., None] + s[..., None] * np.arange(4)
    err = np.abs(y[..., None] - lv)
    best = err.min(axis=-1)
    mine = np.take_along_axis(err, qr.codes.reshape(400, 4, 32)[..., None].astype(np.int64), -1)[..., 0]
    assert np.all(mine <= best + 1e-12 * np.abs(y).max())


def test_grid_special_case_decodes_exactly():
    # O10: values on the grid z16 + c s16 with f16-exact s and z decode exactly,
    # min -> code 0, max -> code 3.
    rng = np.random.default_rng(4)
    for _ in range(50):
        s16 = np.float16(rng.uniform(0.01, 4)).astype(np.float64)
        z16 = np.float16(rng.uniform(-5, 5)).astype(np.float64)
        c = rng.integers(0, 4, size=32)
        c[0], c[1] = 0, 3
        y = z16 + c * s16
        qr = quant.quantize_rotated(np.tile(y, 2)[None, :])
        if qr.s16[0, 0] != s16:  # (max - min) / 3 == s16 exactly is what the grid implies
            pytest.fail("grid scale not recovered")
        assert qr.codes[0, :32].tolist() == c.tolist()
        np.testing.assert_array_equal(quant.dequantize(qr.codes, qr.s16, qr.z16)[0, :32], y)


def test_degenerate_and_clipped_groups():
    x = np.concatenate([np.full(32, 0.75), np.full(32, 9.0)])[None, :]
    qr = quant.quantize_rows(x, np.eye(64), 2.0)
    assert qr.codes.max() == 0
    assert qr.s16.tolist() == [[0.0, 0.0]]
    assert qr.z16.astype(np.float64).tolist() == [[0.75, 2.0]]
    np.testing.assert_array_equal(quant.dequantize(qr.codes, qr.s16, qr.z16)[0], np.concatenate([np.full(32, 0.75), np.full(32, 2.0)]))


def test_clip_is_symmetric():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((20, 64)) * 10
    y = quant.rotate_clip(x, np.eye(64), 3.0)
    assert y.max() == 3.0 and y.min() == -3.0
    inside = np.abs(x) < 3.0
    np.testing.assert_array_equal(y[inside], x[inside])


def test_boundary_helpers():
    assert quant.boundary_distance(np.array([0.5, 1.25, 3.0, 2.49])).tolist() == pytest.approx([0.0, 0.25, 0.5, 0.01])
    assert quant.f16_midpoint_distance(np.array([1 + 2 ** -11]))[0] == 0.0
    assert quant.f16_midpoint_distance(np.array([1.0]))[0] == pytest.approx(2 ** -12)  # below 1.0 the f16 spacing is 2^-11
