"""Online quantization of a row: rotate, clip, asymmetric INT2 per group (fp64).

[TS] 2.2.B: the middle history is stored in INT2 after the fixed rotation and
clipping; [TS] 1 motivates small groups (outliers set the scale).  Readings:
groups of 32 consecutive rotated channels per token, zero = group minimum,
scale = range / 3, scale and zero stored as f16 (round-half-to-even) and codes
computed against the stored f16 values, codes rounded half-to-even and clamped
to [0, 3], code 0 when the stored scale is 0.

The INT4 cache variant ([TS] 4 "Scalability": the INT4 KV baseline OSCAR's
capacity is compared with) is the same quantizer with 16 levels: scale =
range / 15, codes clamped to [0, 15] (``bits=4``).
"""
from __future__ import annotations

import dataclasses

import numpy as np

GROUP = 32


@dataclasses.dataclass
class QuantRows:
    codes: np.ndarray   # uint8 [n, d]
    s16: np.ndarray     # float16 [n, n_g]
    z16: np.ndarray     # float16 [n, n_g]
    t: np.ndarray       # float64 [n, d]  (y - z16) / s16 before rounding (nan where s16 == 0)
    s: np.ndarray       # float64 [n, n_g] scale before f16 rounding
    z: np.ndarray       # float64 [n, n_g] zero before f16 rounding
    y: np.ndarray       # float64 [n, d]  rotated and clipped rows


def rotate_clip(x: np.ndarray, r: np.ndarray, tau: float) -> np.ndarray:
    """y = clamp(x . R, -tau, tau) in float64."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(r, dtype=np.float64)
    return np.clip(y, -tau, tau)


def levels(bits: int) -> int:
    """Largest code of a ``bits``-bit asymmetric quantizer (3 for INT2, 15 for INT4)."""
    assert bits in (2, 4)
    return (1 << bits) - 1


def quantize_rotated(y: np.ndarray, bits: int = 2) -> QuantRows:
    n, d = y.shape
    ng = d // GROUP
    top = levels(bits)
    yg = y.reshape(n, ng, GROUP)
    mn = yg.min(axis=2)
    mx = yg.max(axis=2)
    s = (mx - mn) / float(top)
    z = mn
    s16 = s.astype(np.float16)
    z16 = z.astype(np.float16)
    s64 = s16.astype(np.float64)[:, :, None]
    z64 = z16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s64 != 0.0, (yg - z64) / s64, np.nan)
    codes = np.where(s64 != 0.0, np.clip(np.rint(np.nan_to_num(t)), 0, top), 0).astype(np.uint8)
    return QuantRows(codes.reshape(n, d), s16, z16, t.reshape(n, d), s, z, y)


def quantize_rows(x: np.ndarray, r: np.ndarray, tau: float, bits: int = 2) -> QuantRows:
    return quantize_rotated(rotate_clip(x, r, tau), bits)


def dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """Decoded rotated values c * s + z (float64), [n, d]."""
    n, d = codes.shape
    ng = d // GROUP
    c = codes.reshape(n, ng, GROUP).astype(np.float64)
    return (c * s16.astype(np.float64)[:, :, None] + z16.astype(np.float64)[:, :, None]).reshape(n, d)


def boundary_distance(t: np.ndarray, bits: int = 2) -> np.ndarray:
    """Distance of t from the nearest rounding boundary k + 1/2, k in {0, .., levels - 1}."""
    bounds = np.arange(levels(bits)) + 0.5
    return np.min(np.abs(np.nan_to_num(t, nan=-10.0)[..., None] - bounds), axis=-1)


def f16_midpoint_distance(v: np.ndarray) -> np.ndarray:
    """Relative distance of float64 values from the nearest f16 rounding midpoint."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16).astype(np.float64)
    up = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    mids = np.stack([(h + up) / 2, (h + dn) / 2])
    scale = np.maximum(np.abs(v), 1e-300)
    return np.min(np.abs(mids - v[None]), axis=0) / scale
