"""Pins of the oracle's MXFP4 encoding of the indexer keys ([Spot] §4; OCP
Microscaling v1.0 MXFP4 element and scale encodings): hand-worked groups
(ties, saturation, zero and subnormal groups), the E2M1 value table, and
properties of the shared scale and of rounding to the nearest value."""
import json
from pathlib import Path

import numpy as np
import pytest

from oracle import spot_oracle as O

SPEC = json.loads((Path(__file__).parent / "golden" / "mxfp4_worked.json").read_text())


def _value(v):
    if isinstance(v, str):      # "2^-128", "-3*2^-130"
        sign = -1.0 if v.startswith("-") else 1.0
        v = v.lstrip("-")
        mul = 1.0
        if "*" in v:
            m, v = v.split("*")
            mul = float(m)
        return sign * mul * 2.0 ** float(v.split("^")[1])
    return float(v)


@pytest.mark.parametrize("gi", range(len(SPEC["groups"])))
def test_worked_groups(gi):
    grp = SPEC["groups"][gi]
    x = np.array([_value(v) for v in grp["values"]])
    if gi == 0:
        x[10] = -0.0
    codes, scales = O.mxfp4_quantize(x)
    assert scales.tolist() == [grp["scale_byte"]]
    assert codes.tolist() == grp["codes"]


def test_code_value_table():
    codes = np.tile(np.arange(16, dtype=np.uint8), 2).reshape(1, 32)
    vals = O.mxfp4_dequantize(codes, np.array([127], dtype=np.uint8))
    want = np.array(SPEC["code_values"]["values"], dtype=np.float64)
    np.testing.assert_array_equal(vals[0, :16], want)
    assert np.signbit(vals[0, 8])


def test_scale_and_nearest_rounding_properties():
    """max|x| / scale lies in [4, 8); every decoded element is a nearest E2M1
    multiple of the scale (or the saturated 6 * scale)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 32)) * np.exp2(rng.integers(-20, 20, size=(200, 1)))).astype(np.float32)
    x = x.astype(np.float64)
    codes, scales = O.mxfp4_quantize(x)
    sc = 2.0 ** (scales.astype(np.float64) - 127)
    r = np.abs(x).max(axis=1) / sc[:, 0]
    assert np.all((r >= 4) & (r < 8))
    deq = O.mxfp4_dequantize(codes, scales)
    grid = np.array(O.E2M1_MAGNITUDES)
    y = np.abs(x) / sc
    best = np.abs(grid[None, None, :] - np.minimum(y, 6.0)[..., None]).min(axis=-1)
    err = np.abs(np.abs(deq) / sc - np.minimum(y, 6.0))
    assert np.all(err <= best + 1e-12)
    assert np.all(np.sign(deq[deq != 0]) == np.sign(x[deq != 0]))


def test_grid_values_round_trip_and_packing():
    rng = np.random.default_rng(6)
    grid = np.array(O.E2M1_MAGNITUDES)
    mags = grid[rng.integers(0, 8, size=(50, 64))]
    mags[:, 0] = 6.0                                  # max 6 -> scale 2^0
    x = mags * np.where(rng.random((50, 64)) < 0.5, -1.0, 1.0) * 2.0 ** 3
    codes, scales = O.mxfp4_quantize(x)
    np.testing.assert_array_equal(O.mxfp4_dequantize(codes, scales), x)
    packed = O.mxfp4_pack(codes)
    assert packed.shape == (50, 32)
    np.testing.assert_array_equal(O.mxfp4_unpack(packed), codes)
    assert packed[0, 0] == (codes[0, 0] | (codes[0, 1] << 4))
