"""Pins of the oracle's INT4 encoding of the indexer keys ([Spot] §4: the
selector's K-cache as INT4 or FP4 microscale): hand-worked groups (exact and
rounded scales, ties, an all-zero group, a negative largest magnitude),
properties of the scale and of rounding to the nearest integer on random
bf16 groups, the packing order, and the decode step through the encoding."""
import json
from pathlib import Path

import numpy as np
import pytest

from block_sparse_attention_amd import inputs as I
from oracle import spot_oracle as O

SPEC = json.loads((Path(__file__).parent / "golden" / "int4_worked.json").read_text())


@pytest.mark.parametrize("gi", range(len(SPEC["groups"])))
def test_worked_groups(gi):
    grp = SPEC["groups"][gi]
    x = np.array(grp["values"], dtype=np.float64)
    assert np.array_equal(I.round_bf16(x.astype(np.float32)).astype(np.float64), x)   # inputs are bf16 values
    codes, scales = O.int4_quantize(x)
    assert scales.tolist() == [grp["scale"]]
    assert codes.tolist() == grp["codes"]
    assert np.array_equal(O.int4_dequantize(codes, scales), np.array(grp["codes"], float) * grp["scale"])


def _bf16_groups(n, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, 32)).astype(np.float32) * np.exp2(r.integers(-20, 20, (n, 1))).astype(np.float32)
    x[::7, :] = 0.0
    x[3::11, ::3] = 0.0
    return I.round_bf16(x).astype(np.float64)


def test_scale_and_rounding_properties():
    x = _bf16_groups(4000, 5)
    codes, scales = O.int4_quantize(x)
    deq = O.int4_dequantize(codes, scales)
    scales = scales[:, 0]                      # one group per row
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    # the scale is a bf16 value within half a bf16 spacing of max|x| / 7
    s32 = scales.astype(np.float32)
    assert np.array_equal(s32.astype(np.float64), scales)
    assert np.all((s32.view(np.uint32) & 0xFFFF) == 0)
    spacing = np.exp2(np.floor(np.log2(np.where(nz, amax / 7, 1.0))) - 7)
    assert np.all(np.abs(scales[nz] - amax[nz] / 7) <= spacing[nz] / 2)
    assert np.all(scales[~nz] == 0) and np.all(codes[~nz] == 0)
    # codes are integers in [-7, 7]; the largest magnitude of a group codes to +-7
    assert codes.min() >= -7 and codes.max() <= 7
    assert np.all(np.abs(codes[nz]).max(axis=1) == 7)
    # every element goes to its nearest multiple of the scale (within [-7, 7] of it)
    err = np.abs(deq - x)
    assert np.all(err <= scales[:, None] / 2 + 1e-300)
    # and no other code in range is nearer
    for dc in (-1, 1):
        other = np.clip(codes.astype(int) + dc, -7, 7)
        assert np.all(np.abs(other * scales[:, None] - x) >= err - 1e-300)


def test_packing_order_and_twos_complement():
    codes = np.array([[-7, 7, -1, 0, 3, -4] + [0] * 26], dtype=np.int8)
    packed = O.int4_pack(codes)
    assert packed.shape == (1, 16)
    # element 2k in the low nibble, 2k+1 in the high one, 4-bit two's complement
    assert packed[0, :3].tolist() == [0x9 | (0x7 << 4), 0xF | (0x0 << 4), 0x3 | (0xC << 4)]


def test_size_ratio_matches_the_page():
    # 4 bits per element + one 16-bit scale per 32 elements, against 16 bits per element
    assert abs(16 / (4 + 16 / 32) - 3.5) < 0.1


def test_decode_through_int4_keys_is_decode_on_the_decoded_keys():
    r = np.random.default_rng(12)
    hq, hkv, d, B, T = 4, 2, 8, 16, 16 * 40
    nt, h_idx, d_idx = T // B, 2, 32
    kc, vc = r.standard_normal((hkv, T, d)), r.standard_normal((hkv, T, d))
    q = r.standard_normal((hq, d))
    qI = I.round_bf16(r.standard_normal((h_idx, d_idx)).astype(np.float32)).astype(np.float64)
    kI = I.round_bf16(r.standard_normal((nt, h_idx, d_idx)).astype(np.float32)).astype(np.float64)
    w = np.array([0.3, 0.7])
    out = O.decode(q, kc, vc, qI, w, kI, B, T, top_p=0.7, idx_format="int4")
    codes, scales = O.int4_quantize(kI.reshape(nt, h_idx * d_idx))
    kdq = O.int4_dequantize(codes, scales).reshape(nt, h_idx, d_idx)
    ref = O.decode(q, kc, vc, qI, w, kdq, B, T, top_p=0.7)
    assert np.array_equal(out["scores"], ref["scores"])
    assert list(out["kept"]) == list(ref["kept"])
    # the encoding moves each score by at most the dot products' rounding bound
    exact = O.indexer_scores(qI, w, kI)
    bound = np.zeros(nt)
    for h in range(h_idx):
        bound += w[h] * (np.abs(qI[h]) @ np.repeat(scales[:, h:h + 1], d_idx, axis=1).T / 2)
    assert np.all(np.abs(out["scores"] - exact) <= bound + 1e-12)
