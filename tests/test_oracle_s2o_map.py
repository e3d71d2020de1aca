"""Pins of the oracle's representative-query history map ([S2O] §1: historical
keys scored against a representative query of the segment under a causal
prefix; the sorted indices form the segment's logical map) and of the
early-stopped attention walking that map ([S2O] §2-3)."""
import math

import numpy as np
import pytest
import torch

from oracle import spot_oracle as O
from tests.test_oracle_early_stop import _sdpa


def test_representative_query_is_the_segment_mean():
    """Rows built as a per-segment constant plus noise that cancels in pairs
    of heads: the representative query is exactly the constant, also for a
    partial last segment."""
    rng = np.random.default_rng(1)
    hkv, G, L, S, d = 2, 2, 22, 8, 5
    c = rng.standard_normal((hkv, 3, d))
    noise = rng.standard_normal((L, d))
    q = np.empty((hkv * G, L, d))
    for g in range(hkv):
        for t in range(L):
            q[g * G, t] = c[g, t // S] + noise[t]
            q[g * G + 1, t] = c[g, t // S] - noise[t]
    rq = O.representative_queries(q, hkv, S)
    np.testing.assert_allclose(rq, c, atol=1e-14)


def test_history_map_hand_example():
    """One head, d = 2, sm_scale = 1, every query (1, 0), keys (v_t, 0) with
    v = 3 1 4 1 5 9 2 6 5 3 5 8, segments of 4.  Segment 1 sorts v[0:4]
    descending: positions 2 0 1 3 (the two 1s by position); segment 2 sorts
    v[0:8]: positions 5 7 4 2 0 6 1 3."""
    v = [3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5, 8]
    L = len(v)
    q = np.zeros((1, L, 2))
    q[0, :, 0] = 1.0
    k = np.zeros((1, L, 2))
    k[0, :, 0] = v
    hmap, score = O.history_map(q, k, 4, 1.0)
    assert hmap[0, 1, :4].tolist() == [2, 0, 1, 3]
    assert hmap[0, 2, :8].tolist() == [5, 7, 4, 2, 0, 6, 1, 3]
    assert (hmap[0, 0] == -1).all() and (hmap[0, 1, 4:] == -1).all()
    np.testing.assert_array_equal(score[0, 2, :8], np.array(v[:8], dtype=float))


def test_history_map_properties():
    """Each segment's map is a permutation of its prefix, scores non-increasing
    along it, equal scores by ascending position."""
    rng = np.random.default_rng(2)
    hq, hkv, L, S, d = 4, 2, 300, 64, 8
    q = rng.standard_normal((hq, L, d))
    k = np.round(rng.standard_normal((hkv, L, d)), 0)       # many exact score ties
    hmap, score = O.history_map(q, k, S, 0.5)
    for g in range(hkv):
        for sg in range(1, -(-L // S)):
            n = sg * S
            m = hmap[g, sg, :n]
            assert sorted(m.tolist()) == list(range(n))
            sc = score[g, sg, m]
            assert (np.diff(sc) <= 0).all()
            assert (np.diff(m)[np.diff(sc) == 0] > 0).all()


@pytest.mark.parametrize("tau", [0.0, 1.5])
def test_attention_on_the_map_at_the_extremes(tau):
    """tau = 0 takes the whole map (the full prefix): dense causal attention.
    tau > 1 takes exactly the first B positions of the map."""
    rng = np.random.default_rng(3)
    hq, hkv, L, d, B, S = 4, 2, 192, 16, 16, 64
    q = rng.standard_normal((hq, L, d))
    k = rng.standard_normal((hkv, L, d))
    v = rng.standard_normal((hkv, L, d))
    hmap, _ = O.history_map(q, k, S, 0.25)
    o, lse, used = O.attend_prefill_es(q, k, v, None, B, S, 0.25, tau, hmap=hmap)
    G = hq // hkv
    mask = np.zeros((hq, L, L), dtype=bool)
    for h in range(hq):
        g = h // G
        for r in range(L):
            s0 = (r // S) * S
            mask[h, r, s0:r + 1] = True
            if s0:
                mask[h, r, hmap[g, s0 // S, :s0] if tau == 0.0 else hmap[g, s0 // S, :B]] = True
    o_ref, lse_ref = _sdpa(q, k, v, mask, 0.25)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)
    nb = L // B
    for i in range(nb):
        rows = O.block_rows(i, B, L)
        n_hist = (i * B // S) * S // B
        assert (used[:, rows] == (n_hist if tau == 0.0 else min(n_hist, 1))).all()
