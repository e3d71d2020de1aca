"""Pins of the oracle's early-stopping functions ([S2O] §2 Early-stopping rule,
§3 Kernel implementation) against a hand-worked example, library attention
and properties the rule fixes."""
import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

from oracle import spot_oracle as O

GOLDEN = Path(__file__).parent / "golden" / "es_worked.json"


def _worked_inputs(spec):
    L, d, B = spec["L"], spec["d"], spec["block"]
    q = np.zeros((1, L, d))
    q[0, :, 0] = 1.0
    k = np.zeros((1, L, d))
    v = np.zeros((1, L, d))
    k[0, 16:20, 0] = math.log(0.25)
    v[0, 16:20, 0] = 1.0
    for rank, j in enumerate(spec["order"], start=1):
        ts = np.arange(j * B, (j + 1) * B)
        k[0, ts, 0] = math.log(2.0 ** -rank / 2)
        v[0, ts, rank] = 1.0
    return q, k, v


def test_worked_example_matches_hand_values():
    spec = json.loads(GOLDEN.read_text())
    q, k, v = _worked_inputs(spec)
    i = spec["query_block"]
    order = [[None] * 10]
    order[0][i] = np.array(spec["order"])
    o, lse, used = O.attend_prefill_es(q, k, v, order, spec["block"], spec["segment"], spec["sm_scale"],
                                       spec["tau"], qblocks=[i])
    for row, exp in spec["expected"].items():
        r = int(row)
        assert used[0, r] == exp["nused"]
        want = np.array([float(Fraction(x)) for x in exp["o"]])
        np.testing.assert_allclose(o[0, r], want, rtol=0, atol=1e-14)
        assert lse[0, r] == pytest.approx(math.log(float(Fraction(exp["lse_exp"]))), abs=1e-14)


def _sdpa(q, k, v, mask, scale):
    """Library attention in float64: q (Hq, L, d), k/v (Hkv, L, d), mask (Hq|1, L, L) bool."""
    G = q.shape[0] // k.shape[0]
    kk = torch.from_numpy(np.repeat(k, G, axis=0))
    vv = torch.from_numpy(np.repeat(v, G, axis=0))
    qq = torch.from_numpy(q)
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=scale)
    logits = (qq @ kk.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~m, -math.inf), dim=-1)
    return o.numpy(), lse.numpy()


def _case(seed, hq, hkv, L, d, B, S, with_perm):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, L, d))
    k = rng.standard_normal((hkv, L, d))
    v = rng.standard_normal((hkv, L, d))
    perm = None
    if with_perm:
        perm = np.empty((hkv, L), dtype=np.int64)
        for g in range(hkv):
            for s0 in range(0, L, S):
                ts = np.arange(s0, min(s0 + S, L))
                perm[g, ts] = rng.permutation(ts)
    scores = rng.standard_normal((hkv, -(-L // B), -(-L // B)))
    return q, k, v, perm, scores


@pytest.mark.parametrize("with_perm", [False, True])
@pytest.mark.parametrize("hq,hkv,L,d,B,S", [(2, 1, 200, 16, 16, 64), (4, 2, 96, 8, 8, 32)])
def test_tau_zero_is_dense_causal(with_perm, hq, hkv, L, d, B, S):
    """With tau = 0 no block is ever below the threshold: every history block
    is visited, and the union of the history (a permutation of the earlier
    segments) and the causal own segment is exactly dense causal attention."""
    q, k, v, perm, scores = _case(7, hq, hkv, L, d, B, S, with_perm)
    order = O.history_order(scores, B, S)
    o, lse, used = O.attend_prefill_es(q, k, v, order, B, S, 0.3, 0.0, perm=perm)
    mask = np.tril(np.ones((L, L), dtype=bool))[None]
    o_ref, lse_ref = _sdpa(q, k, v, mask, 0.3)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)
    nb = -(-L // B)
    for i in range(nb):
        rows = O.block_rows(i, B, L)
        assert (used[:, rows] == ((i * B) // S) * S // B).all()


@pytest.mark.parametrize("with_perm", [False, True])
def test_large_tau_visits_exactly_one_history_block(with_perm):
    """tau > 1: a block's gain never exceeds the accumulated mass that
    includes it, so every row stops after the first visited block.  The
    result is library attention over the own segment (causal) plus the
    physical rows of the first block in visiting order."""
    hq, hkv, L, d, B, S = 2, 1, 160, 16, 16, 48
    q, k, v, perm, scores = _case(11, hq, hkv, L, d, B, S, with_perm)
    order = O.history_order(scores, B, S)
    o, lse, used = O.attend_prefill_es(q, k, v, order, B, S, 0.25, 1.5, perm=perm)
    nb = -(-L // B)
    mask = np.zeros((L, L), dtype=bool)
    for i in range(nb):
        rows = O.block_rows(i, B, L)
        s0 = ((i * B) // S) * S
        for r in rows:
            mask[r, s0:r + 1] = True
        if len(order[0][i]):
            j = int(order[0][i][0])
            phys = O.block_rows(j, B, L) if perm is None else perm[0, O.block_rows(j, B, L)]
            mask[np.ix_(rows, phys)] = True
            assert (used[:, rows] == 1).all()
        else:
            assert (used[:, rows] == 0).all()
    o_ref, lse_ref = _sdpa(q, k, v, mask[None], 0.25)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_history_order_is_the_unique_sorted_order():
    """Visiting order: exactly the history blocks, scores non-increasing, equal
    scores by ascending block id (these properties fix the order)."""
    rng = np.random.default_rng(3)
    B, S, nb = 16, 64, 40
    scores = np.round(rng.standard_normal((2, nb, nb)), 1)   # many exact ties
    order = O.history_order(scores, B, S)
    for g in range(2):
        for i in range(nb):
            n_hist = (i * B // S) * S // B
            o = order[g][i]
            assert sorted(o.tolist()) == list(range(n_hist))
            s = scores[g, i, o]
            assert (np.diff(s) <= 0).all()
            ties = np.diff(s) == 0
            assert (np.diff(o)[ties] > 0).all()
    # the first segment has no history
    assert all(len(order[0][i]) == 0 for i in range(S // B))


def test_stop_count_is_monotone_in_tau():
    """A larger threshold can only stop earlier: the rule stops at the first
    block whose ratio is below tau."""
    q, k, v, perm, scores = _case(5, 2, 1, 256, 16, 16, 64, True)
    order = O.history_order(scores, 16, 64)
    prev = None
    for tau in (0.0, 0.002, 0.01, 0.05, 0.2, 1.5):
        _, _, used = O.attend_prefill_es(q, k, v, order, 16, 64, 0.25, tau, perm=perm)
        if prev is not None:
            assert (used <= prev).all()
        prev = used


def test_given_stop_counts_reproduce_the_rule():
    """Evaluating at the rule's own stop counts gives the same output, and the
    gain ratios place every stop where the rule says (first ratio below tau)."""
    q, k, v, perm, scores = _case(9, 2, 1, 192, 16, 16, 64, True)
    order = O.history_order(scores, 16, 64)
    o, lse, used = O.attend_prefill_es(q, k, v, order, 16, 64, 0.25, 0.03, perm=perm)
    o2, lse2, used2 = O.attend_prefill_es(q, k, v, order, 16, 64, 0.25, 0.03, perm=perm, nused=used)
    np.testing.assert_array_equal(used, used2)
    np.testing.assert_allclose(o2, o, atol=0)
    for i in (5, 11):
        rows = O.block_rows(i, 16, 192)
        for h in range(2):
            ratio = O.es_gain_ratios(q, k, i, 0, h, order[0][i], 16, 64, 0.25, perm)
            for ri, r in enumerate(rows):
                n = used[h, r]
                assert (ratio[ri, :n - 1] >= 0.03).all()
                assert n == ratio.shape[1] or ratio[ri, n - 1] < 0.03
