"""Pins of the oracle's second-order Taylor block score ([SPLA] §2.1):
block variances in closed form, the first-order special case, and the order
of the expansion error against the exact block mass it approximates."""
import math

import numpy as np
import pytest

from oracle import spot_oracle as O


def _axis_pair_block(mean, amps, axes, B):
    """B rows: mean + a e_m and mean - a e_m for each (a, m) pair; remaining
    rows equal the mean.  Mean exactly `mean`, covariance exactly diagonal
    with var_m = (2 * sum of a^2 over pairs on axis m) / B."""
    rows = np.tile(mean, (B, 1))
    r = 0
    for a, m in zip(amps, axes):
        rows[r, m] += a
        rows[r + 1, m] -= a
        r += 2
    var = np.zeros_like(mean)
    for a, m in zip(amps, axes):
        var[m] += 2 * a * a / B
    return rows, var


def test_block_variance_closed_form_natural_and_permuted():
    rng = np.random.default_rng(1)
    B, d, nb = 8, 5, 3
    k = np.zeros((1, B * nb, d))
    want = np.zeros((nb, d))
    for j in range(nb):
        mean = rng.standard_normal(d)
        rows, var = _axis_pair_block(mean, [0.5 * (j + 1), 1.25, 0.75], [0, 2, (j + 1) % d], B)
        k[0, j * B:(j + 1) * B] = rows
        want[j] = var
    vn, vp = O.key_block_variance(k, B)
    np.testing.assert_allclose(vn[0], want, atol=1e-12)
    np.testing.assert_array_equal(vp, vn)
    # a permutation that swaps the rows of blocks 0 and 2 (one segment of 3 blocks)
    perm = np.concatenate([np.arange(2 * B, 3 * B), np.arange(B, 2 * B), np.arange(0, B)])[None]
    vn2, vp2 = O.key_block_variance(k, B, perm)
    np.testing.assert_allclose(vp2[0, 0], want[2], atol=1e-12)
    np.testing.assert_allclose(vp2[0, 2], want[0], atol=1e-12)
    np.testing.assert_allclose(vn2[0], want, atol=1e-12)


def test_zero_variance_reduces_to_the_first_order_score():
    """Constant keys inside every block: the second-order term vanishes and the
    score is sm_scale * <qbar, kbar>, the mean-pooled score."""
    rng = np.random.default_rng(2)
    B, d, nb, G = 4, 8, 6, 2
    kb = rng.standard_normal((1, nb, d))
    k = np.repeat(kb, B, axis=1)
    q = rng.standard_normal((G, nb * B, d))
    qbar, kn, kp = O.pool_blocks(q, k, B)
    vn, vp = O.key_block_variance(k, B)
    assert np.all(vn == 0)
    t = O.taylor_scores(qbar, kn, kp, vn, vp, B, 0, 0.3)
    m = O.meanpool_scores(qbar, kn, kp, B, 0, 0.3)
    np.testing.assert_allclose(t, m, atol=1e-14)


def _exact_and_scores(eps, scale=0.4, seed=3):
    """One query block whose rows all equal q0 (so qbar = q0) and key blocks of
    axis-aligned +-eps pairs around their means."""
    rng = np.random.default_rng(seed)
    B, d, nb = 8, 6, 4
    q0 = rng.standard_normal(d)
    q = np.tile(q0, (1, nb * B, 1))
    k = np.zeros((1, nb * B, d))
    for j in range(nb):
        mean = rng.standard_normal(d)
        rows, _ = _axis_pair_block(mean, [eps * 1.0, eps * 0.7, eps * 1.3, eps * 0.4], [0, 1, 3, 5], B)
        k[0, j * B:(j + 1) * B] = rows
    qbar, kn, kp = O.pool_blocks(q, k, B)
    vn, vp = O.key_block_variance(k, B)
    i = nb - 1
    t = O.taylor_scores(qbar, kn, kp, vn, vp, B, 0, scale)[0, i]
    m = O.meanpool_scores(qbar, kn, kp, B, 0, scale)[0, i]
    exact = np.array([math.log(np.mean(np.exp(scale * (k[0, j * B:(j + 1) * B] @ q0)))) for j in range(nb)])
    return t, m, exact


def test_expansion_error_is_fourth_order():
    """The exact quantity the score approximates is the block's log mean of
    exp(sm_scale * q . k).  With a symmetric spread eps around the block mean
    the first-order (mean-pool) score is off by O(eps^2) and the second-order
    one by O(eps^4): halving eps divides the errors by about 4 and 16."""
    errs_t, errs_m = [], []
    for eps in (0.2, 0.1, 0.05):
        t, m, exact = _exact_and_scores(eps)
        errs_t.append(np.abs(t - exact).max())
        errs_m.append(np.abs(m - exact).max())
    for a, b in zip(errs_m, errs_m[1:]):
        assert 3.5 < a / b < 4.5
    for a, b in zip(errs_t, errs_t[1:]):
        assert 13.0 < a / b < 19.0
    assert errs_t[-1] < 1e-2 * errs_m[-1]


def test_history_blocks_use_permuted_statistics():
    """Under a segment permutation, history blocks are scored with the mean and
    variance of the rows the permutation gathers (checked against a second
    call on physically permuted keys, where the permuted rows are natural)."""
    rng = np.random.default_rng(4)
    B, S, d, G, L = 4, 8, 6, 2, 24
    q = rng.standard_normal((G, L, d))
    k = rng.standard_normal((1, L, d)) * rng.uniform(0.2, 2.0, size=(1, L, 1))
    perm = np.concatenate([s0 + rng.permutation(S) for s0 in range(0, L, S)])[None]
    qbar, kn, kp = O.pool_blocks(q, k, B, perm)
    vn, vp = O.key_block_variance(k, B, perm)
    t = O.taylor_scores(qbar, kn, kp, vn, vp, B, S, 0.35)
    kq = k[:, perm[0]]
    _, kn2, _ = O.pool_blocks(q, kq, B)
    vn2, _ = O.key_block_variance(kq, B)
    t_all_perm = O.taylor_scores(qbar, kn2, kn2, vn2, vn2, B, 0, 0.35)
    t_nat = O.taylor_scores(qbar, kn, kn, vn, vn, B, 0, 0.35)
    nb = L // B
    for i in range(nb):
        for j in range(i + 1):
            ref = t_all_perm if O.is_history(j, i, B, S) else t_nat
            assert t[0, i, j] == pytest.approx(ref[0, i, j], abs=1e-12)


def test_worked_example_matches_hand_values():
    import json
    from fractions import Fraction
    from pathlib import Path
    spec = json.loads((Path(__file__).parent / "golden" / "taylor_worked.json").read_text())
    keys = np.array(spec["keys"])[None]
    q = np.tile(np.array(spec["q_row"]), (1, len(spec["keys"]), 1))
    qbar, kn, kp = O.pool_blocks(q, keys, spec["block"])
    vn, vp = O.key_block_variance(keys, spec["block"])
    np.testing.assert_allclose(kn[0, 0], spec["expected_mean"], atol=1e-15)
    np.testing.assert_allclose(vn[0, 0], spec["expected_var"], atol=1e-15)
    s = O.taylor_scores(qbar, kn, kp, vn, vp, spec["block"], 0, spec["sm_scale"])
    assert s[0, 0, 0] == pytest.approx(math.log(float(Fraction(spec["expected_score_exp"]))), abs=1e-15)
