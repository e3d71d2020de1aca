"""Pins of the residual linear attention oracle ([SPLA] §2.2-2.3).

What fixes the oracle here, independently of its own code:
  * hand-worked examples (tests/golden/rla_worked.json): prefill rows with
    and without a permutation of the history, and a decode query;
  * keeping every block leaves nothing: the output is exactly zero;
  * the page's subtraction form: the result equals linear attention over
    all visible keys (a running state of outer products, built here) minus
    linear attention over the kept keys (a direct sum, keys gathered here);
  * the exponential feature map: adding c to every query (or key) entry
    scales the output by exp(c); the output is linear in V;
  * the decode query equals the last prefill row for the same kept blocks.
"""
import json
from pathlib import Path

import numpy as np
import pytest

import oracle
from oracle import spot_oracle as O

GOLD = json.loads((Path(__file__).parent / "golden" / "rla_worked.json").read_text())


def _num(x):
    if isinstance(x, dict):
        return np.log(x["ln"])
    if isinstance(x, list):
        return [_num(y) for y in x]
    return float(x)


def _arr(x):
    return np.array(_num(x), dtype=np.float64)


def _lists(kept):
    return [[np.array(row, dtype=np.int64) for row in head] for head in kept]


def test_worked_prefill():
    c = GOLD["prefill"]
    got = O.rla_prefill(_arr(c["q"]), _arr(c["k"]), _arr(c["v"]), _lists(c["kept"]), c["block"])
    np.testing.assert_allclose(got, _arr(c["o_rla"]), rtol=1e-12, atol=1e-12)


def test_worked_prefill_permuted():
    c, p = GOLD["prefill"], GOLD["prefill_permuted"]
    got = O.rla_prefill(_arr(c["q"]), _arr(c["k"]), _arr(c["v"]), _lists(p["kept"]), c["block"],
                        segment=p["segment"], perm=np.array(p["perm"]))
    np.testing.assert_allclose(got, _arr(p["o_rla"]), rtol=1e-12, atol=1e-12)


def test_worked_decode():
    c = GOLD["decode"]
    k, v = _arr(c["k"]), _arr(c["v"])
    got = O.rla_decode(_arr(c["q"]), k, v, c["kept"], c["block"], k.shape[1])
    np.testing.assert_allclose(got, _arr(c["o_rla"]), rtol=1e-12, atol=1e-12)


def _case(seed, L=40, block=4, d=8, hq=4, hkv=2):
    rng = np.random.default_rng(seed)
    q = 0.5 * rng.standard_normal((hq, L, d))
    k = 0.5 * rng.standard_normal((hkv, L, d))
    v = rng.standard_normal((hkv, L, d))
    return q, k, v


def _random_lists(rng, nb, hkv, n_sink=1, n_recent=1):
    lists = []
    for _ in range(hkv):
        rows = []
        for i in range(nb):
            js = np.arange(i + 1)
            keep = (js < n_sink) | (js > i - n_recent) | (rng.random(i + 1) < 0.5)
            rows.append(js[keep])
        lists.append(rows)
    return lists


def _rla_by_subtraction(q, k, v, lists, block, segment=0, perm=None):
    """Linear attention over all visible keys (running outer-product state)
    minus linear attention over the kept keys (direct sum)."""
    hq, L, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    out = np.zeros((hq, L, d))
    for g in range(hkv):
        fk = np.exp(k[g])
        state = np.cumsum(fk[:, :, None] * v[g][:, None, :], axis=0)     # (L, d, d): sum over t' <= t
        for h in range(g * G, (g + 1) * G):
            for r in range(L):
                i = r // block
                fq = np.exp(q[h, r])
                all_vis = fq @ state[r]
                kept = []
                for j in lists[g][i]:
                    ts = np.arange(j * block, min((j + 1) * block, L))
                    if perm is not None and segment and (j * block) // segment < (i * block) // segment:
                        kept.extend(perm[g, ts].tolist())
                    else:
                        kept.extend(t for t in ts.tolist() if t <= r)
                kept = np.array(sorted(kept), dtype=np.int64)
                kept_part = (np.exp(k[g, kept]) @ fq) @ v[g, kept] if kept.size else 0.0
                out[h, r] = all_vis - kept_part
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_difference_of_all_and_kept(seed):
    q, k, v = _case(seed)
    rng = np.random.default_rng(100 + seed)
    lists = _random_lists(rng, 10, 2)
    got = O.rla_prefill(q, k, v, lists, 4)
    ref = _rla_by_subtraction(q, k, v, lists, 4)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_difference_of_all_and_kept_permuted():
    q, k, v = _case(7)
    rng = np.random.default_rng(8)
    segment, block, L = 8, 4, 40
    perm = np.stack([np.concatenate([s + rng.permutation(min(segment, L - s)) for s in range(0, L, segment)])
                     for _ in range(2)])
    lists = _random_lists(rng, 10, 2)
    got = O.rla_prefill(q, k, v, lists, block, segment=segment, perm=perm)
    ref = _rla_by_subtraction(q, k, v, lists, block, segment=segment, perm=perm)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_keep_all_is_zero():
    q, k, v = _case(3)
    res = oracle.prefill(q, k, v, 4, 1.0)
    got = O.rla_prefill(q, k, v, res["kept"], 4)
    assert np.all(got == 0.0)
    nt = 10
    got = O.rla_decode(q[:, -1], k, v, list(range(nt)), 4, 40)
    assert np.all(got == 0.0)


def test_feature_map_shift_and_linearity():
    q, k, v = _case(4)
    lists = _random_lists(np.random.default_rng(5), 10, 2)
    base = O.rla_prefill(q, k, v, lists, 4)
    c = 0.3
    np.testing.assert_allclose(O.rla_prefill(q + c, k, v, lists, 4), np.exp(c) * base, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.rla_prefill(q, k - c, v, lists, 4), np.exp(-c) * base, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.rla_prefill(q, k, 3.0 * v, lists, 4), 3.0 * base, rtol=1e-12, atol=1e-12)


def test_decode_equals_last_prefill_row():
    q, k, v = _case(6)
    L, block = 40, 4
    nb = L // block
    kept = np.array([0, 3, 4, 8, 9])
    lists = [[np.arange(i + 1) for i in range(nb)] for _ in range(2)]
    for g in range(2):
        lists[g][nb - 1] = kept
    pre = O.rla_prefill(q, k, v, lists, block, qblocks=[nb - 1])
    dec = O.rla_decode(q[:, L - 1], k, v, kept, block, L)
    np.testing.assert_allclose(dec, pre[:, L - 1], rtol=1e-12, atol=1e-12)
