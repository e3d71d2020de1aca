"""Pins for the float64 oracle, against things other than the oracle itself:
a hand-worked example, library attention (torch, float64, CPU), closed forms,
brute-force enumeration and invariants of attention under permutation.

CPU only (no GPU marker)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from block_sparse_attention_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def sdpa(q, k, v, mask=None, causal=False, scale=None):
    """Library attention in float64 on the CPU. q (H,Lq,d), k/v (H,Lk,d)."""
    tq = torch.from_numpy(np.asarray(q, np.float64))[None]
    tk = torch.from_numpy(np.asarray(k, np.float64))[None]
    tv = torch.from_numpy(np.asarray(v, np.float64))[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal, scale=scale)
    return out[0].numpy()


def expand_kv(k, G):
    return np.repeat(np.asarray(k, np.float64), G, axis=0)


# ----------------------------------------------------------------- worked example
def test_hand_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "tiny_worked.json")))
    P = fx["params"]
    q = np.array(fx["q"], np.float64)
    k = np.array(fx["k"], np.float64)
    v = np.array(fx["v"], np.float64)
    perm = np.array(fx["perm"])
    out = oracle.prefill(q, k, v, P["block"], P["top_p"], P["n_sink"], P["n_recent"], P["k_min"],
                         sm_scale=P["sm_scale"], segment=P["segment"], perm=perm)
    E = fx["expected"]
    np.testing.assert_array_equal(out["qbar"], np.array(E["qbar"], np.float64))
    np.testing.assert_array_equal(out["kbar_nat"], np.array(E["kbar_nat"], np.float64))
    np.testing.assert_array_equal(out["kbar_perm"], np.array(E["kbar_perm"], np.float64))
    exp_s = np.array([[[(-np.inf if x is None else x) for x in row] for row in g] for g in E["scores"]])
    np.testing.assert_array_equal(out["scores"], exp_s)
    for g, rows in enumerate(E["kept"]):
        for i, kept in enumerate(rows):
            assert list(out["kept"][g][i]) == kept, (g, i)
    for row in E["rows"]:
        w = [math.exp(x) for x in row["logits"]]
        z = sum(w)
        o_exp = [sum(wi * v[0, key, c] for wi, key in zip(w, row["keys"])) / z for c in range(2)]
        np.testing.assert_allclose(out["o"][row["head"], row["row"]], o_exp, rtol=1e-14, atol=1e-14)
        m = max(row["logits"])
        lse = m + math.log(sum(math.exp(x - m) for x in row["logits"]))
        assert abs(out["lse"][row["head"], row["row"]] - lse) < 1e-13


# ----------------------------------------------------------------- attention vs library
@pytest.mark.parametrize("L,B,hq,hkv,d", [(100, 16, 4, 2, 8), (64, 16, 1, 1, 16), (257, 32, 6, 3, 4)])
def test_keep_all_is_dense_causal(L, B, hq, hkv, d):
    r = _rng(L + B)
    q = r.standard_normal((hq, L, d))
    k = r.standard_normal((hkv, L, d))
    v = r.standard_normal((hkv, L, d))
    out = oracle.prefill(q, k, v, B, top_p=1.0)
    ref = sdpa(q, expand_kv(k, hq // hkv), expand_kv(v, hq // hkv), causal=True)
    np.testing.assert_allclose(out["o"], ref, rtol=1e-12, atol=1e-12)
    # every block kept
    for g in range(hkv):
        for i, kept in out["kept"][g].items():
            assert list(kept) == list(range(i + 1))
    # LSE against the library logsumexp of the causal logits
    logits = torch.from_numpy(q) @ torch.from_numpy(expand_kv(k, hq // hkv)).transpose(1, 2) / math.sqrt(d)
    logits = logits.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(out["lse"], torch.logsumexp(logits, -1).numpy(), rtol=1e-12, atol=1e-12)


def _random_segment_perm(r, hkv, L, S):
    perm = np.empty((hkv, L), dtype=np.int64)
    for g in range(hkv):
        for s0 in range(0, L, S):
            ts = np.arange(s0, min(s0 + S, L))
            perm[g, ts] = r.permutation(ts)
    return perm


def test_keep_all_with_segment_permutation_is_dense():
    """PBS-Attn section 1: permuting key/value pairs (inside segments) does not
    change attention; with every block kept the permuted path is dense causal."""
    r = _rng(5)
    hq, hkv, L, d, B, S = 4, 2, 200, 8, 16, 64
    q, k, v = r.standard_normal((hq, L, d)), r.standard_normal((hkv, L, d)), r.standard_normal((hkv, L, d))
    perm = _random_segment_perm(r, hkv, L, S)
    out = oracle.prefill(q, k, v, B, top_p=1.0, segment=S, perm=perm)
    ref = sdpa(q, expand_kv(k, 2), expand_kv(v, 2), causal=True)
    np.testing.assert_allclose(out["o"], ref, rtol=1e-12, atol=1e-12)


def _physical_mask(kept, i, g, B, S, perm, L):
    """Independent formulation: which PHYSICAL key rows each query row of block
    i sees, as a boolean mask over all L rows."""
    rows = np.arange(i * B, min((i + 1) * B, L))
    mask = np.zeros((rows.size, L), dtype=bool)
    for j in kept:
        ts = np.arange(j * B, min((j + 1) * B, L))
        if perm is not None and (j * B) // S < (i * B) // S:
            mask[:, perm[g, ts]] = True
        else:
            for a, rr in enumerate(rows):
                mask[a, ts[ts <= rr]] = True
    return rows, mask


@pytest.mark.parametrize("top_p", [0.0, 0.3, 0.7])
def test_sparse_attention_is_masked_library_attention(top_p):
    """Partial selection with a permutation: the oracle's gather equals library
    attention over all rows with a mask on the physical positions."""
    r = _rng(17)
    hq, hkv, L, d, B, S = 4, 2, 160, 8, 16, 64
    q, k, v = r.standard_normal((hq, L, d)), r.standard_normal((hkv, L, d)), r.standard_normal((hkv, L, d))
    perm = _random_segment_perm(r, hkv, L, S)
    out = oracle.prefill(q, k, v, B, top_p=top_p, segment=S, perm=perm)
    G = hq // hkv
    nb = L // B
    for g in range(hkv):
        for i in range(nb):
            rows, mask = _physical_mask(out["kept"][g][i], i, g, B, S, perm, L)
            for h in range(g * G, (g + 1) * G):
                ref = sdpa(q[h:h + 1, rows], k[g:g + 1], v[g:g + 1], mask=mask)[0]
                np.testing.assert_allclose(out["o"][h, rows], ref, rtol=1e-12, atol=1e-12)


def test_forced_only_closed_form():
    """p = 0 keeps only the sink block and the diagonal: for i > 0 the keys of
    row r are block 0 and [iB, r]; for i = 0 they are [0, r]."""
    r = _rng(3)
    hq, hkv, L, d, B = 2, 1, 96, 8, 16
    q, k, v = r.standard_normal((hq, L, d)), r.standard_normal((hkv, L, d)), r.standard_normal((hkv, L, d))
    out = oracle.prefill(q, k, v, B, top_p=0.0)
    mask = np.zeros((L, L), dtype=bool)
    for rr in range(L):
        i = rr // B
        mask[rr, :B] = True
        mask[rr, i * B: rr + 1] = True
        mask[rr, rr + 1:] = False
    ref = sdpa(q, expand_kv(k, 2), expand_kv(v, 2), mask=mask)
    np.testing.assert_allclose(out["o"], ref, rtol=1e-12, atol=1e-12)
    # two recency blocks: block i-1 joins
    out2 = oracle.prefill(q, k, v, B, top_p=0.0, n_recent=2)
    for i in range(L // B):
        assert list(out2["kept"][0][i]) == sorted({0, max(i - 1, 0), i})


# ----------------------------------------------------------------- block score closed form
@pytest.mark.parametrize("B,G", [(1, 1), (1, 2), (8, 2), (16, 4)])
def test_meanpool_score_is_block_average_of_token_logits(B, G):
    """mean(q) . mean(k) is the average of q_r . k_t over the block pair, so the
    pooled score equals the block-average of the library's token logits."""
    r = _rng(B * 10 + G)
    hkv, L, d = 2, 64, 8
    hq = hkv * G
    q, k = r.standard_normal((hq, L, d)), r.standard_normal((hkv, L, d))
    scale = 0.37
    qbar, kn, kp = oracle.pool_blocks(q, k, B)
    s = oracle.meanpool_scores(qbar, kn, kp, B, 0, scale)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    nb = L // B
    for g in range(hkv):
        logits = scale * (tq[g * G:(g + 1) * G] @ tk[g].T)          # (G, L, L)
        blk = logits.reshape(G, nb, B, nb, B).mean(dim=(0, 2, 4)).numpy()
        tril = np.tril(np.ones((nb, nb), dtype=bool))
        np.testing.assert_allclose(s[g][tril], blk[tril], rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(s[g][~tril]))


def test_meanpool_score_uses_permuted_keys_for_history():
    r = _rng(8)
    hkv, G, L, d, B, S = 1, 2, 64, 4, 8, 32
    q, k = r.standard_normal((hkv * G, L, d)), r.standard_normal((hkv, L, d))
    perm = _random_segment_perm(r, hkv, L, S)
    qbar, kn, kp = oracle.pool_blocks(q, k, B, perm)
    s = oracle.meanpool_scores(qbar, kn, kp, B, S, 1.0)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    for i in range(L // B):
        for j in range(i + 1):
            hist = (j * B) // S < (i * B) // S
            rows_k = perm[0, j * B:(j + 1) * B] if hist else np.arange(j * B, (j + 1) * B)
            ref = (tq[:, i * B:(i + 1) * B] @ tk[0, rows_k].T).mean().item()
            assert abs(s[0, i, j] - ref) < 1e-12


# ----------------------------------------------------------------- selection
def _brute_force_keep(scores, forced, p):
    resid = [j for j in range(len(scores)) if not forced[j]]
    if not resid:
        return sorted(j for j in range(len(scores)) if forced[j])
    sr = np.array([scores[j] for j in resid])
    w = np.exp(sr - sr.max())
    pi = dict(zip(resid, w / w.sum()))
    best = None
    for n in range(0, len(resid) + 1):
        cands = []
        for sub in itertools.combinations(resid, n):
            mass = sum(pi[j] for j in sub)
            if mass >= p:
                cands.append((mass, sub))
        if cands:
            top = max(m for m, _ in cands)
            ties = sorted(sub for m, sub in cands if m == top)
            best = ties[0]
            break
    return sorted(set(best) | {j for j in range(len(scores)) if forced[j]})


@pytest.mark.parametrize("seed", range(40))
def test_topp_matches_brute_force(seed):
    r = _rng(1000 + seed)
    n = int(r.integers(1, 13))
    scores = r.standard_normal(n) * r.choice([0.1, 1.0, 3.0])
    if seed % 4 == 0:                      # exact ties
        scores = np.round(scores, 0)
    forced = r.random(n) < 0.25
    p = float(r.choice([0.05, 0.3, 0.5, 0.75, 0.9, 0.97]))
    # keep the draw off the float boundary: no subset mass within 1e-9 of p
    resid = [j for j in range(n) if not forced[j]]
    if resid:
        sr = scores[resid]
        w = np.exp(sr - sr.max())
        pis = w / w.sum()
        for m in range(len(resid) + 1):
            for sub in itertools.combinations(range(len(resid)), m):
                if abs(pis[list(sub)].sum() - p) < 1e-9:
                    pytest.skip("draw on the float boundary")
    got = oracle.topp_keep(scores, forced, p, 0)
    assert list(got) == _brute_force_keep(scores, forced, p)


def test_topp_constant_scores_closed_form():
    """Q = 0 makes every block score 0: uniform residual mass 1/n, so
    ceil(p*n) residual blocks are kept, lowest indices first."""
    L, B, d = 192, 16, 8
    r = _rng(2)
    q = np.zeros((2, L, d))
    k, v = r.standard_normal((1, L, d)), r.standard_normal((1, L, d))
    p = 0.85
    out = oracle.prefill(q, k, v, B, top_p=p)
    for i in range(L // B):
        resid = [j for j in range(i + 1) if not (j < 1 or j > i - 1)]
        n = len(resid)
        kk = math.ceil(p * n)
        assert list(out["kept"][0][i]) == sorted({0, i} | set(resid[:kk]))


def test_topp_extremes_and_floor():
    s = np.array([0.0, 5.0, 4.0, 3.0, 2.0, 1.0, 0.5])
    f = np.array([True] + [False] * 5 + [True])
    assert list(oracle.topp_keep(s, f, 1.0, 0)) == list(range(7))
    assert list(oracle.topp_keep(s, f, 0.0, 0)) == [0, 6]
    assert list(oracle.topp_keep(s, f, 0.0, 2)) == [0, 1, 2, 6]
    assert list(oracle.topp_keep(s, f, 0.0, 99)) == list(range(7))
    # one dominant block carries the mass
    assert list(oracle.topp_keep(s, f, 0.5, 0)) == [0, 1, 6]
    # the crossing is inclusive: equal scores give exact masses 1/4, so mass
    # 1/2 is reached (not exceeded) by two blocks, which is where selection stops
    eq = np.zeros(6)
    fe = np.array([True, False, False, False, False, True])
    assert list(oracle.topp_keep(eq, fe, 0.5, 0)) == [0, 1, 2, 5]
    assert list(oracle.topp_keep(eq, fe, 0.25, 0)) == [0, 1, 5]


# ----------------------------------------------------------------- indexer score
def test_indexer_special_cases():
    r = _rng(4)
    nt, h_idx, d_idx = 50, 4, 16
    qI = r.standard_normal((h_idx, d_idx))
    kI = r.standard_normal((nt, h_idx, d_idx))
    # one head, unit weight: ReLU(q . k) (library relu of a library matmul)
    s1 = oracle.indexer_scores(qI[:1], np.ones(1), kI[:, :1])
    ref = torch.relu(torch.from_numpy(kI[:, 0]) @ torch.from_numpy(qI[0])).numpy()
    np.testing.assert_allclose(s1, ref, rtol=1e-13, atol=1e-13)
    # one-hot weight picks a single head
    for h in range(h_idx):
        w = np.zeros(h_idx)
        w[h] = 1.0
        sh = oracle.indexer_scores(qI, w, kI)
        ref = torch.relu(torch.from_numpy(kI[:, h]) @ torch.from_numpy(qI[h])).numpy()
        np.testing.assert_allclose(sh, ref, rtol=1e-13, atol=1e-13)
    # hand example: ReLU acts on each head's dot before weighting
    qh = np.array([[1.0, 2.0], [1.0, -1.0]])
    kh = np.array([[[3.0, -1.0], [1.0, 3.0]]])    # dots: 1 and -2
    assert oracle.indexer_scores(qh, np.array([0.25, 0.75]), kh)[0] == 0.25
    # a negative mixing weight subtracts the clipped dot (ReLU before weighting)
    assert oracle.indexer_scores(qh, np.array([-1.0, 0.5]), kh)[0] == -1.0
    # weights are linear: scores of w1 + w2 = sum of scores
    w1, w2 = r.random(h_idx), r.random(h_idx)
    np.testing.assert_allclose(oracle.indexer_scores(qI, w1 + w2, kI),
                               oracle.indexer_scores(qI, w1, kI) + oracle.indexer_scores(qI, w2, kI),
                               rtol=1e-12)


# ----------------------------------------------------------------- decode
@pytest.mark.parametrize("T", [160, 157])
def test_decode_keep_all_is_last_row_of_dense(T):
    r = _rng(T)
    hq, hkv, d, B = 4, 2, 8, 16
    kc, vc = r.standard_normal((hkv, T, d)), r.standard_normal((hkv, T, d))
    q = r.standard_normal((hq, d))
    nt = -(-T // B)
    o, lse = oracle.attend_decode(q, kc, vc, np.arange(nt), B, T, 1 / math.sqrt(d))
    ref = sdpa(q[:, None], expand_kv(kc, 2), expand_kv(vc, 2))[:, 0]
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # the prefill oracle's last row with the same keys
    qq = np.zeros((hq, T, d))
    qq[:, T - 1] = q
    op, lp = oracle.attend_prefill(qq, kc, vc, [{(T - 1) // B: np.arange(nt)} for _ in range(hkv)], B,
                                   1 / math.sqrt(d), qblocks=[(T - 1) // B])
    np.testing.assert_allclose(o, op[:, T - 1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lp[:, T - 1], rtol=1e-12, atol=1e-12)


def _decode_reserved(nt, n_sink, n_recent):
    """Reserved blocks of a decode row written from the dual top-p rule's
    definition (SpotAttention §3, reserved blocks): the first n_sink blocks
    of the context and its last n_recent blocks."""
    return set(range(min(n_sink, nt))) | set(range(max(nt - n_recent, 0), nt))


@pytest.mark.parametrize("n_sink,n_recent", [(1, 1), (2, 1), (1, 2), (0, 1), (1, 0), (3, 2)])
@pytest.mark.parametrize("nt", [12, 23])
def test_decode_reserved_blocks_closed_form(n_sink, n_recent, nt):
    """Indexer dots all <= 0 make every decode score exactly 0 (ReLU), so the
    residual distribution is uniform (1/n each): the kept set is the reserved
    blocks plus the ceil(p*n) lowest residual ids.  Several p off the 1/n grid
    make a sink or recency window one block too wide or too narrow change the
    kept set; the output must be library attention over exactly those keys."""
    r = _rng(40 + 7 * n_sink + n_recent + nt)
    B, h_idx, d_idx, hq, hkv, d = 16, 2, 8, 4, 2, 8
    T = nt * B - 5                                   # ragged last block
    qI = np.abs(r.standard_normal((h_idx, d_idx))) + 0.1
    kI = -np.abs(r.standard_normal((nt, h_idx, d_idx)))
    w = np.array([0.4, 0.6])
    kc, vc = r.standard_normal((hkv, T, d)), r.standard_normal((hkv, T, d))
    q = r.standard_normal((hq, d))
    reserved = _decode_reserved(nt, n_sink, n_recent)
    resid = [t for t in range(nt) if t not in reserved]
    n = len(resid)
    for p in (0.13, 0.37, 0.62, 0.87):
        assert abs(p * n - round(p * n)) > 1e-6         # off the 1/n grid
        out = oracle.decode(q, kc, vc, qI, w, kI, B, T, top_p=p, n_sink=n_sink, n_recent=n_recent)
        assert np.all(out["scores"] == 0.0)
        want = sorted(reserved | set(resid[:math.ceil(p * n)]))
        assert list(out["kept"]) == want, (p, n_sink, n_recent)
        mask = np.zeros((1, T), dtype=bool)
        for t in want:
            mask[0, t * B: min(T, (t + 1) * B)] = True
        ref = sdpa(q[:, None], np.repeat(kc, 2, 0), np.repeat(vc, 2, 0), mask=np.repeat(mask[None], hq, 0))
        np.testing.assert_allclose(out["o"], ref[:, 0], rtol=1e-12, atol=1e-12)
    # p <= 0 keeps the reserved blocks only; p >= 1 keeps every block
    assert list(oracle.select_decode(np.zeros(nt), n_sink, n_recent, 0.0, 0)) == sorted(reserved)
    assert list(oracle.select_decode(np.zeros(nt), n_sink, n_recent, 1.0, 0)) == list(range(nt))


@pytest.mark.parametrize("seed", range(24))
def test_decode_select_matches_brute_force(seed):
    """Decode rows of at most 14 blocks with random sink / recency sizes:
    the oracle's selection equals the smallest subset of the residual blocks
    reaching mass p (largest mass, then lowest ids), plus the reserved blocks
    written from their definition."""
    r = _rng(3000 + seed)
    nt = int(r.integers(2, 15))
    n_sink, n_recent = int(r.integers(0, 4)), int(r.integers(0, 4))
    if n_sink + n_recent == 0:
        n_recent = 1
    scores = r.standard_normal(nt) * r.choice([0.3, 1.0, 3.0])
    if seed % 3 == 0:
        scores = np.maximum(np.round(scores, 0), 0.0)   # ReLU-like ties at zero
    p = float(r.choice([0.2, 0.45, 0.7, 0.9]))
    reserved = _decode_reserved(nt, n_sink, n_recent)
    forced = np.array([t in reserved for t in range(nt)])
    resid = [t for t in range(nt) if not forced[t]]
    if resid:
        sr = scores[resid]
        e = np.exp(sr - sr.max())
        pis = e / e.sum()
        for m in range(len(resid) + 1):
            for sub in itertools.combinations(range(len(resid)), m):
                if abs(pis[list(sub)].sum() - p) < 1e-9:
                    pytest.skip("draw on the float boundary")
    got = oracle.select_decode(scores, n_sink, n_recent, p, 0)
    assert list(got) == _brute_force_keep(scores, forced, p)


def test_decode_sparse_is_masked_library_attention():
    r = _rng(9)
    hq, hkv, d, B, T = 4, 1, 8, 16, 200
    kc, vc = r.standard_normal((hkv, T, d)), r.standard_normal((hkv, T, d))
    q = r.standard_normal((hq, d))
    qI, w, kI = r.standard_normal((2, 8)), np.array([0.3, 0.7]), r.standard_normal((13, 2, 8))
    out = oracle.decode(q, kc, vc, qI, w, kI, B, T, top_p=0.6)
    mask = np.zeros((1, T), dtype=bool)
    for t in out["kept"]:
        mask[0, t * B: min(T, (t + 1) * B)] = True
    assert mask[0, :B].all() and mask[0, 12 * B:].all()       # sink and last block forced
    ref = sdpa(q[:, None], np.repeat(kc, hq, 0), np.repeat(vc, hq, 0), mask=np.repeat(mask[None], hq, 0))
    np.testing.assert_allclose(out["o"], ref[:, 0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- key permutation
def test_key_permutation_invariants():
    r = _rng(21)
    hq, hkv, L, d, B, S = 4, 2, 256, 16, 32, 64
    q, k = r.standard_normal((hq, L, d)), r.standard_normal((hkv, L, d))
    # plant one dominant key per segment aligned with the last block's queries
    u = q[0, -B:].mean(axis=0)
    u /= np.linalg.norm(u)
    hot = [10, 100, 150, 200]
    for t in hot:
        k[:, t] = 12.0 * u
    perm, imp = oracle.key_permutation(q, k, B, S, 1 / math.sqrt(d))
    np.testing.assert_allclose(imp.sum(axis=1), 1.0, rtol=1e-12)        # mean of distributions
    for g in range(hkv):
        for s0 in range(0, L, S):
            seg = perm[g, s0:s0 + S]
            assert sorted(seg) == list(range(s0, s0 + S))               # bijection onto the segment
            assert np.all(np.diff(imp[g, seg]) <= 0)                    # importance non-increasing
        for t in hot:
            assert perm[g, (t // S) * S] == t                            # heavy key leads its segment
    # importance against library softmax of the masked last-block logits
    rows = np.arange(L - B, L)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    for g in range(hkv):
        lg = (tq[2 * g:2 * g + 2, rows] @ tk[g].T) / math.sqrt(d)
        lg = lg.masked_fill(torch.from_numpy(np.arange(L)[None, :] > rows[:, None]), -math.inf)
        ref = torch.softmax(lg, -1).mean(dim=(0, 1)).numpy()
        np.testing.assert_allclose(imp[g], ref, rtol=1e-10, atol=1e-15)


# ----------------------------------------------------------------- generators
def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, -3.0 - 2 ** -7, 2 ** -130], np.float32)
    got = I.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got, ref)
    y = _rng(0).standard_normal(100000).astype(np.float32)
    np.testing.assert_array_equal(I.round_bf16(y), torch.from_numpy(y).to(torch.bfloat16).float().numpy())


def test_heavy_hitters_planted():
    cfg = I.small_prefill(L=500, hq=4, hkv=2, d=16, heavy_hitters=True, seed=3)
    q, k, v = I.prefill_inputs(cfg)
    pos, u = I.heavy_hitter_plan(cfg.seed, cfg.L, cfg.d)
    assert len(pos) == 10
    rows = k[0, :, pos].astype(np.float64)
    cos = rows @ u / np.linalg.norm(rows, axis=-1)
    assert np.all(cos > 0.999)
