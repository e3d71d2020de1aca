"""Float64 CPU oracle for block-sparse causal attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import or call this module; the product
path never does.  It shares no code with the HIP library and imports nothing
from it (nor from torch).

Everything here is plain NumPy in float64.  Inputs are the exact values the
GPU receives (bf16 or fp32 bit patterns widened exactly to float64).

Page key (titles of the five summarised papers):
  [Spot]  SpotAttention: Plug-In Block-Sparse Routing for Pretrained
          Long-Context Transformers
  [PBS]   Sparsere Blok-Sparse Attention via Tokenpermutatie (PBS-Attn)
  [S2O]   S2O - Vroege Stoppering voor Sparse Attention via Online Permutatie
  [SPLA]  SPLA - Block Sparse Plus Linear Attention

What each function follows:
  pool_blocks        [PBS] §4 (mean pooling for block selection, on permuted keys)
  meanpool_scores    [PBS] §4 with the attention scale; [Spot] §1 (score every
                     previous block)
  topp_keep          [Spot] §3 Dual top-p rule (reserved sink/recency blocks,
                     nucleus on the residual distribution, stop once the mass
                     reaches p, floor K_min)
  indexer_scores     [Spot] §1 scoring equation (head-weighted ReLU of q.k)
  mxfp4_quantize,    [Spot] §4 (selector K-cache in FP4 microscaling); the
  mxfp4_dequantize   format is the OCP Microscaling (MX) v1.0 MXFP4 element
                     and scale encoding: FP4 E2M1 elements, one E8M0
                     power-of-two scale per 32 elements
  int4_quantize,     [Spot] §4 (selector K-cache in INT4 microscaling): groups
  int4_dequantize    of 32 elements with one bf16 scale max|x|/7, elements
                     rounded to integers in [-7, 7], ties to even
  key_block_variance [SPLA] §2.1 (block statistics: per-dimension variance,
                     the diagonal of the block covariance)
  taylor_scores      [SPLA] §2.1 second-order Taylor block score, as a log mass
  attend_prefill     [PBS] Problem + §2 (block-sparse attention, segment-local
                     causality), [S2O] §1 (index-array loads) and §3 (own
                     segment as a dense causal window, history through the
                     permutation)
  attend_decode      [Spot] Problem (decode re-reads the KV cache): one query at
                     the last position, softmax over the kept blocks
  key_permutation    [PBS] §3 (importance from the last query block by mean
                     pooling of attention, keys sorted descending per segment)
  history_order      [S2O] §2 (candidate blocks visited in descending estimated
                     importance)
  representative_queries, history_map
                     [S2O] §1 (historical keys scored against a representative
                     query of the segment, prefix only; the sorted positions
                     form the segment's logical map of its history)
  attend_prefill_es  [S2O] §2 (monotone-gain early stopping) and §3 (dense
                     causal pass over the own segment, then the permuted
                     history in that order, resuming the same softmax state)
  rla_prefill,       [SPLA] §2.2 (residual linear attention: the long tail
  rla_decode         outside the kept blocks through linear attention) and
                     §2.3 (parameter-free exponential feature map)

Readings taken where the pages leave a step open (each is also listed with the
design notes): the block distribution for top-p is the softmax of the block
scores over the residual candidates; the mean-pool score carries the attention
scale 1/sqrt(d); one kept list per KV head (queries pooled over the group);
crossing is inclusive; ties go to the lower block index; p >= 1 keeps every
residual block and p <= 0 keeps none; history blocks (earlier segments) are
read through the permutation and fully visible, blocks of the query's own
segment are read in natural order under the positional causal mask.
Early stopping: the stop rule is applied per query row; the marginal gain of a
history block is the softmax mass its keys add and it is compared with the
mass accumulated including that block (stop once gain < tau * accumulated);
the block that triggers the stop is kept.
MXFP4: the shared exponent is floor(log2(max |x|)) - 2 (the largest E2M1
exponent), clamped to the E8M0 range, -127 for an all-zero group; elements
are rounded to the nearest E2M1 value, ties to the even code, and saturate at
6; the sign bit is the input's sign bit (so -0 keeps its sign).
INT4: symmetric integers in [-7, 7] with one scale per 32 elements, the
scale being max|x| / 7 rounded to bf16 (4.5 bits per element, 16 / 4.5 =
3.56x smaller than bf16, the page's "about 3.5x"); x / scale rounded to the
nearest integer with ties to the even one, clamped; an all-zero group has
scale 0 and codes 0.
Representative query: the mean of Q over the group's heads and the segment's
rows; the history map sorts the prefix by sm_scale * <representative, key>
descending, ties by position; early-stopped attention on the map visits its
consecutive runs of B positions in order.
Residual linear attention: phi(x) = exp(x) elementwise on the raw query and
key rows (no scale); the linear attention carries no normaliser, so the
page's difference of the all-blocks and kept-blocks estimates is exactly the
linear attention over the keys outside the kept blocks (normalisation is the
RMS norm the page applies afterwards, with trained scales: not part of this
output); the keys are the causally visible ones, {t <= r}, in prefill and
every cached key in decode.
Taylor score: the second-order expansion is taken for the scaled query
(sm_scale * qbar) and enters the top-p rule as the log of the estimated block
mass, so the softmax over blocks is the normalised mass estimate; variances
are population variances (divide by the block's row count).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- helpers
def n_blocks(n: int, block: int) -> int:
    return -(-n // block)


def block_rows(j: int, block: int, n: int) -> np.ndarray:
    """Token positions of block j: [jB, min((j+1)B, n))."""
    return np.arange(j * block, min((j + 1) * block, n))


def is_history(j: int, i: int, block: int, segment: int) -> bool:
    """Key block j lies in a segment strictly before query block i's segment."""
    if segment <= 0:
        return False
    return (j * block) // segment < (i * block) // segment


# ----------------------------------------------------------------- O1 pool
def pool_blocks(q, k, block, perm=None):
    """Per-block means ([PBS] §4).

    q: (Hq, L, d), k: (Hkv, L, d), perm: (Hkv, L) int or None.
    Returns qbar (Hkv, nB, d): mean of Q over the G heads of the group and the
    rows of the block; kbar_nat (Hkv, nB, d): mean of the block's K rows in
    natural order; kbar_perm: mean of the K rows the permutation maps the
    block's positions to (equal to kbar_nat without a permutation).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, L, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    nb = n_blocks(L, block)
    qbar = np.empty((hkv, nb, d))
    kn = np.empty((hkv, nb, d))
    kp = np.empty((hkv, nb, d))
    for g in range(hkv):
        for i in range(nb):
            rows = block_rows(i, block, L)
            qbar[g, i] = q[g * G:(g + 1) * G, rows].mean(axis=(0, 1))
            kn[g, i] = k[g, rows].mean(axis=0)
            kp[g, i] = k[g, perm[g, rows]].mean(axis=0) if perm is not None else kn[g, i]
    return qbar, kn, kp


# ----------------------------------------------------------------- O2 score
def meanpool_scores(qbar, kbar_nat, kbar_perm, block, segment, sm_scale):
    """s[g, i, j] = sm_scale * <qbar[g,i], kbar[g,j]> for j <= i, -inf for j > i.

    kbar is the permuted-key mean for blocks of earlier segments and the
    natural one otherwise ([PBS] §4 scores blocks of the permuted keys; the
    query's own segment is read unpermuted, [S2O] §3).
    """
    hkv, nb, _ = qbar.shape
    s = np.full((hkv, nb, nb), -np.inf)
    for g in range(hkv):
        for i in range(nb):
            js = np.arange(i + 1)
            hist = np.array([is_history(j, i, block, segment) for j in js], dtype=bool)
            kb = np.where(hist[:, None], kbar_perm[g, :i + 1], kbar_nat[g, :i + 1])
            s[g, i, :i + 1] = sm_scale * (kb @ qbar[g, i])
    return s


def key_block_variance(k, block, perm=None):
    """[SPLA] §2.1: per-dimension variance of the K rows of every block
    (natural order, and through the permutation), divided by the row count.

    k: (Hkv, L, d).  Returns var_nat, var_perm (Hkv, nB, d).
    """
    k = np.asarray(k, dtype=np.float64)
    hkv, L, d = k.shape
    nb = n_blocks(L, block)
    vn = np.empty((hkv, nb, d))
    vp = np.empty((hkv, nb, d))
    for g in range(hkv):
        for j in range(nb):
            rows = block_rows(j, block, L)
            x = k[g, rows]
            vn[g, j] = ((x - x.mean(axis=0)) ** 2).mean(axis=0)
            if perm is not None:
                y = k[g, perm[g, rows]]
                vp[g, j] = ((y - y.mean(axis=0)) ** 2).mean(axis=0)
            else:
                vp[g, j] = vn[g, j]
    return vn, vp


def taylor_scores(qbar, kbar_nat, kbar_perm, var_nat, var_perm, block, segment, sm_scale):
    """[SPLA] §2.1: the block mass E_t[exp(x . k_t)] of the scaled pooled query
    x = sm_scale * qbar, expanded to second order around the block mean with a
    diagonal covariance: exp(x . kbar) * (1 + 1/2 * sum_d x_d^2 var_d).
    Returned as its logarithm for j <= i (-inf for j > i); history blocks use
    the permuted statistics as in meanpool_scores."""
    hkv, nb, _ = qbar.shape
    s = np.full((hkv, nb, nb), -np.inf)
    for g in range(hkv):
        for i in range(nb):
            js = np.arange(i + 1)
            hist = np.array([is_history(j, i, block, segment) for j in js], dtype=bool)
            kb = np.where(hist[:, None], kbar_perm[g, :i + 1], kbar_nat[g, :i + 1])
            vb = np.where(hist[:, None], var_perm[g, :i + 1], var_nat[g, :i + 1])
            x = sm_scale * qbar[g, i]
            s[g, i, :i + 1] = kb @ x + np.log(1.0 + 0.5 * (vb @ (x * x)))
    return s


# ----------------------------------------------------------------- MXFP4 indexer keys
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)   # codes 0..7; bit 3 is the sign
MX_GROUP = 32


def mxfp4_quantize(x):
    """[Spot] §4 FP4 microscaling of the selector keys.

    x: (..., n) with n a multiple of 32, groups of 32 consecutive elements.
    Returns codes uint8 (..., n), one 4-bit code per element (sign << 3 |
    magnitude index into E2M1_MAGNITUDES), and scale bytes uint8
    (..., n // 32): the group scale is 2 ** (byte - 127).
    """
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    g = x.reshape(-1, MX_GROUP)
    grid = np.array(E2M1_MAGNITUDES)
    even = (np.arange(len(grid)) % 2 == 0)
    codes = np.zeros(g.shape, dtype=np.uint8)
    scales = np.zeros(g.shape[0], dtype=np.uint8)
    for r0 in range(0, g.shape[0], 1 << 14):          # groups in chunks (memory only)
        gc = g[r0:r0 + (1 << 14)]
        amax = np.abs(gc).max(axis=1)
        _, ex = np.frexp(amax)                           # amax = m * 2**ex, 0.5 <= m < 1
        e = np.where(amax == 0, -127, np.clip(ex.astype(np.int64) - 1 - 2, -127, 127))   # floor(log2) - 2
        scales[r0:r0 + len(gc)] = (e + 127).astype(np.uint8)
        y = gc / np.exp2(e.astype(np.float64))[:, None]
        a = np.abs(y)
        dist = np.abs(grid[None, None, :] - a[..., None])
        nearest = dist == dist.min(axis=-1, keepdims=True)
        # the nearest value; of two equally near, the one with the even code
        m = np.where((nearest & even).any(axis=-1), np.argmax(nearest & even, axis=-1), np.argmax(nearest, axis=-1))
        m = np.where(a >= grid[-1], len(grid) - 1, m)
        codes[r0:r0 + len(gc)] = (np.where(np.signbit(y), 8, 0) | m).astype(np.uint8)
    return codes.reshape(shape), scales.reshape(shape[:-1] + (shape[-1] // MX_GROUP,))


def mxfp4_dequantize(codes, scales):
    """Values of MXFP4 codes: (-1)^sign * E2M1 magnitude * 2 ** (scale - 127)."""
    codes = np.asarray(codes)
    mag = np.array(E2M1_MAGNITUDES)[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    sc = 2.0 ** (np.repeat(np.asarray(scales, dtype=np.float64), MX_GROUP, axis=-1) - 127.0)
    return sign * mag * sc


def mxfp4_pack(codes):
    """Two codes per byte: element 2k in the low nibble, 2k+1 in the high one."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_unpack(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


# ----------------------------------------------------------------- INT4 indexer keys
INT4_GROUP = 32
INT4_MAX = 7


def _round_bf16(x):
    """float64 values rounded to the nearest bf16 value (8 significant bits), ties to even; bf16 has the
    float32 exponent range, so below 2^-126 the spacing stays 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                                  # a = m * 2**ex, 0.5 <= m < 1
    ulp = np.exp2(np.maximum(ex.astype(np.float64) - 8.0, -133.0))
    r = np.rint(a / ulp) * ulp                           # a / ulp is exact; rint: ties to even
    return np.where(a == 0, 0.0, np.sign(x) * r)


def int4_quantize(x):
    """[Spot] §4 INT4 microscaling of the selector keys.

    Groups of 32 consecutive elements share one scale s = max|x| / 7 rounded to
    bf16; each element is round(x / s) to the nearest integer (ties to the even
    one), clamped to [-7, 7] (0 for an all-zero group, whose scale is 0).
    x: (..., n) with n a multiple of 32.  Returns codes int8 (..., n) and scales
    float64 (..., n // 32) holding bf16 values.
    """
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    g = x.reshape(-1, INT4_GROUP)
    scales = _round_bf16(np.abs(g).max(axis=1) / INT4_MAX)
    safe = np.where(scales > 0, scales, 1.0)
    codes = np.clip(np.rint(g / safe[:, None]), -INT4_MAX, INT4_MAX)
    codes = np.where(scales[:, None] > 0, codes, 0.0).astype(np.int8)
    return codes.reshape(shape), scales.reshape(shape[:-1] + (shape[-1] // INT4_GROUP,))


def int4_dequantize(codes, scales):
    """Values of INT4 codes: code * scale of its group."""
    codes = np.asarray(codes, dtype=np.float64)
    return codes * np.repeat(np.asarray(scales, dtype=np.float64), INT4_GROUP, axis=-1)


def int4_pack(codes):
    """Two 4-bit two's-complement codes per byte: element 2k in the low nibble, 2k+1 in the high one."""
    u = (np.asarray(codes, dtype=np.int16) & 15).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


# ----------------------------------------------------------------- D1 indexer score
def indexer_scores(idx_q, idx_w, idx_k):
    """[Spot] §1: s[t] = sum_h w_h * ReLU(q^I_h . k^I_{h,t}).

    idx_q: (H_idx, d_idx), idx_w: (H_idx,), idx_k: (nT, H_idx, d_idx) -> (nT,)
    """
    idx_q = np.asarray(idx_q, dtype=np.float64)
    idx_w = np.asarray(idx_w, dtype=np.float64)
    idx_k = np.asarray(idx_k, dtype=np.float64)
    nt, h_idx, _ = idx_k.shape
    s = np.zeros(nt)
    for h in range(h_idx):
        dots = idx_k[:, h, :] @ idx_q[h]
        s += idx_w[h] * np.maximum(dots, 0.0)
    return s


# ----------------------------------------------------------------- O3 select
def topp_detail(scores, forced, top_p, k_min):
    """[Spot] §3 dual top-p on one row; returns the steps for inspection.

    scores: (n,) candidate scores; forced: (n,) bool (sink and recency blocks).
    Residual R = candidates not forced, ordered by (score desc, index asc);
    pi = softmax over R; c_k = sum of the first k of pi (c_0 = 0);
    k* = min{k >= 0 : c_k >= p}, raised to min(K_min, |R|); p >= 1 keeps R.
    """
    scores = np.asarray(scores, dtype=np.float64)
    forced = np.asarray(forced, dtype=bool)
    cand = np.arange(scores.shape[0])
    resid = cand[~forced]
    order = resid[np.lexsort((resid, -scores[resid]))]
    n = order.shape[0]
    if n:
        sr = scores[order]
        e = np.exp(sr - sr[0])
        pi = e / e.sum()
        c = np.cumsum(pi)
    else:
        pi = np.zeros(0)
        c = np.zeros(0)
    if top_p >= 1.0:
        kstar = n
    elif top_p <= 0.0:
        kstar = 0
    else:
        hit = np.nonzero(c >= top_p)[0]
        kstar = int(hit[0]) + 1 if hit.size else n
    kstar = max(kstar, min(int(k_min), n))
    kept = np.sort(np.concatenate([cand[forced], order[:kstar]])).astype(np.int64)
    return dict(kept=kept, order=order, pi=pi, cum=c, kstar=kstar)


def topp_keep(scores, forced, top_p, k_min):
    return topp_detail(scores, forced, top_p, k_min)["kept"]


def prefill_forced(i, n_sink, n_recent):
    """Sink blocks j < n_sink and recency blocks i - n_recent < j <= i."""
    js = np.arange(i + 1)
    return (js < n_sink) | (js > i - n_recent)


def decode_forced(nt, n_sink, n_recent):
    ts = np.arange(nt)
    return (ts < n_sink) | (ts > nt - 1 - n_recent)


def select_prefill(scores, n_sink, n_recent, top_p, k_min, rows=None):
    """Kept block lists per (KV head, query block): list[g][i] -> sorted array."""
    hkv, nb, _ = scores.shape
    rows = range(nb) if rows is None else rows
    out = [dict() for _ in range(hkv)]
    for g in range(hkv):
        for i in rows:
            out[g][int(i)] = topp_keep(scores[g, i, :i + 1], prefill_forced(i, n_sink, n_recent),
                                       top_p, k_min)
    return out


def select_decode(scores, n_sink, n_recent, top_p, k_min):
    nt = scores.shape[0]
    return topp_keep(scores, decode_forced(nt, n_sink, n_recent), top_p, k_min)


# ----------------------------------------------------------------- O4 attend (prefill)
def prefill_key_set(kept, i, g, block, segment, perm, L):
    """Key rows and their logical positions for query block i.

    History blocks (earlier segments) contribute perm[g, t] for t in the
    block and are fully visible (logical position -1 marks 'always visible');
    own-segment blocks contribute their natural rows t, visible to row r iff
    t <= r.
    """
    phys, lim = [], []
    for j in kept:
        ts = block_rows(int(j), block, L)
        if perm is not None and is_history(int(j), i, block, segment):
            phys.append(perm[g, ts])
            lim.append(np.full(ts.shape, -1))
        else:
            phys.append(ts)
            lim.append(ts)
    return np.concatenate(phys), np.concatenate(lim)


def attend_prefill(q, k, v, kept_lists, block, sm_scale, segment=0, perm=None, qblocks=None):
    """Softmax attention of each query row over the union of its kept keys.

    q: (Hq, L, d); k, v: (Hkv, L, d); kept_lists[g][i] -> kept block indices.
    Returns O (Hq, L, d) and natural-log LSE (Hq, L); rows of query blocks
    not in `qblocks` are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, L, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    nb = n_blocks(L, block)
    qblocks = range(nb) if qblocks is None else qblocks
    o = np.full((hq, L, d), np.nan)
    lse = np.full((hq, L), np.nan)
    for g in range(hkv):
        for i in qblocks:
            i = int(i)
            rows = block_rows(i, block, L)
            phys, lim = prefill_key_set(kept_lists[g][i], i, g, block, segment, perm, L)
            visible = lim[None, :] <= rows[:, None]          # (rows, keys)
            ks, vs = k[g, phys], v[g, phys]
            for h in range(g * G, (g + 1) * G):
                logits = sm_scale * (q[h, rows] @ ks.T)
                logits = np.where(visible, logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                e = np.exp(logits - m)
                z = e.sum(axis=1, keepdims=True)
                o[h, rows] = (e @ vs) / z
                lse[h, rows] = (m + np.log(z))[:, 0]
    return o, lse


# ----------------------------------------------------------------- D3 attend (decode)
def attend_decode(q, k_cache, v_cache, kept, block, T, sm_scale):
    """One query at position T-1 per head over the keys of the kept blocks.

    q: (Hq, d); k_cache, v_cache: (Hkv, T, d); kept: block indices.
    Returns O (Hq, d) and LSE (Hq,).
    """
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_cache.shape[0]
    G = hq // hkv
    keys = np.concatenate([block_rows(int(t), block, T) for t in kept])
    o = np.empty((hq, d))
    lse = np.empty(hq)
    for g in range(hkv):
        ks = np.asarray(k_cache[g, keys], dtype=np.float64)
        vs = np.asarray(v_cache[g, keys], dtype=np.float64)
        for h in range(g * G, (g + 1) * G):
            logits = sm_scale * (ks @ q[h])
            m = logits.max()
            e = np.exp(logits - m)
            z = e.sum()
            o[h] = (e @ vs) / z
            lse[h] = m + np.log(z)
    return o, lse


# ----------------------------------------------------------------- residual linear attention
def rla_feature(x):
    """[SPLA] §2.3: the parameter-free exponential feature map, elementwise."""
    return np.exp(np.asarray(x, dtype=np.float64))


def rla_prefill(q, k, v, kept_lists, block, segment=0, perm=None, qblocks=None):
    """[SPLA] §2.2 residual linear attention of every query row.

    The row's linear attention (feature map phi = exp, no normaliser) over
    the causally visible keys that its kept blocks do not hold:
        o_rla[h, r] = sum over t <= r, t not a kept key of r, of
                      (phi(q[h, r]) . phi(k[g, t])) * v[g, t]
    (the keys of earlier segments are all visible whether or not the
    permutation reorders them, so the visible set is {t <= r} either way).
    q: (Hq, L, d); k, v: (Hkv, L, d).  Returns (Hq, L, d), rows of query
    blocks not in `qblocks` NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, L, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    nb = n_blocks(L, block)
    qblocks = range(nb) if qblocks is None else qblocks
    out = np.full((hq, L, d), np.nan)
    qblocks = [int(i) for i in qblocks]
    top = min(L, (max(qblocks) + 1) * block) if qblocks else 0   # no row of these blocks sees a key beyond
    for g in range(hkv):
        fk = rla_feature(k[g, :top])
        for i in qblocks:
            rows = block_rows(i, block, L)
            hi = rows[-1] + 1
            phys, lim = prefill_key_set(kept_lists[g][i], i, g, block, segment, perm, L)
            rest = np.arange(hi)[None, :] <= rows[:, None]              # visible keys of each row
            for r_idx, r in enumerate(rows):
                rest[r_idx, phys[lim <= r]] = False                     # minus the row's kept keys
            for h in range(g * G, (g + 1) * G):
                w = (rla_feature(q[h, rows]) @ fk[:hi].T) * rest        # (rows, keys up to the last row)
                out[h, rows] = w @ v[g, :hi]
    return out


def rla_decode(q, k_cache, v_cache, kept, block, T):
    """[SPLA] §2.2 residual linear attention of the decode query (position
    T-1, every cached key visible) over the keys outside the kept blocks.
    q: (Hq, d); k_cache, v_cache: (Hkv, T, d).  Returns (Hq, d)."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_cache.shape[0]
    G = hq // hkv
    rest = np.ones(T, dtype=bool)
    for t in kept:
        rest[block_rows(int(t), block, T)] = False
    out = np.empty((hq, d))
    for g in range(hkv):
        fk = rla_feature(np.asarray(k_cache[g, :T], dtype=np.float64)[rest])
        vs = np.asarray(v_cache[g, :T], dtype=np.float64)[rest]
        for h in range(g * G, (g + 1) * G):
            out[h] = (fk @ rla_feature(q[h])) @ vs
    return out


# ----------------------------------------------------------------- key permutation
def key_importance(q, k, block, sm_scale):
    """[PBS] §3: importance of every key from the last query block.

    For each KV head g: the causal attention probabilities of every query row
    r of the last block, for every head of the group, averaged (mean pooling)
    over those rows and heads.  Keys after r get probability 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, L, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    rows = block_rows(n_blocks(L, block) - 1, block, L)
    pos = np.arange(L)
    imp = np.zeros((hkv, L))
    for g in range(hkv):
        for h in range(g * G, (g + 1) * G):
            logits = sm_scale * (q[h, rows] @ k[g].T)
            logits = np.where(pos[None, :] <= rows[:, None], logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            imp[g] += (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
        imp[g] /= G * rows.shape[0]
    return imp


def key_permutation(q, k, block, segment, sm_scale):
    """[PBS] §2-3: inside each segment, positions sorted by importance
    descending (ties by position ascending).  perm[g, t] is the physical row
    that logical position t reads."""
    imp = key_importance(q, k, block, sm_scale)
    hkv, L = imp.shape
    perm = np.empty((hkv, L), dtype=np.int64)
    for g in range(hkv):
        for s0 in range(0, L, segment):
            ts = np.arange(s0, min(s0 + segment, L))
            perm[g, ts] = ts[np.lexsort((ts, -imp[g, ts]))]
    return perm, imp


# ----------------------------------------------------------------- early stopping
def history_order(scores, block, segment, rows=None):
    """[S2O] §2: the history blocks of query block i (those in segments
    before i's segment) in descending block score, ties by block index.

    scores: (Hkv, nB, nB).  Returns order[g][i] -> int array (empty for the
    first segment); entries for query blocks outside `rows` are None.
    """
    hkv, nb, _ = scores.shape
    rows = range(nb) if rows is None else rows
    order = [[None] * nb for _ in range(hkv)]
    for g in range(hkv):
        for i in rows:
            i = int(i)
            n_hist = ((i * block) // segment) * segment // block
            js = np.arange(n_hist)
            order[g][i] = js[np.lexsort((js, -np.asarray(scores[g, i, :n_hist], dtype=np.float64)))]
    return order


def _es_blocks(q, k, i, g, h, order_gi, block, segment, sm_scale, perm, hmap=None):
    """Masses of one query block's rows for head h, in one fixed frame.

    Returns (e_own, own_phys, e_hist, hist_phys, shift): e_own (rows, n_own)
    = exp(logit - shift) over the own-segment keys (0 where the causal mask
    hides the key), e_hist (rows, n_hist_blocks, B) the same for the history
    blocks in visiting order, shift (rows,) the row's largest visible logit.
    With `hmap` (the history maps of history_map), the history blocks are the
    consecutive runs of B positions of the segment's map, in map order, and
    `order_gi` and `perm` are not used.
    """
    L = q.shape[1]
    rows = block_rows(i, block, L)
    s0 = ((i * block) // segment) * segment
    own = np.arange(s0, min(rows[-1] + 1, L))
    if hmap is not None:
        hist = list(np.asarray(hmap[g, s0 // segment, :s0], dtype=np.int64).reshape(-1, block))
    else:
        hist = [perm[g, block_rows(int(j), block, L)] if perm is not None else block_rows(int(j), block, L)
                for j in order_gi]
    hist_phys = np.stack(hist) if hist else np.zeros((0, block), dtype=np.int64)
    lo = sm_scale * (q[h, rows] @ k[g, own].T)
    lo = np.where(own[None, :] <= rows[:, None], lo, -np.inf)
    lh = (sm_scale * (q[h, rows] @ k[g, hist_phys.reshape(-1)].T)).reshape(rows.shape[0], -1, block)
    shift = lo.max(axis=1)
    if hist:
        shift = np.maximum(shift, lh.max(axis=(1, 2)))
    return np.exp(lo - shift[:, None]), own, np.exp(lh - shift[:, None, None]), hist_phys, shift


def es_gain_ratios(q, k, i, g, h, order_gi, block, segment, sm_scale, perm=None, hmap=None):
    """[S2O] §2: for each row of query block i and head h, the marginal gain
    of each visited history block relative to the mass accumulated including
    it: ratio[r, n] = gain_n / (own mass + gain_1 + ... + gain_n)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    e_own, _, e_hist, _, _ = _es_blocks(q, k, i, g, h, order_gi, block, segment, sm_scale, perm, hmap)
    gain = e_hist.sum(axis=2)
    acc = e_own.sum(axis=1)[:, None] + np.cumsum(gain, axis=1)
    return gain / acc


def attend_prefill_es(q, k, v, order, block, segment, sm_scale, tau, perm=None, qblocks=None,
                      nused=None, hmap=None):
    """[S2O] §2-3 early-stopped attention for every query row.

    Pass 1: the row's own segment in natural order under the causal mask.
    Pass 2: the history blocks order[g][i] (rows through `perm`, all visible)
    one at a time; after each, the row stops once the block's gain is below
    tau times the mass accumulated so far (that block included).  The output
    is the softmax attention over the own-segment keys and the visited blocks.

    nused (Hq, L) int, optional: use these numbers of visited history blocks
    instead of the rule (to evaluate the output at another implementation's
    decisions).  With `hmap`, pass 2 visits the runs of B positions of the
    segment's history map (history_map) in order instead.  Returns O
    (Hq, L, d), LSE (Hq, L) and the numbers of visited history blocks
    (Hq, L); rows outside `qblocks` are NaN / -1.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, L, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    nb = n_blocks(L, block)
    qblocks = range(nb) if qblocks is None else qblocks
    o = np.full((hq, L, d), np.nan)
    lse = np.full((hq, L), np.nan)
    used = np.full((hq, L), -1, dtype=np.int64)
    for g in range(hkv):
        for i in qblocks:
            i = int(i)
            rows = block_rows(i, block, L)
            for h in range(g * G, (g + 1) * G):
                e_own, own, e_hist, hist_phys, shift = _es_blocks(
                    q, k, i, g, h, None if order is None else order[g][i], block, segment, sm_scale, perm, hmap)
                n_h = e_hist.shape[1]
                gain = e_hist.sum(axis=2)
                acc = e_own.sum(axis=1)[:, None] + np.cumsum(gain, axis=1)
                for ri, r in enumerate(rows):
                    if nused is not None:
                        n = int(nused[h, r])
                    else:
                        below = np.nonzero(gain[ri] < tau * acc[ri])[0]
                        n = int(below[0]) + 1 if below.size else n_h
                    z = e_own[ri].sum() + e_hist[ri, :n].sum()
                    num = e_own[ri] @ v[g, own]
                    if n:
                        num = num + e_hist[ri, :n].reshape(-1) @ v[g, hist_phys[:n].reshape(-1)]
                    o[h, r] = num / z
                    lse[h, r] = shift[ri] + np.log(z)
                    used[h, r] = n
    return o, lse, used


def representative_queries(q, hkv, segment):
    """[S2O] §1: per KV head g and segment s, the mean of Q over the G heads
    of the group and the rows of the segment.  q: (Hq, L, d) -> (Hkv, nseg, d)."""
    q = np.asarray(q, dtype=np.float64)
    hq, L, d = q.shape
    G = hq // hkv
    nseg = n_blocks(L, segment)
    rep_q = np.empty((hkv, nseg, d))
    for g in range(hkv):
        for sg in range(nseg):
            rep_q[g, sg] = q[g * G:(g + 1) * G, sg * segment:min((sg + 1) * segment, L)].mean(axis=(0, 1))
    return rep_q


def history_map(q, k, segment, sm_scale):
    """[S2O] §1: for KV head g and segment s >= 1, the prefix positions
    t < s*S sorted by sm_scale * <representative query of s, k_t> descending,
    ties by position ascending.

    Returns hmap (Hkv, nseg, L) int64 (entries t >= s*S are -1) and the
    scores (Hkv, nseg, L) (NaN outside the prefix)."""
    k = np.asarray(k, dtype=np.float64)
    hkv, L, _ = k.shape
    rep_q = representative_queries(q, hkv, segment)
    nseg = rep_q.shape[1]
    hmap = np.full((hkv, nseg, L), -1, dtype=np.int64)
    score = np.full((hkv, nseg, L), np.nan)
    for g in range(hkv):
        for sg in range(1, nseg):
            n = sg * segment
            c = sm_scale * (k[g, :n] @ rep_q[g, sg])
            ts = np.arange(n)
            hmap[g, sg, :n] = ts[np.lexsort((ts, -c))]
            score[g, sg, :n] = c
    return hmap, score


# ----------------------------------------------------------------- pipelines
def prefill(q, k, v, block, top_p, n_sink=1, n_recent=1, k_min=0, sm_scale=None,
            segment=0, perm=None, qblocks=None, score="meanpool"):
    """Whole prefill path for one sequence: pool -> score -> select -> attend.

    q: (Hq, L, d), k/v: (Hkv, L, d).  Returns dict with scores, kept lists,
    O and LSE (rows outside `qblocks` NaN).
    """
    d = q.shape[-1]
    sm_scale = 1.0 / np.sqrt(d) if not sm_scale else sm_scale
    qbar, kn, kp = pool_blocks(q, k, block, perm)
    if score == "taylor":
        vn, vp = key_block_variance(k, block, perm)
        s = taylor_scores(qbar, kn, kp, vn, vp, block, segment, sm_scale)
    else:
        s = meanpool_scores(qbar, kn, kp, block, segment, sm_scale)
    kept = select_prefill(s, n_sink, n_recent, top_p, k_min, rows=qblocks)
    o, lse = attend_prefill(q, k, v, kept, block, sm_scale, segment, perm, qblocks)
    return dict(scores=s, kept=kept, o=o, lse=lse, qbar=qbar, kbar_nat=kn, kbar_perm=kp)


def decode(q, k_cache, v_cache, idx_q, idx_w, idx_k, block, T, top_p, n_sink=1, n_recent=1,
           k_min=0, sm_scale=None, idx_format="bf16"):
    """Whole decode step for one sequence: indexer score -> select -> attend.
    idx_format "mxfp4" or "int4": the indexer keys are scored from that encoding."""
    d = q.shape[-1]
    sm_scale = 1.0 / np.sqrt(d) if not sm_scale else sm_scale
    if idx_format == "mxfp4":
        nt, h_idx, d_idx = idx_k.shape
        codes, scales = mxfp4_quantize(np.asarray(idx_k, dtype=np.float64).reshape(nt, h_idx * d_idx))
        idx_k = mxfp4_dequantize(codes, scales).reshape(nt, h_idx, d_idx)
    elif idx_format == "int4":
        nt, h_idx, d_idx = idx_k.shape
        codes, scales = int4_quantize(np.asarray(idx_k, dtype=np.float64).reshape(nt, h_idx * d_idx))
        idx_k = int4_dequantize(codes, scales).reshape(nt, h_idx, d_idx)
    s = indexer_scores(idx_q, idx_w, idx_k)
    kept = select_decode(s, n_sink, n_recent, top_p, k_min)
    o, lse = attend_decode(q, k_cache, v_cache, kept, block, T, sm_scale)
    return dict(scores=s, kept=kept, o=o, lse=lse)
