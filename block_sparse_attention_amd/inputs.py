"""Seeded synthetic inputs for block-sparse causal attention.

This module is the one piece shared by the HIP path and the float64 oracle.
It draws random numbers, rounds them to bf16 and assembles the synthetic
workloads; it contains no step of the attention method (no block score, no
top-p rule, no softmax over keys, no permutation by importance).

Recipe (stated once here, used by tests and the benchmark):

* Every tensor is drawn per (batch, head) slice from its own stream,
  ``numpy.random.default_rng([seed, tensor_code, b, h])`` with
  ``standard_normal(dtype=float32)``, so large inputs can be generated on
  several threads and any slice can be regenerated alone.
* bf16 tensors are the float32 draws rounded to nearest-even.
* Heavy hitters: ``round(0.02 * L)`` key positions, shared by every KV head,
  drawn without replacement; one unit direction ``u``; every planted key row is
  replaced by ``4 * ||row|| * u`` (queries untouched), then rounded.
* Decode indexer inputs: random projections of the decode query (for the
  indexer query and the softmax-normalised head weights) and of the 16-token
  block means of the KV cache (for the indexer key cache), each with
  N(0, 1/fan_in) entries, computed in float64 and rounded to bf16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# stream codes per tensor
_Q, _K, _V, _HH, _DQ, _WQI, _WW, _WKI = 1, 2, 3, 4, 5, 6, 7, 8


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------- bf16
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------- configs
@dataclass(frozen=True)
class PrefillConfig:
    name: str
    L: int
    hq: int
    hkv: int
    d: int
    dtype: str          # "f32" | "bf16"
    block: int
    top_p: float
    seed: int
    batch: int = 1
    heavy_hitters: bool = False
    segment: int = 0    # > 0: intra-segment key permutation of this size
    n_sink: int = 1
    n_recent: int = 1
    k_min: int = 0
    oracle_qblocks: int = 0   # > 0: the oracle checks this many seeded query blocks

    @property
    def nb(self) -> int:
        return -(-self.L // self.block)

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    T: int
    hq: int
    hkv: int
    d: int
    block: int
    h_idx: int
    d_idx: int
    top_p: float
    seed: int
    n_sink: int = 1
    n_recent: int = 1
    k_min: int = 0

    @property
    def nt(self) -> int:
        return -(-self.T // self.block)

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


# The five synthetic workloads (long-context shapes of the pages: 8K-128K).
C1 = PrefillConfig("tiny-fp32-L256", L=256, hq=1, hkv=1, d=64, dtype="f32", block=16, top_p=0.9, seed=1)
C2 = PrefillConfig("gqa-bf16-L8192", L=8192, hq=32, hkv=8, d=128, dtype="bf16", block=64, top_p=0.9, seed=2)
C3 = PrefillConfig("heavy-perm-bf16-L32768", L=32768, hq=32, hkv=8, d=128, dtype="bf16", block=128,
                   top_p=0.95, seed=3, heavy_hitters=True, segment=2048)
C4 = DecodeConfig("decode-b16-T131072", batch=16, T=131072, hq=32, hkv=8, d=128, block=16,
                  h_idx=4, d_idx=64, top_p=0.9, seed=4)
C5 = PrefillConfig("long-bf16-L131072", L=131072, hq=32, hkv=8, d=128, dtype="bf16", block=128,
                   top_p=0.9, seed=5, heavy_hitters=True, oracle_qblocks=64)
CONFIGS = {1: C1, 2: C2, 3: C3, 4: C4, 5: C5}


# --------------------------------------------------------------------------- draws
def _normal_slices(seed: int, code: int, shape: tuple[int, ...], bf16: bool) -> np.ndarray:
    """Array of shape (batch, heads, ...) with one seeded N(0,1) stream per (b, h)."""
    b_n, h_n = shape[0], shape[1]
    inner = shape[2:]
    out = np.empty(shape, dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, h_n)
        rng = np.random.default_rng([seed, code, b, h])
        x = rng.standard_normal(inner, dtype=np.float32)
        out[b, h] = round_bf16(x) if bf16 else x

    n = b_n * h_n
    if n * math.prod(inner) >= (1 << 22):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n)))
    else:
        for bh in range(n):
            fill(bh)
    return out


def heavy_hitter_plan(seed: int, L: int, d: int):
    """Positions (shared by all KV heads) and the shared unit direction."""
    rng = np.random.default_rng([seed, _HH])
    n_hh = int(round(0.02 * L))
    pos = np.sort(rng.choice(L, n_hh, replace=False))
    z = rng.standard_normal(d)
    return pos, z / np.linalg.norm(z)


def plant_heavy_hitters(k: np.ndarray, seed: int, bf16: bool) -> np.ndarray:
    """k: (batch, Hkv, L, d) float32, modified in place and returned."""
    L, d = k.shape[2], k.shape[3]
    pos, u = heavy_hitter_plan(seed, L, d)
    rows = k[:, :, pos, :].astype(np.float64)
    norms = np.linalg.norm(rows, axis=-1, keepdims=True)
    planted = (4.0 * norms * u).astype(np.float32)
    k[:, :, pos, :] = round_bf16(planted) if bf16 else planted
    return k


def prefill_inputs(cfg: PrefillConfig):
    """Q (batch,Hq,L,d), K, V (batch,Hkv,L,d) as float32 arrays holding exact
    input values (bf16-representable when cfg.dtype == 'bf16')."""
    bf16 = cfg.dtype == "bf16"
    q = _normal_slices(cfg.seed, _Q, (cfg.batch, cfg.hq, cfg.L, cfg.d), bf16)
    k = _normal_slices(cfg.seed, _K, (cfg.batch, cfg.hkv, cfg.L, cfg.d), bf16)
    v = _normal_slices(cfg.seed, _V, (cfg.batch, cfg.hkv, cfg.L, cfg.d), bf16)
    if cfg.heavy_hitters:
        plant_heavy_hitters(k, cfg.seed, bf16)
    return q, k, v


def oracle_query_blocks(cfg: PrefillConfig) -> np.ndarray:
    """Seeded sample of query blocks the oracle checks on long workloads:
    always blocks 0, 1 and the last one, the rest drawn without replacement."""
    nb = cfg.nb
    if cfg.oracle_qblocks <= 0 or cfg.oracle_qblocks >= nb:
        return np.arange(nb)
    rng = np.random.default_rng([cfg.seed, 77])
    must = {0, 1, nb - 1}
    rest = [int(x) for x in rng.permutation(nb) if int(x) not in must]
    pick = sorted(must | set(rest[: cfg.oracle_qblocks - len(must)]))
    return np.asarray(pick, dtype=np.int64)


def decode_inputs(cfg: DecodeConfig):
    """Decode-step inputs.

    Returns dict with q (batch,Hq,d), k_cache/v_cache (batch,Hkv,T,d) as
    bf16-exact float32, idx_q (batch,H_idx,d_idx) bf16-exact float32,
    idx_w (batch,H_idx) float32 and idx_k (batch,nT,H_idx,d_idx) bf16-exact
    float32.
    """
    b_n, T, d, B = cfg.batch, cfg.T, cfg.d, cfg.block
    kc = _normal_slices(cfg.seed, _K, (b_n, cfg.hkv, T, d), True)
    vc = _normal_slices(cfg.seed, _V, (b_n, cfg.hkv, T, d), True)
    q = _normal_slices(cfg.seed, _DQ, (b_n, 1, cfg.hq, d), True)[:, 0]
    width = cfg.h_idx * cfg.d_idx
    x = q.reshape(b_n, cfg.hq * d).astype(np.float64)
    fan = cfg.hq * d
    w_qi = np.random.default_rng([cfg.seed, _WQI]).standard_normal((width, fan)) / math.sqrt(fan)
    w_w = np.random.default_rng([cfg.seed, _WW]).standard_normal((cfg.h_idx, fan)) / math.sqrt(fan)
    kfan = cfg.hkv * d
    w_ki = np.random.default_rng([cfg.seed, _WKI]).standard_normal((width, kfan)) / math.sqrt(kfan)

    idx_q = round_bf16((x @ w_qi.T).reshape(b_n, cfg.h_idx, cfg.d_idx).astype(np.float32))
    logits = x @ w_w.T
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    idx_w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)

    nt = cfg.nt
    idx_k = np.empty((b_n, nt, cfg.h_idx, cfg.d_idx), dtype=np.float32)
    for b in range(b_n):
        # 16-token means of the cache, flattened over (KV head, d), re-standardised
        means = np.empty((nt, cfg.hkv * d), dtype=np.float64)
        for t0 in range(0, nt, 4096):
            t1 = min(nt, t0 + 4096)
            rows = kc[b, :, t0 * B: min(T, t1 * B), :].astype(np.float64)   # (Hkv, n, d)
            n_rows = rows.shape[1]
            full = (n_rows // B) * B
            blk = rows[:, :full].reshape(cfg.hkv, full // B, B, d).mean(axis=2)  # (Hkv, nb, d)
            parts = [blk]
            if full < n_rows:
                parts.append(rows[:, full:].mean(axis=1, keepdims=True))
            blk = np.concatenate(parts, axis=1)
            means[t0:t1] = blk.transpose(1, 0, 2).reshape(t1 - t0, cfg.hkv * d)
        proj = (math.sqrt(B) * means) @ w_ki.T
        idx_k[b] = round_bf16(proj.reshape(nt, cfg.h_idx, cfg.d_idx).astype(np.float32))
    return dict(q=q, k_cache=kc, v_cache=vc, idx_q=idx_q, idx_w=idx_w, idx_k=idx_k)


def small_prefill(name="small", L=1000, hq=8, hkv=2, d=128, dtype="bf16", block=64, top_p=0.9,
                  seed=11, heavy_hitters=False, segment=0, **kw) -> PrefillConfig:
    """A parity-size prefill workload with the same recipe as the full ones."""
    return PrefillConfig(name, L=L, hq=hq, hkv=hkv, d=d, dtype=dtype, block=block, top_p=top_p,
                         seed=seed, heavy_hitters=heavy_hitters, segment=segment, **kw)
