"""INT4 selector key cache ([Spot] §4) on the GPU: codes and scales compared
bit for bit with the oracle's (hand-worked groups and random keys over a
wide range of magnitudes), the scores from the encoded cache and the whole
decode step against the float64 oracle on the decoded keys."""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P
from tests.test_gpu_parity import log

pytestmark = pytest.mark.gpu


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def gpu_quantize(xb, gpu):
    """xb (batch, nT, h_idx, d_idx) bf16 torch tensor on the host -> packed codes, scales (float64)."""
    codes, scales = B.quantize_indexer_keys_int4(xb.to(gpu).contiguous(), 16, 16 * xb.shape[1])
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.float().cpu().numpy().astype(np.float64)


def test_quantize_worked_groups_bit_exact(gpu):
    spec = json.loads((Path(__file__).parent / "golden" / "int4_worked.json").read_text())
    x = np.array([g["values"] for g in spec["groups"]], dtype=np.float32).reshape(1, -1, 1, 32)
    xb = _bf16(x)
    assert np.array_equal(xb.float().numpy(), x)
    codes, scales = gpu_quantize(xb, gpu)
    for gi, grp in enumerate(spec["groups"]):
        assert scales[0, gi, 0] == grp["scale"], gi
        assert codes[0, gi].tolist() == oracle.int4_pack(np.array([grp["codes"]], np.int8))[0].tolist(), gi


@pytest.mark.parametrize("h_idx,d_idx", [(4, 64), (2, 128), (1, 32), (8, 32)])
def test_quantize_random_bit_exact(gpu, h_idx, d_idx):
    rng = np.random.default_rng(h_idx * 100 + d_idx + 7)
    nt = 517
    x = rng.standard_normal((2, nt, h_idx, d_idx)).astype(np.float32)
    x *= np.exp2(rng.integers(-60, 60, size=(2, nt, h_idx, 1))).astype(np.float32)
    x[0, 3] = 0.0
    x[1, 5, 0, :8] = np.array([7, 3.5, 2.5, 0.5, -1.5, -2.5, 6.5, 1], dtype=np.float32)   # ties at scale 1
    xb = _bf16(x)
    xr = xb.float().numpy().astype(np.float64)
    codes, scales = gpu_quantize(xb, gpu)
    oc, osc = oracle.int4_quantize(xr.reshape(2, nt, h_idx * d_idx))
    assert np.array_equal(scales, osc)
    assert np.array_equal(codes, oracle.int4_pack(oc))
    log("int4 quantize", h_idx, d_idx, "groups", osc.size, "bit-exact")


def _decode_case(cfg, gpu):
    D = I.decode_inputs(cfg)
    dev = {k: (torch.from_numpy(v).to(gpu) if k == "idx_w" else P.to_dev(v, "bf16", gpu)) for k, v in D.items()}
    codes, scales = B.quantize_indexer_keys_int4(dev["idx_k"], cfg.block, cfg.T)
    return D, dev, codes, scales


def check_int4_decode(cfg, D, bufs, codes, scales):
    gs = bufs.scores.cpu().numpy()[:, 0, 0]
    gl = bufs.idx.cpu().numpy()[:, 0, 0]
    gc = bufs.cnt.cpu().numpy()[:, 0, 0]
    go = bufs.o.float().cpu().numpy()
    cn, sn = codes.cpu().numpy(), scales.float().cpu().numpy().astype(np.float64)
    rep = P.SelectionReport()
    worst = 0.0
    scale = 1 / math.sqrt(cfg.d)
    for b in range(cfg.batch):
        nt, h_idx, d_idx = D["idx_k"][b].shape
        oc, osc = oracle.int4_quantize(np.asarray(D["idx_k"][b], dtype=np.float64).reshape(nt, h_idx * d_idx))
        assert np.array_equal(cn[b], oracle.int4_pack(oc)) and np.array_equal(sn[b], osc)
        kd = oracle.int4_dequantize(oc, osc).reshape(nt, h_idx, d_idx)
        s = oracle.indexer_scores(D["idx_q"][b], D["idx_w"][b], kd)
        err = np.abs(gs[b] - s)
        assert np.all(err <= 1e-5 * np.abs(s) + 1e-5), float(err.max())
        P.compare_selection(rep, gl[b, :gc[b]], s, oracle.decode_forced(cfg.nt, cfg.n_sink, cfg.n_recent),
                            cfg.top_p, cfg.k_min, b)
        o_ref, _ = oracle.attend_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], gl[b, :gc[b]], cfg.block,
                                        cfg.T, scale)
        worst = max(worst, P.max_abs(go[b], o_ref))
    log(cfg.name, "int4 selection", rep, "kept", gc.tolist(), f"max|dO|={worst:.3g}")
    assert not rep.violations, rep.violations[:5]
    assert worst <= P.BF16_ATOL


@pytest.mark.parametrize("kw", [dict(batch=2, T=16 * 1000 + 5), dict(batch=3, T=4096, hq=16, hkv=2, d=64),
                                dict(batch=2, T=3000, h_idx=2, d_idx=128), dict(batch=1, T=10),
                                # three groups per key row (the scan's lane count rounds up to four)
                                dict(batch=2, T=2000, h_idx=3, d_idx=32), dict(batch=2, T=2000, h_idx=3, d_idx=64)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_int4_decode_small(gpu, kw):
    cfg = I.C4.with_(name="dec-int4", seed=37, **kw)
    D, dev, codes, scales = _decode_case(cfg, gpu)
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], (codes, scales),
                    cfg.block, cfg.top_p)
    torch.cuda.synchronize()
    check_int4_decode(cfg, D, bufs, codes, scales)


def test_int4_c4_decode_full(gpu):
    """The decode workload (batch 16, T=131072) with the INT4 indexer cache: encoding, scores, selection
    and output checked for every sequence."""
    cfg = I.C4
    D, dev, codes, scales = _decode_case(cfg, gpu)
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], (codes, scales),
                    cfg.block, cfg.top_p)
    torch.cuda.synchronize()
    check_int4_decode(cfg, D, bufs, codes, scales)
