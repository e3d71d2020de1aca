"""MXFP4 selector key cache ([Spot] §4) on the GPU: the encoding is compared
bit for bit with the oracle's, the scores from the encoded cache and the
whole decode step against the float64 oracle on the decoded keys."""
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
from tests.test_oracle_mxfp4 import _value

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def gpu_quantize(x_bf16, gpu, h_idx, d_idx):
    """x (batch, nT, h_idx, d_idx) bf16 torch tensor on the host."""
    dk = x_bf16.to(gpu).contiguous()
    codes, scales = B.quantize_indexer_keys(dk, 16, 16 * x_bf16.shape[1])
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_quantize_worked_groups_bit_exact(gpu):
    spec = json.loads((Path(__file__).parent / "golden" / "mxfp4_worked.json").read_text())
    vals = []
    for gi, grp in enumerate(spec["groups"]):
        x = [_value(v) for v in grp["values"]]
        if gi == 0:
            x[10] = -0.0
        vals.append(x)
    x = np.array(vals, dtype=np.float32).reshape(1, len(vals), 1, 32)   # one 32-wide head per key block
    xb = _bf16_bits(x)
    assert np.array_equal(xb.float().numpy(), x)                        # the fixture is bf16-exact
    codes, scales = gpu_quantize(xb, gpu, 1, 32)
    got = oracle.mxfp4_unpack(codes)[0]
    for gi, grp in enumerate(spec["groups"]):
        assert scales[0, gi, 0] == grp["scale_byte"], gi
        assert got[gi].tolist() == grp["codes"], gi


@pytest.mark.parametrize("h_idx,d_idx", [(4, 64), (2, 128), (1, 32), (8, 32)])
def test_quantize_random_bit_exact(gpu, h_idx, d_idx):
    """Random bf16 keys over a wide range of magnitudes (with zero groups,
    exact ties and subnormal values): codes and scales equal the oracle's."""
    rng = np.random.default_rng(h_idx * 100 + d_idx)
    nt = 517
    x = rng.standard_normal((2, nt, h_idx, d_idx)).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 100, size=(2, nt, h_idx, 1))).astype(np.float32)
    x[0, 3] = 0.0
    x[1, 5, 0, :8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=np.float32)
    xb = _bf16_bits(x)
    xr = xb.float().numpy().astype(np.float64)
    codes, scales = gpu_quantize(xb, gpu, h_idx, d_idx)
    oc, osc = oracle.mxfp4_quantize(xr.reshape(2, nt, h_idx * d_idx))
    assert np.array_equal(scales, osc)
    assert np.array_equal(oracle.mxfp4_unpack(codes), oc)
    log("mxfp4 quantize", h_idx, d_idx, "groups", osc.size, "bit-exact")


def _decode_case(cfg, gpu):
    D = I.decode_inputs(cfg)
    dev = {k: (torch.from_numpy(v).to(gpu) if k == "idx_w" else P.to_dev(v, "bf16", gpu)) for k, v in D.items()}
    codes, scales = B.quantize_indexer_keys(dev["idx_k"], cfg.block, cfg.T)
    return D, dev, codes, scales


def _oracle_scores(D, b):
    nt, h_idx, d_idx = D["idx_k"][b].shape
    c, s = oracle.mxfp4_quantize(np.asarray(D["idx_k"][b], dtype=np.float64).reshape(nt, h_idx * d_idx))
    kd = oracle.mxfp4_dequantize(c, s).reshape(nt, h_idx, d_idx)
    return oracle.indexer_scores(D["idx_q"][b], D["idx_w"][b], kd), c, s


@pytest.mark.parametrize("kw", [dict(batch=2, T=16 * 1000 + 5), dict(batch=3, T=4096, hq=16, hkv=2, d=64),
                                dict(batch=2, T=3000, h_idx=2, d_idx=128), dict(batch=1, T=10),
                                # three groups per key row (the scan's lane count rounds up to four)
                                dict(batch=2, T=2000, h_idx=3, d_idx=32), dict(batch=2, T=2000, h_idx=3, d_idx=64)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_mxfp4_decode_small(gpu, kw):
    cfg = I.C4.with_(name="dec-mx", seed=31, **kw)
    D, dev, codes, scales = _decode_case(cfg, gpu)
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], (codes, scales),
                    cfg.block, cfg.top_p)
    torch.cuda.synchronize()
    check_mxfp4_decode(cfg, D, bufs, codes, scales)


def check_mxfp4_decode(cfg, D, bufs, codes, scales, batches=None):
    gs = bufs.scores.cpu().numpy()[:, 0, 0]
    gl = bufs.idx.cpu().numpy()[:, 0, 0]
    gc = bufs.cnt.cpu().numpy()[:, 0, 0]
    go = bufs.o.float().cpu().numpy()
    cn, sn = codes.cpu().numpy(), scales.cpu().numpy()
    rep = P.SelectionReport()
    worst = 0.0
    scale = 1 / math.sqrt(cfg.d)
    for b in (range(cfg.batch) if batches is None else batches):
        s, oc, osc = _oracle_scores(D, b)
        assert np.array_equal(oracle.mxfp4_unpack(cn[b]), oc) and np.array_equal(sn[b], osc)
        err = np.abs(gs[b] - s)
        assert np.all(err <= 1e-5 * np.abs(s) + 1e-5), float(err.max())
        P.compare_selection(rep, gl[b, :gc[b]], s, oracle.decode_forced(cfg.nt, cfg.n_sink, cfg.n_recent),
                            cfg.top_p, cfg.k_min, b)
        o_ref, _ = oracle.attend_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], gl[b, :gc[b]], cfg.block,
                                        cfg.T, scale)
        worst = max(worst, P.max_abs(go[b], o_ref))
    log(cfg.name, "mxfp4 selection", rep, "kept", gc.tolist(), f"max|dO|={worst:.3g}")
    assert not rep.violations, rep.violations[:5]
    assert worst <= P.BF16_ATOL


def test_mxfp4_c4_decode_full(gpu):
    """The decode workload (batch 16, T=131072) with the MXFP4 indexer cache:
    encoding, scores, selection and output checked for every sequence."""
    cfg = I.C4
    D, dev, codes, scales = _decode_case(cfg, gpu)
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], (codes, scales),
                    cfg.block, cfg.top_p)
    torch.cuda.synchronize()
    check_mxfp4_decode(cfg, D, bufs, codes, scales)
