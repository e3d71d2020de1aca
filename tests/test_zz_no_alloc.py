"""The allocation-free decode entry point against the workspace one: the same
kept lists, two calls in a row (the second on a smaller input, so the shared
device scratch still holds the first call's partials), outputs equal."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu


def _run_both(cfg, gpu):
    D = I.decode_inputs(cfg)
    dev = {k: (torch.from_numpy(v).to(gpu) if k == "idx_w" else P.to_dev(v, "bf16", gpu)) for k, v in D.items()}
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], dev["idx_k"], cfg.block,
                    cfg.top_p)
    desc = B.decode_desc(dev["q"], dev["k_cache"], cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    o = torch.full_like(bufs.o, 3.0)
    lse = torch.full_like(bufs.lse, 5.0)
    B.spot_sparse_attn_decode_noalloc(desc, dev["q"], dev["k_cache"], dev["v_cache"], bufs.idx, bufs.cnt, o, lse)
    torch.cuda.synchronize()
    return D, bufs, o, lse


def test_decode_noalloc_matches_workspace_call(gpu):
    scale = None
    for kw in (dict(batch=6, T=16 * 3000 + 7, top_p=0.95), dict(batch=2, T=16 * 400, hq=16, hkv=2, top_p=0.8)):
        cfg = I.C4.with_(name="noalloc", seed=41, **kw)
        D, bufs, o, lse = _run_both(cfg, gpu)
        # same kernels, same split: the outputs are identical to the workspace call's
        assert torch.equal(o, bufs.o), kw
        assert torch.equal(lse, bufs.lse), kw
        # and within the parity bar of the oracle on the same kept lists
        scale = 1 / math.sqrt(cfg.d)
        gl, gc = bufs.idx.cpu().numpy()[:, 0, 0], bufs.cnt.cpu().numpy()[:, 0, 0]
        go, glse = o.float().cpu().numpy(), lse.cpu().numpy()
        for b in range(cfg.batch):
            o_ref, lse_ref = oracle.attend_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], gl[b, :gc[b]],
                                                  cfg.block, cfg.T, scale)
            assert P.max_abs(go[b], o_ref) <= P.BF16_ATOL
            assert P.max_abs(glse[b], lse_ref) <= P.BF16_LSE_ATOL
        print("[parity] noalloc", kw, "kept", gc.tolist(), flush=True)


def test_decode_noalloc_rejects_inputs_beyond_the_scratch(gpu):
    # 512 sequences x 32 heads: one split each, 512 * 32 * 130 * 4 bytes of partials > 8 MiB
    desc = B.make_desc(dtype=B.SPOT_BF16, batch=512, hq=32, hkv=4, d=128, q_len=1, kv_len=4096, block=16,
                       score_kind=B.SPOT_SCORE_RELU_INDEXER, h_idx=4, d_idx=64)
    x = torch.zeros(16, dtype=torch.bfloat16, device=gpu)
    i = torch.zeros(16, dtype=torch.int32, device=gpu)
    with pytest.raises(B.SpotError) as e:
        B.spot_sparse_attn_decode_noalloc(desc, x, x, x, i, i, x)
    assert e.value.status == B.SPOT_ERR_UNSUPPORTED
