"""C ABI boundary on the CPU: the library loads, exports every function
include/spot.h declares, and every validation path returns its documented
status before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "spot.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(spot_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_entry_points_and_helpers():
    names = header_functions()
    for n in ("spot_block_score", "spot_select_topp", "spot_sparse_attn_prefill", "spot_sparse_attn_decode",
              "spot_workspace_size", "spot_status_string", "spot_last_error", "spot_version"):
        assert n in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    for n in header_functions():
        assert hasattr(lib, n), n
    assert B.spot_version() == B.ABI_VERSION


def test_descriptor_layout_matches_header():
    # int32 x6, int64 x2, int32 x5, float x2, int32 x3 -> 80 bytes with natural alignment
    assert ctypes.sizeof(B.spot_desc) == 80
    assert B.spot_desc.q_len.offset == 24 and B.spot_desc.top_p.offset == 60


def test_status_strings():
    lib = B.load_library()
    for st in (0, -1, -2, -3, -4):
        assert lib.spot_status_string(st)
    assert lib.spot_status_string(7) == b"unknown status"


def _prefill(**kw):
    base = dict(dtype=B.SPOT_BF16, batch=1, hq=8, hkv=2, d=128, q_len=1024, kv_len=1024, block=64, top_p=0.9)
    base.update(kw)
    return B.make_desc(**base)


def _decode(**kw):
    base = dict(dtype=B.SPOT_BF16, batch=2, hq=8, hkv=2, d=128, q_len=1, kv_len=4096, block=16, top_p=0.9,
                score_kind=B.SPOT_SCORE_RELU_INDEXER, h_idx=4, d_idx=64)
    base.update(kw)
    return B.make_desc(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def call_score(d, ws_bytes=1 << 30, q=FAKE, k=FAKE, perm=None, iq=None, iw=None, ik=None, scores=FAKE, ws=FAKE):
    lib = B.load_library()
    return lib.spot_block_score(ctypes.byref(d) if d is not None else None, q, k, perm, iq, iw, ik, scores, ws,
                                ws_bytes, None)


def call_select(d, scores=FAKE, idx=FAKE, cnt=FAKE):
    return B.load_library().spot_select_topp(ctypes.byref(d), scores, idx, cnt, None, 0, None)


def call_prefill(d, q=FAKE, k=FAKE, v=FAKE, perm=None, idx=FAKE, cnt=FAKE, o=FAKE):
    return B.load_library().spot_sparse_attn_prefill(ctypes.byref(d), q, k, v, perm, idx, cnt, o, None, None, 0, None)


def call_decode(d, ws=FAKE, ws_bytes=1 << 30, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE, o=FAKE):
    return B.load_library().spot_sparse_attn_decode(ctypes.byref(d), q, k, v, idx, cnt, o, None, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(version=2), B.SPOT_ERR_INVALID),
    (dict(dtype=7), B.SPOT_ERR_INVALID),
    (dict(batch=0), B.SPOT_ERR_INVALID),
    (dict(hq=6, hkv=4), B.SPOT_ERR_INVALID),
    (dict(d=96), B.SPOT_ERR_UNSUPPORTED),
    (dict(block=48), B.SPOT_ERR_UNSUPPORTED),
    (dict(block=256), B.SPOT_ERR_UNSUPPORTED),
    (dict(q_len=0, kv_len=0), B.SPOT_ERR_INVALID),
    (dict(kv_len=1000), B.SPOT_ERR_INVALID),            # prefill needs q_len == kv_len
    (dict(segment=100), B.SPOT_ERR_INVALID),            # not a multiple of the block
    (dict(segment=-64), B.SPOT_ERR_INVALID),
    (dict(sm_scale=-1.0), B.SPOT_ERR_INVALID),
    (dict(sm_scale=float("inf")), B.SPOT_ERR_INVALID),
])
def test_common_validation(case, expect):
    case = dict(case)
    version = case.pop("version", None)
    d = _prefill(**case)
    if version is not None:
        d.version = version
    assert call_score(d) == expect
    assert B.load_library().spot_last_error()


def test_null_and_missing_arguments():
    assert call_score(None) == B.SPOT_ERR_INVALID
    assert call_score(_prefill(), q=None) == B.SPOT_ERR_INVALID
    assert call_score(_prefill(), scores=None) == B.SPOT_ERR_INVALID
    assert call_score(_prefill(), perm=FAKE) == B.SPOT_ERR_INVALID          # perm without a segment
    assert call_score(_prefill(), ws=None) == B.SPOT_ERR_WORKSPACE
    assert call_score(_prefill(), ws_bytes=100) == B.SPOT_ERR_WORKSPACE
    assert call_score(_prefill(score_kind=9)) == B.SPOT_ERR_INVALID
    assert call_prefill(_prefill(), v=None) == B.SPOT_ERR_INVALID
    assert call_prefill(_prefill(), perm=FAKE) == B.SPOT_ERR_INVALID
    assert call_prefill(_prefill(), o=None) == B.SPOT_ERR_INVALID
    for kw in (dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2), dict(o=FAKE + 4)):   # bf16: 16-byte q/k/v, 8-byte o
        assert call_prefill(_prefill(), **kw) == B.SPOT_ERR_INVALID, kw
    assert call_select(_prefill(), cnt=None) == B.SPOT_ERR_INVALID
    for kw in (dict(q=FAKE + 8), dict(k=FAKE + 4)):      # pooled scores read q and k rows in 16-byte pieces
        assert call_score(_prefill(), **kw) == B.SPOT_ERR_INVALID, kw
        assert call_score(_prefill(dtype=B.SPOT_F32), **kw) == B.SPOT_ERR_INVALID, kw


def test_selection_parameters():
    assert call_select(_prefill(n_sink=0, n_recent=0)) == B.SPOT_ERR_INVALID
    assert call_select(_prefill(n_sink=-1)) == B.SPOT_ERR_INVALID
    assert call_select(_prefill(k_min=-2)) == B.SPOT_ERR_INVALID
    assert call_select(_prefill(top_p=float("nan"))) == B.SPOT_ERR_INVALID
    # too many candidate blocks for one row
    assert call_select(_prefill(q_len=16 * 20000, kv_len=16 * 20000, block=16)) == B.SPOT_ERR_UNSUPPORTED


def test_indexer_and_decode_validation():
    assert call_score(_decode(), q=None, k=None) == B.SPOT_ERR_INVALID                 # idx_* missing
    assert call_score(_decode(d_idx=48), iq=FAKE, iw=FAKE, ik=FAKE) == B.SPOT_ERR_UNSUPPORTED
    assert call_score(_decode(h_idx=8, d_idx=64), iq=FAKE, iw=FAKE, ik=FAKE) == B.SPOT_ERR_UNSUPPORTED
    assert call_decode(_decode(q_len=2)) == B.SPOT_ERR_INVALID
    assert call_decode(_decode(dtype=B.SPOT_F32)) == B.SPOT_ERR_UNSUPPORTED
    assert call_decode(_decode(hq=12, hkv=4)) == B.SPOT_ERR_UNSUPPORTED                 # G = 3
    assert call_decode(_decode(), ws=None) == B.SPOT_ERR_WORKSPACE
    assert call_decode(_decode(), ws_bytes=8) == B.SPOT_ERR_WORKSPACE
    assert call_decode(_decode(), o=None) == B.SPOT_ERR_INVALID
    for kw in (dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2), dict(ws=FAKE + 8)):   # 16-byte loads/stores
        assert call_decode(_decode(), **kw) == B.SPOT_ERR_INVALID, kw
    for kw in (dict(iq=FAKE + 8), dict(ik=FAKE + 2)):    # indexer rows in 16-byte pieces
        args = dict(iq=FAKE, iw=FAKE, ik=FAKE)
        args.update(kw)
        assert call_score(_decode(), q=None, k=None, **args) == B.SPOT_ERR_INVALID, kw


def test_decode_noalloc_validation():
    lib = B.load_library()

    def call(d, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE, o=FAKE):
        return lib.spot_sparse_attn_decode_noalloc(ctypes.byref(d), q, k, v, idx, cnt, o, None, None)

    assert call(_decode(q_len=2)) == B.SPOT_ERR_INVALID
    assert call(_decode(dtype=B.SPOT_F32)) == B.SPOT_ERR_UNSUPPORTED
    assert call(_decode(hq=12, hkv=4)) == B.SPOT_ERR_UNSUPPORTED
    assert call(_decode(), o=None) == B.SPOT_ERR_INVALID
    for kw in (dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2)):
        assert call(_decode(), **kw) == B.SPOT_ERR_INVALID, kw
    # partials beyond the built-in 8 MiB scratch: 512 sequences x 32 heads x 1 split x 130 floats
    assert call(_decode(batch=512, hq=32, hkv=4)) == B.SPOT_ERR_UNSUPPORTED
    assert b"scratch" in lib.spot_last_error()


def call_perm(d, q=FAKE, k=FAKE, perm=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return B.load_library().spot_key_permutation(ctypes.byref(d), q, k, perm, None, ws, ws_bytes, None)


def test_key_permutation_validation():
    assert call_perm(_prefill(segment=256, dtype=B.SPOT_F32)) == B.SPOT_ERR_UNSUPPORTED
    assert call_perm(_prefill(segment=0)) == B.SPOT_ERR_INVALID
    assert call_perm(_prefill(segment=96)) == B.SPOT_ERR_INVALID                 # not a multiple of the block
    assert call_perm(_prefill(segment=32768, q_len=65536, kv_len=65536)) == B.SPOT_ERR_UNSUPPORTED
    assert call_perm(_prefill(segment=256), perm=None) == B.SPOT_ERR_INVALID
    assert call_perm(_prefill(segment=256), ws=None) == B.SPOT_ERR_WORKSPACE
    assert call_perm(_prefill(segment=256), ws_bytes=64) == B.SPOT_ERR_WORKSPACE
    assert B.spot_workspace_size(_prefill(segment=256), B.SPOT_OP_KEY_PERMUTATION) > 0
    assert call_perm(_prefill(segment=256), q=FAKE + 8) == B.SPOT_ERR_INVALID
    assert call_perm(_prefill(segment=256), k=FAKE + 2) == B.SPOT_ERR_INVALID


def call_vperm(d, perm=FAKE, bad=FAKE):
    return B.load_library().spot_validate_perm(ctypes.byref(d), perm, bad, None)


def test_validate_perm_validation():
    assert call_vperm(_prefill(segment=0)) == B.SPOT_ERR_INVALID
    assert call_vperm(_prefill(segment=32768, q_len=65536, kv_len=65536)) == B.SPOT_ERR_UNSUPPORTED
    assert call_vperm(_prefill(segment=256), perm=None) == B.SPOT_ERR_INVALID
    assert call_vperm(_prefill(segment=256), bad=None) == B.SPOT_ERR_INVALID
    assert call_vperm(_prefill(segment=256, q_len=512)) == B.SPOT_ERR_INVALID          # q_len != kv_len


def call_order(d, scores=FAKE, order=FAKE, cnt=FAKE):
    return B.load_library().spot_order_history(ctypes.byref(d), scores, order, cnt, None, 0, None)


def call_es(d, tau=0.01, q=FAKE, k=FAKE, v=FAKE, perm=None, order=FAKE, cnt=FAKE, o=FAKE):
    return B.load_library().spot_sparse_attn_prefill_early_stop(ctypes.byref(d), tau, q, k, v, perm, order, cnt, o,
                                                                 None, None, None, 0, None)


def test_early_stop_validation():
    assert call_order(_prefill(segment=0)) == B.SPOT_ERR_INVALID
    assert call_order(_prefill(segment=96)) == B.SPOT_ERR_INVALID                 # not a multiple of the block
    assert call_order(_prefill(segment=256), order=None) == B.SPOT_ERR_INVALID
    assert call_order(_prefill(segment=256, q_len=64 * 5000, kv_len=64 * 5000)) == B.SPOT_ERR_UNSUPPORTED
    assert call_es(_prefill(segment=0)) == B.SPOT_ERR_INVALID
    assert call_es(_prefill(segment=256), tau=-0.5) == B.SPOT_ERR_INVALID
    assert call_es(_prefill(segment=256), tau=float("nan")) == B.SPOT_ERR_INVALID
    assert call_es(_prefill(segment=256), tau=float("inf")) == B.SPOT_ERR_INVALID
    assert call_es(_prefill(segment=256), order=None) == B.SPOT_ERR_INVALID
    assert call_es(_prefill(segment=256), o=None) == B.SPOT_ERR_INVALID
    for kw in (dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2), dict(o=FAKE + 4)):
        assert call_es(_prefill(segment=256), **kw) == B.SPOT_ERR_INVALID, kw
    assert call_es(_prefill(segment=256, dtype=B.SPOT_F32)) == B.SPOT_ERR_UNSUPPORTED
    assert call_es(_prefill(segment=256, block=32)) == B.SPOT_ERR_UNSUPPORTED
    assert call_es(_prefill(segment=256, q_len=64 * 3000, kv_len=64 * 3000)) == B.SPOT_ERR_UNSUPPORTED
    assert B.spot_workspace_size(_prefill(segment=256), B.SPOT_OP_ORDER_HISTORY) == 0
    assert B.spot_workspace_size(_prefill(segment=256), B.SPOT_OP_PREFILL_EARLY_STOP) == 0


def test_workspace_sizes():
    d = _prefill()
    assert B.spot_workspace_size(d, B.SPOT_OP_BLOCK_SCORE) == 3 * 1 * 2 * 16 * 128 * 4
    assert B.spot_workspace_size(d, B.SPOT_OP_SELECT_TOPP) == 0
    assert B.spot_workspace_size(d, B.SPOT_OP_PREFILL) == 0
    dd = _decode()
    assert B.spot_workspace_size(dd, B.SPOT_OP_DECODE) > 0
    assert B.spot_workspace_size(_decode(), B.SPOT_OP_BLOCK_SCORE) == 0
    with pytest.raises(B.SpotError):
        B.spot_workspace_size(d, 17)
    with pytest.raises(B.SpotError):
        B.spot_workspace_size(_prefill(d=80), B.SPOT_OP_BLOCK_SCORE)


def test_error_message_is_thread_local_and_cleared():
    lib = B.load_library()
    assert call_score(None) == B.SPOT_ERR_INVALID
    assert lib.spot_last_error() == b"desc is NULL"
    B.spot_workspace_size(_prefill(), B.SPOT_OP_PREFILL)
    assert lib.spot_last_error() == b""


def test_taylor_score_workspace_and_validation():
    d = _prefill(score_kind=B.SPOT_SCORE_TAYLOR)
    assert B.spot_workspace_size(d, B.SPOT_OP_BLOCK_SCORE) == 5 * 1 * 2 * 16 * 128 * 4
    need = B.spot_workspace_size(d, B.SPOT_OP_BLOCK_SCORE)
    assert call_score(d, ws_bytes=need - 1) == B.SPOT_ERR_WORKSPACE
    assert call_score(d, q=None) == B.SPOT_ERR_INVALID


def test_mxfp4_indexer_validation():
    lib = B.load_library()

    def q(d, x=FAKE, c=FAKE, s=FAKE):
        return lib.spot_quantize_indexer_keys(ctypes.byref(d), x, c, s, None)

    def sc(d, iq=FAKE, iw=FAKE, c=FAKE, s=FAKE, out=FAKE):
        return lib.spot_indexer_score_mxfp4(ctypes.byref(d), iq, iw, c, s, out, None)

    assert q(_decode(d_idx=16, h_idx=4)) == B.SPOT_ERR_UNSUPPORTED          # groups of 32 need d_idx % 32 == 0
    assert sc(_decode(d_idx=16, h_idx=4)) == B.SPOT_ERR_UNSUPPORTED
    assert q(_decode(h_idx=8, d_idx=64)) == B.SPOT_ERR_UNSUPPORTED           # row wider than 256
    assert q(_decode(score_kind=B.SPOT_SCORE_MEANPOOL)) == B.SPOT_ERR_INVALID
    assert q(_decode(), x=None) == B.SPOT_ERR_INVALID
    assert sc(_decode(), s=None) == B.SPOT_ERR_INVALID
    assert sc(_decode(), out=None) == B.SPOT_ERR_INVALID
    assert q(_decode(), x=FAKE + 2) == B.SPOT_ERR_INVALID                  # 16-byte loads and stores
    assert q(_decode(), c=FAKE + 8) == B.SPOT_ERR_INVALID
    assert sc(_decode(), iq=FAKE + 4) == B.SPOT_ERR_INVALID
    assert sc(_decode(), c=FAKE + 1) == B.SPOT_ERR_INVALID


def test_int4_indexer_validation():
    lib = B.load_library()

    def q(d, x=FAKE, c=FAKE, s=FAKE):
        return lib.spot_quantize_indexer_keys_int4(ctypes.byref(d), x, c, s, None)

    def sc(d, iq=FAKE, iw=FAKE, c=FAKE, s=FAKE, out=FAKE):
        return lib.spot_indexer_score_int4(ctypes.byref(d), iq, iw, c, s, out, None)

    assert q(_decode(d_idx=16, h_idx=4)) == B.SPOT_ERR_UNSUPPORTED          # groups of 32 need d_idx % 32 == 0
    assert sc(_decode(d_idx=16, h_idx=4)) == B.SPOT_ERR_UNSUPPORTED
    assert q(_decode(h_idx=8, d_idx=64)) == B.SPOT_ERR_UNSUPPORTED           # row wider than 256
    assert q(_decode(score_kind=B.SPOT_SCORE_MEANPOOL)) == B.SPOT_ERR_INVALID
    assert q(_decode(), x=None) == B.SPOT_ERR_INVALID
    assert sc(_decode(), s=None) == B.SPOT_ERR_INVALID
    assert sc(_decode(), out=None) == B.SPOT_ERR_INVALID
    assert q(_decode(), x=FAKE + 2) == B.SPOT_ERR_INVALID                   # 16-byte loads and stores
    assert q(_decode(), c=FAKE + 8) == B.SPOT_ERR_INVALID
    assert q(_decode(), s=FAKE + 1) == B.SPOT_ERR_INVALID                   # bf16 scales
    assert sc(_decode(), iq=FAKE + 4) == B.SPOT_ERR_INVALID
    assert sc(_decode(), s=FAKE + 1) == B.SPOT_ERR_INVALID


def test_history_map_validation():
    lib = B.load_library()

    def hm(d, q=FAKE, k=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.spot_history_map(ctypes.byref(d), q, k, out, ws, ws_bytes, None)

    def att(d, tau=0.01, hmap=FAKE, o=FAKE, q=FAKE, k=FAKE, v=FAKE):
        return lib.spot_sparse_attn_prefill_history_map(ctypes.byref(d), tau, q, k, v, hmap, o, None, None,
                                                         None, 0, None)

    assert hm(_prefill(segment=0)) == B.SPOT_ERR_INVALID
    assert hm(_prefill(segment=256, dtype=B.SPOT_F32)) == B.SPOT_ERR_UNSUPPORTED
    assert hm(_prefill(segment=256), out=None) == B.SPOT_ERR_INVALID
    assert hm(_prefill(segment=256), ws=None) == B.SPOT_ERR_WORKSPACE
    assert hm(_prefill(segment=256), ws_bytes=16) == B.SPOT_ERR_WORKSPACE
    assert hm(_prefill(segment=256), q=FAKE + 8) == B.SPOT_ERR_INVALID
    assert hm(_prefill(segment=256), k=FAKE + 2) == B.SPOT_ERR_INVALID
    assert hm(_prefill(segment=64, q_len=64 * 65, kv_len=64 * 65)) == B.SPOT_ERR_UNSUPPORTED        # 65 segments
    assert hm(_prefill(segment=8192, q_len=8192 * 6, kv_len=8192 * 6)) == B.SPOT_ERR_UNSUPPORTED    # prefix 40960
    assert B.spot_workspace_size(_prefill(segment=256), B.SPOT_OP_HISTORY_MAP) > 0
    assert att(_prefill(segment=0)) == B.SPOT_ERR_INVALID
    assert att(_prefill(segment=256), hmap=None) == B.SPOT_ERR_INVALID
    assert att(_prefill(segment=256), tau=-1.0) == B.SPOT_ERR_INVALID
    for kw in (dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2), dict(o=FAKE + 4)):
        assert att(_prefill(segment=256), **kw) == B.SPOT_ERR_INVALID, kw
    assert att(_prefill(segment=256, block=16)) == B.SPOT_ERR_UNSUPPORTED


def test_rla_validation():
    """Residual linear attention entry points: every rejected call returns
    before anything is launched (the pointers here are never dereferenced)."""
    lib = B.load_library()

    def st(d, k=FAKE, v=FAKE, perm=None, s=FAKE, sp=None):
        return lib.spot_rla_block_states(ctypes.byref(d), k, v, perm, s, sp, None)

    def pre(d, q=FAKE, s=FAKE, sp=None, idx=FAKE, cnt=FAKE, o=FAKE):
        return lib.spot_rla_prefill(ctypes.byref(d), q, s, sp, idx, cnt, o, None)

    def dst(d, k=FAKE, v=FAKE, s=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return lib.spot_rla_decode_state(ctypes.byref(d), k, v, s, ws, ws_bytes, None)

    def dec(d, q=FAKE, k=FAKE, v=FAKE, s=FAKE, idx=FAKE, cnt=FAKE, o=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return lib.spot_rla_decode(ctypes.byref(d), q, k, v, s, idx, cnt, o, ws, ws_bytes, None)

    assert st(_prefill(), k=None) == B.SPOT_ERR_INVALID
    assert st(_prefill(), s=None) == B.SPOT_ERR_INVALID
    assert st(_prefill(), perm=FAKE) == B.SPOT_ERR_INVALID                     # perm needs segment > 0
    assert st(_prefill(segment=256), perm=FAKE) == B.SPOT_ERR_INVALID          # ... and states_perm
    assert st(_prefill(), sp=FAKE) == B.SPOT_ERR_INVALID                       # states_perm without perm
    assert st(_prefill(), v=FAKE + 8) == B.SPOT_ERR_INVALID                    # 16-byte loads
    assert st(_prefill(), s=FAKE + 4) == B.SPOT_ERR_INVALID
    assert st(_prefill(d=96)) == B.SPOT_ERR_UNSUPPORTED
    assert st(_prefill(batch=70000)) == B.SPOT_ERR_UNSUPPORTED                 # batch * hkv beyond the grid
    assert pre(_prefill(), o=None) == B.SPOT_ERR_INVALID
    assert pre(_prefill(), cnt=None) == B.SPOT_ERR_INVALID
    assert pre(_prefill(n_recent=0)) == B.SPOT_ERR_UNSUPPORTED                 # own block must be kept
    assert pre(_prefill(), sp=FAKE) == B.SPOT_ERR_INVALID                      # permuted states need segments
    assert pre(_prefill(q_len=64 * 4097, kv_len=64 * 4097)) == B.SPOT_ERR_UNSUPPORTED   # 4097 blocks
    assert pre(_prefill(), q=FAKE + 2) == B.SPOT_ERR_INVALID
    assert dst(_decode(), ws=None) == B.SPOT_ERR_WORKSPACE
    assert dst(_decode(), ws_bytes=16) == B.SPOT_ERR_WORKSPACE
    assert dst(_decode(dtype=B.SPOT_F32)) == B.SPOT_ERR_UNSUPPORTED
    assert dst(_decode(q_len=2)) == B.SPOT_ERR_INVALID
    assert dst(_decode(), s=FAKE + 4) == B.SPOT_ERR_INVALID
    assert dec(_decode(hq=6, hkv=2)) == B.SPOT_ERR_UNSUPPORTED                 # G = 3
    assert dec(_decode(), s=None) == B.SPOT_ERR_INVALID
    assert dec(_decode(), k=FAKE + 2) == B.SPOT_ERR_INVALID
    assert dec(_decode(), q=FAKE + 1) == B.SPOT_ERR_INVALID
    assert dec(_decode(), ws=None) == B.SPOT_ERR_WORKSPACE
    assert dec(_decode(), ws_bytes=4) == B.SPOT_ERR_WORKSPACE
    assert dec(_decode(), ws=FAKE + 2) == B.SPOT_ERR_INVALID
    def fused(d, rs=FAKE, o_rla=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return lib.spot_sparse_attn_decode_rla(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, rs, FAKE, None, o_rla,
                                               ws, ws_bytes, None)

    assert fused(_decode(), rs=None) == B.SPOT_ERR_INVALID
    assert fused(_decode(), o_rla=None) == B.SPOT_ERR_INVALID
    assert fused(_decode(), ws_bytes=16) == B.SPOT_ERR_WORKSPACE
    assert fused(_decode(), rs=FAKE + 2) == B.SPOT_ERR_INVALID
    assert fused(_decode(hq=6, hkv=2)) == B.SPOT_ERR_UNSUPPORTED
    dd = _decode(kv_len=131072)
    assert B.spot_workspace_size(dd, B.SPOT_OP_DECODE_RLA) == (B.spot_workspace_size(dd, B.SPOT_OP_DECODE)
                                                               + 2 * 8 * 32 * 128 * 4)
    assert B.spot_workspace_size(dd, B.SPOT_OP_RLA_DECODE_STATE) == 2 * 2 * 32 * 128 * 128 * 4
    assert B.spot_workspace_size(dd, B.SPOT_OP_RLA_DECODE) == 2 * 8 * 64 * 128 * 4     # 64 splits of 4 pairs
