"""Thin ctypes binding of libspot.so: same names as the C ABI, argument
marshalling only.  Torch tensors provide device memory; the current torch
stream is the launch stream.  Every step of the path runs in the library's
HIP kernels; there is no fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPOT_LIBRARY names another build of the same library (for example the host-sanitizer build)
LIB_PATH = os.environ.get("SPOT_LIBRARY") or os.path.join(_PKG, "libspot.so")

SPOT_OK, SPOT_ERR_INVALID, SPOT_ERR_UNSUPPORTED, SPOT_ERR_WORKSPACE, SPOT_ERR_LAUNCH = 0, -1, -2, -3, -4
SPOT_F32, SPOT_BF16 = 0, 1
SPOT_SCORE_MEANPOOL, SPOT_SCORE_RELU_INDEXER, SPOT_SCORE_TAYLOR = 0, 1, 2
SPOT_OP_BLOCK_SCORE, SPOT_OP_SELECT_TOPP, SPOT_OP_PREFILL, SPOT_OP_DECODE, SPOT_OP_KEY_PERMUTATION = 0, 1, 2, 3, 4
SPOT_OP_ORDER_HISTORY, SPOT_OP_PREFILL_EARLY_STOP, SPOT_OP_HISTORY_MAP, SPOT_OP_RLA_DECODE_STATE = 5, 6, 7, 8
SPOT_OP_RLA_DECODE, SPOT_OP_DECODE_RLA = 9, 10
ABI_VERSION = 1

EXPORTS = ("spot_version", "spot_status_string", "spot_last_error", "spot_workspace_size", "spot_block_score",
           "spot_select_topp", "spot_sparse_attn_prefill", "spot_sparse_attn_decode", "spot_key_permutation",
           "spot_order_history", "spot_sparse_attn_prefill_early_stop", "spot_quantize_indexer_keys",
           "spot_indexer_score_mxfp4", "spot_history_map", "spot_sparse_attn_prefill_history_map",
           "spot_validate_perm", "spot_sparse_attn_decode_noalloc", "spot_quantize_indexer_keys_int4",
           "spot_indexer_score_int4", "spot_rla_block_states", "spot_rla_prefill", "spot_rla_decode_state",
           "spot_rla_decode", "spot_sparse_attn_decode_rla")


class spot_desc(ctypes.Structure):
    _fields_ = [
        ("version", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
        ("block", ctypes.c_int32), ("segment", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32), ("k_min", ctypes.c_int32),
        ("top_p", ctypes.c_float), ("sm_scale", ctypes.c_float),
        ("score_kind", ctypes.c_int32), ("h_idx", ctypes.c_int32), ("d_idx", ctypes.c_int32),
    ]


class SpotError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspot.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m block_sparse_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    D = ctypes.POINTER(spot_desc)
    lib.spot_version.restype = I
    lib.spot_status_string.restype = ctypes.c_char_p
    lib.spot_status_string.argtypes = [I]
    lib.spot_last_error.restype = ctypes.c_char_p
    lib.spot_workspace_size.argtypes = [D, I, ctypes.POINTER(S)]
    lib.spot_block_score.argtypes = [D, P, P, P, P, P, P, P, P, S, P]
    lib.spot_select_topp.argtypes = [D, P, P, P, P, S, P]
    lib.spot_sparse_attn_prefill.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
    lib.spot_sparse_attn_decode.argtypes = [D, P, P, P, P, P, P, P, P, S, P]
    lib.spot_key_permutation.argtypes = [D, P, P, P, P, P, S, P]
    lib.spot_order_history.argtypes = [D, P, P, P, P, S, P]
    lib.spot_quantize_indexer_keys.argtypes = [D, P, P, P, P]
    lib.spot_indexer_score_mxfp4.argtypes = [D, P, P, P, P, P, P]
    lib.spot_history_map.argtypes = [D, P, P, P, P, S, P]
    lib.spot_sparse_attn_prefill_history_map.argtypes = [D, ctypes.c_float, P, P, P, P, P, P, P, P, S, P]
    lib.spot_sparse_attn_prefill_early_stop.argtypes = [D, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.spot_validate_perm.argtypes = [D, P, P, P]
    lib.spot_sparse_attn_decode_noalloc.argtypes = [D, P, P, P, P, P, P, P, P]
    lib.spot_quantize_indexer_keys_int4.argtypes = [D, P, P, P, P]
    lib.spot_indexer_score_int4.argtypes = [D, P, P, P, P, P, P]
    lib.spot_rla_block_states.argtypes = [D, P, P, P, P, P, P]
    lib.spot_rla_prefill.argtypes = [D, P, P, P, P, P, P, P]
    lib.spot_rla_decode_state.argtypes = [D, P, P, P, P, S, P]
    lib.spot_rla_decode.argtypes = [D, P, P, P, P, P, P, P, P, S, P]
    lib.spot_sparse_attn_decode_rla.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
    for name in EXPORTS[3:]:
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, st: int) -> None:
    if st != SPOT_OK:
        raise SpotError(fn, st, load_library().spot_last_error().decode())


# ----------------------------------------------------------------- raw C ABI
def spot_version() -> int:
    return load_library().spot_version()


def spot_workspace_size(desc: spot_desc, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("spot_workspace_size", load_library().spot_workspace_size(ctypes.byref(desc), op, ctypes.byref(n)))
    return n.value


def spot_block_score(desc, q, k, perm, idx_q, idx_w, idx_k, scores, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_block_score(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(perm), _ptr(idx_q), _ptr(idx_w),
                                         _ptr(idx_k), _ptr(scores), _ptr(workspace), ws_bytes,
                                         _stream() if stream is None else stream)
    _check("spot_block_score", st)


def spot_select_topp(desc, scores, idx, cnt, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_select_topp(ctypes.byref(desc), _ptr(scores), _ptr(idx), _ptr(cnt), _ptr(workspace),
                                         ws_bytes, _stream() if stream is None else stream)
    _check("spot_select_topp", st)


def spot_sparse_attn_prefill(desc, q, k, v, perm, idx, cnt, o, lse=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_sparse_attn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(perm),
                                                 _ptr(idx), _ptr(cnt), _ptr(o), _ptr(lse), _ptr(workspace),
                                                 ws_bytes, _stream() if stream is None else stream)
    _check("spot_sparse_attn_prefill", st)


def spot_sparse_attn_decode(desc, q, k_cache, v_cache, idx, cnt, o, lse=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_sparse_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                _ptr(idx), _ptr(cnt), _ptr(o), _ptr(lse), _ptr(workspace),
                                                ws_bytes, _stream() if stream is None else stream)
    _check("spot_sparse_attn_decode", st)


def spot_sparse_attn_decode_noalloc(desc, q, k_cache, v_cache, idx, cnt, o, lse=None, stream=None):
    st = load_library().spot_sparse_attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                        _ptr(idx), _ptr(cnt), _ptr(o), _ptr(lse),
                                                        _stream() if stream is None else stream)
    _check("spot_sparse_attn_decode_noalloc", st)


def spot_key_permutation(desc, q, k, perm, importance=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_key_permutation(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(perm), _ptr(importance),
                                             _ptr(workspace), ws_bytes, _stream() if stream is None else stream)
    _check("spot_key_permutation", st)


def spot_validate_perm(desc, perm, bad, stream=None):
    st = load_library().spot_validate_perm(ctypes.byref(desc), _ptr(perm), _ptr(bad),
                                           _stream() if stream is None else stream)
    _check("spot_validate_perm", st)


def spot_quantize_indexer_keys(desc, idx_k, k_codes, k_scales, stream=None):
    st = load_library().spot_quantize_indexer_keys(ctypes.byref(desc), _ptr(idx_k), _ptr(k_codes), _ptr(k_scales),
                                                   _stream() if stream is None else stream)
    _check("spot_quantize_indexer_keys", st)


def spot_indexer_score_mxfp4(desc, idx_q, idx_w, k_codes, k_scales, scores, stream=None):
    st = load_library().spot_indexer_score_mxfp4(ctypes.byref(desc), _ptr(idx_q), _ptr(idx_w), _ptr(k_codes),
                                                 _ptr(k_scales), _ptr(scores), _stream() if stream is None else stream)
    _check("spot_indexer_score_mxfp4", st)


def spot_quantize_indexer_keys_int4(desc, idx_k, k_codes, k_scales, stream=None):
    st = load_library().spot_quantize_indexer_keys_int4(ctypes.byref(desc), _ptr(idx_k), _ptr(k_codes),
                                                        _ptr(k_scales), _stream() if stream is None else stream)
    _check("spot_quantize_indexer_keys_int4", st)


def spot_indexer_score_int4(desc, idx_q, idx_w, k_codes, k_scales, scores, stream=None):
    st = load_library().spot_indexer_score_int4(ctypes.byref(desc), _ptr(idx_q), _ptr(idx_w), _ptr(k_codes),
                                                _ptr(k_scales), _ptr(scores), _stream() if stream is None else stream)
    _check("spot_indexer_score_int4", st)


def spot_history_map(desc, q, k, hmap, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_history_map(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(hmap), _ptr(workspace), ws_bytes,
                                         _stream() if stream is None else stream)
    _check("spot_history_map", st)


def spot_sparse_attn_prefill_history_map(desc, tau, q, k, v, hmap, o, lse=None, nused=None, workspace=None,
                                         stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_sparse_attn_prefill_history_map(
        ctypes.byref(desc), float(tau), _ptr(q), _ptr(k), _ptr(v), _ptr(hmap), _ptr(o), _ptr(lse), _ptr(nused),
        _ptr(workspace), ws_bytes, _stream() if stream is None else stream)
    _check("spot_sparse_attn_prefill_history_map", st)


def spot_order_history(desc, scores, order, cnt, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_order_history(ctypes.byref(desc), _ptr(scores), _ptr(order), _ptr(cnt), _ptr(workspace),
                                           ws_bytes, _stream() if stream is None else stream)
    _check("spot_order_history", st)


def spot_sparse_attn_prefill_early_stop(desc, tau, q, k, v, perm, order, cnt, o, lse=None, nused=None,
                                        workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_sparse_attn_prefill_early_stop(
        ctypes.byref(desc), float(tau), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(order), _ptr(cnt), _ptr(o),
        _ptr(lse), _ptr(nused), _ptr(workspace), ws_bytes, _stream() if stream is None else stream)
    _check("spot_sparse_attn_prefill_early_stop", st)


def spot_rla_block_states(desc, k, v, perm, states, states_perm=None, stream=None):
    st = load_library().spot_rla_block_states(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(perm), _ptr(states),
                                              _ptr(states_perm), _stream() if stream is None else stream)
    _check("spot_rla_block_states", st)


def spot_rla_prefill(desc, q, states, states_perm, idx, cnt, o_rla, stream=None):
    st = load_library().spot_rla_prefill(ctypes.byref(desc), _ptr(q), _ptr(states), _ptr(states_perm), _ptr(idx),
                                         _ptr(cnt), _ptr(o_rla), _stream() if stream is None else stream)
    _check("spot_rla_prefill", st)


def spot_rla_decode_state(desc, k_cache, v_cache, state, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_rla_decode_state(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(state),
                                              _ptr(workspace), ws_bytes, _stream() if stream is None else stream)
    _check("spot_rla_decode_state", st)


def spot_rla_decode(desc, q, k_cache, v_cache, state, idx, cnt, o_rla, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_rla_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(state),
                                        _ptr(idx), _ptr(cnt), _ptr(o_rla), _ptr(workspace), ws_bytes,
                                        _stream() if stream is None else stream)
    _check("spot_rla_decode", st)


def spot_sparse_attn_decode_rla(desc, q, k_cache, v_cache, idx, cnt, rla_state, o, lse, o_rla, workspace=None,
                                stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().spot_sparse_attn_decode_rla(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                    _ptr(idx), _ptr(cnt), _ptr(rla_state), _ptr(o), _ptr(lse),
                                                    _ptr(o_rla), _ptr(workspace), ws_bytes,
                                                    _stream() if stream is None else stream)
    _check("spot_sparse_attn_decode_rla", st)


# ----------------------------------------------------------------- descriptors
def make_desc(*, dtype: int, batch: int, hq: int, hkv: int, d: int, q_len: int, kv_len: int, block: int,
              segment: int = 0, n_sink: int = 1, n_recent: int = 1, k_min: int = 0, top_p: float = 0.9,
              sm_scale: float = 0.0, score_kind: int = SPOT_SCORE_MEANPOOL, h_idx: int = 0,
              d_idx: int = 0) -> spot_desc:
    return spot_desc(ABI_VERSION, dtype, batch, hq, hkv, d, q_len, kv_len, block, segment, n_sink, n_recent, k_min,
                     top_p, sm_scale, score_kind, h_idx, d_idx)


def torch_dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPOT_BF16
    if t.dtype == torch.float32:
        return SPOT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _require(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ----------------------------------------------------------------- pipelines
@dataclass
class PrefillBuffers:
    scores: torch.Tensor
    idx: torch.Tensor
    cnt: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    workspace: torch.Tensor


def prefill_desc(q: torch.Tensor, k: torch.Tensor, block: int, top_p: float, *, segment: int = 0, n_sink: int = 1,
                 n_recent: int = 1, k_min: int = 0, sm_scale: float = 0.0,
                 score_kind: int = SPOT_SCORE_MEANPOOL) -> spot_desc:
    b, hq, L, d = q.shape
    return make_desc(dtype=torch_dtype_code(q), batch=b, hq=hq, hkv=k.shape[1], d=d, q_len=L, kv_len=L, block=block,
                     segment=segment, n_sink=n_sink, n_recent=n_recent, k_min=k_min, top_p=top_p, sm_scale=sm_scale,
                     score_kind=score_kind)


def alloc_prefill(desc: spot_desc, device) -> PrefillBuffers:
    nb = -(-desc.q_len // desc.block)
    rows = (desc.batch, desc.hkv, nb)
    ws = spot_workspace_size(desc, SPOT_OP_BLOCK_SCORE)
    odt = torch.bfloat16 if desc.dtype == SPOT_BF16 else torch.float32
    return PrefillBuffers(
        scores=torch.empty(*rows, nb, dtype=torch.float32, device=device),
        idx=torch.empty(*rows, nb, dtype=torch.int32, device=device),
        cnt=torch.empty(*rows, dtype=torch.int32, device=device),
        o=torch.empty(desc.batch, desc.hq, desc.q_len, desc.d, dtype=odt, device=device),
        lse=torch.empty(desc.batch, desc.hq, desc.q_len, dtype=torch.float32, device=device),
        workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device),
    )


def prefill(q, k, v, block: int, top_p: float, *, perm=None, segment: int = 0, n_sink: int = 1, n_recent: int = 1,
            k_min: int = 0, sm_scale: float = 0.0, score_kind: int = SPOT_SCORE_MEANPOOL,
            bufs: PrefillBuffers | None = None) -> PrefillBuffers:
    """Whole prefill path: block scores -> top-p selection -> sparse attention.

    q (batch, hq, L, d), k/v (batch, hkv, L, d) bf16 or fp32 device tensors;
    perm (batch, hkv, L) int32 or None; score_kind MEANPOOL or TAYLOR.
    """
    desc = prefill_desc(q, k, block, top_p, segment=segment, n_sink=n_sink, n_recent=n_recent, k_min=k_min,
                        sm_scale=sm_scale, score_kind=score_kind)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, dtype=q.dtype)
    if perm is not None:
        _require(perm, "perm", dtype=torch.int32, shape=(k.shape[0], k.shape[1], k.shape[2]))
    if bufs is None:
        bufs = alloc_prefill(desc, q.device)
    spot_block_score(desc, q, k, perm, None, None, None, bufs.scores, bufs.workspace)
    spot_select_topp(desc, bufs.scores, bufs.idx, bufs.cnt)
    spot_sparse_attn_prefill(desc, q, k, v, perm, bufs.idx, bufs.cnt, bufs.o, bufs.lse)
    return bufs


def key_permutation(q, k, block: int, segment: int, *, sm_scale: float = 0.0, with_importance: bool = False):
    """Intra-segment key permutation by last-query-block importance.

    q (batch, hq, L, d), k (batch, hkv, L, d) bf16 device tensors.  Returns
    perm (batch, hkv, L) int32 [and importance (batch, hkv, L) fp32]."""
    _require(q, "q", dtype=torch.bfloat16)
    _require(k, "k", dtype=torch.bfloat16)
    desc = prefill_desc(q, k, block, 1.0, segment=segment, sm_scale=sm_scale)
    ws = torch.empty(max(spot_workspace_size(desc, SPOT_OP_KEY_PERMUTATION), 1), dtype=torch.uint8, device=q.device)
    perm = torch.empty(k.shape[0], k.shape[1], k.shape[2], dtype=torch.int32, device=q.device)
    imp = torch.empty(perm.shape, dtype=torch.float32, device=q.device) if with_importance else None
    spot_key_permutation(desc, q, k, perm, imp, ws)
    return (perm, imp) if with_importance else perm


@dataclass
class EarlyStopBuffers:
    scores: torch.Tensor
    order: torch.Tensor
    cnt: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    nused: torch.Tensor
    workspace: torch.Tensor


def alloc_prefill_early_stop(desc: spot_desc, device) -> EarlyStopBuffers:
    nb = -(-desc.q_len // desc.block)
    rows = (desc.batch, desc.hkv, nb)
    ws = spot_workspace_size(desc, SPOT_OP_BLOCK_SCORE)
    return EarlyStopBuffers(
        scores=torch.empty(*rows, nb, dtype=torch.float32, device=device),
        order=torch.empty(*rows, nb, dtype=torch.int32, device=device),
        cnt=torch.empty(*rows, dtype=torch.int32, device=device),
        o=torch.empty(desc.batch, desc.hq, desc.q_len, desc.d, dtype=torch.bfloat16, device=device),
        lse=torch.empty(desc.batch, desc.hq, desc.q_len, dtype=torch.float32, device=device),
        nused=torch.empty(desc.batch, desc.hq, desc.q_len, dtype=torch.int32, device=device),
        workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device),
    )


def prefill_early_stop(q, k, v, block: int, segment: int, tau: float, *, perm=None, sm_scale: float = 0.0,
                       bufs: EarlyStopBuffers | None = None) -> EarlyStopBuffers:
    """Early-stopped prefill: block scores -> history visiting order ->
    attention that stops taking history blocks per row once their gain
    falls below tau.

    q (batch, hq, L, d), k/v (batch, hkv, L, d) bf16 device tensors;
    perm (batch, hkv, L) int32 or None.
    """
    desc = prefill_desc(q, k, block, 1.0, segment=segment, sm_scale=sm_scale)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, dtype=torch.bfloat16)
    if perm is not None:
        _require(perm, "perm", dtype=torch.int32, shape=(k.shape[0], k.shape[1], k.shape[2]))
    if bufs is None:
        bufs = alloc_prefill_early_stop(desc, q.device)
    spot_block_score(desc, q, k, perm, None, None, None, bufs.scores, bufs.workspace)
    spot_order_history(desc, bufs.scores, bufs.order, bufs.cnt)
    spot_sparse_attn_prefill_early_stop(desc, tau, q, k, v, perm, bufs.order, bufs.cnt, bufs.o, bufs.lse, bufs.nused)
    return bufs


def history_map(q, k, segment: int, *, sm_scale: float = 0.0, workspace=None):
    """Per-segment history maps by the segment's mean query.

    q (batch, hq, L, d), k (batch, hkv, L, d) bf16 device tensors.  Returns
    hmap (batch, hkv, nseg, L) int32."""
    _require(q, "q", dtype=torch.bfloat16)
    _require(k, "k", dtype=torch.bfloat16)
    desc = prefill_desc(q, k, segment, 1.0, segment=segment, sm_scale=sm_scale)
    desc.block = 16   # the map does not depend on the block size
    nseg = -(-q.shape[2] // segment)
    hmap = torch.empty(k.shape[0], k.shape[1], nseg, k.shape[2], dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(spot_workspace_size(desc, SPOT_OP_HISTORY_MAP), 1), dtype=torch.uint8,
                                device=q.device)
    spot_history_map(desc, q, k, hmap, workspace)
    return hmap


def prefill_history_map(q, k, v, block: int, segment: int, tau: float, *, hmap=None, sm_scale: float = 0.0,
                        bufs: EarlyStopBuffers | None = None) -> EarlyStopBuffers:
    """Early-stopped prefill on per-segment history maps (computed here when
    `hmap` is None).  Returns buffers with o, lse and nused (scores, order and
    cnt are not used)."""
    desc = prefill_desc(q, k, block, 1.0, segment=segment, sm_scale=sm_scale)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, dtype=torch.bfloat16)
    if hmap is None:
        hmap = history_map(q, k, segment, sm_scale=sm_scale)
    if bufs is None:
        bufs = alloc_prefill_early_stop(desc, q.device)
    spot_sparse_attn_prefill_history_map(desc, tau, q, k, v, hmap, bufs.o, bufs.lse, bufs.nused)
    return bufs


@dataclass
class RlaPrefillBuffers:
    states: torch.Tensor
    states_perm: torch.Tensor | None
    o_rla: torch.Tensor


def rla_prefill(desc: spot_desc, q, k, v, idx, cnt, *, perm=None,
                bufs: RlaPrefillBuffers | None = None) -> RlaPrefillBuffers:
    """Residual linear attention of every query row over the visible keys
    outside its kept blocks: block states, then the per-block residual.

    desc: the prefill descriptor of the selection; q, k, v as for prefill;
    idx/cnt the kept lists of spot_select_topp; perm as for the attention.
    Returns buffers whose o_rla is fp32 (batch, hq, L, d)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, dtype=q.dtype)
    nb = -(-desc.q_len // desc.block)
    if bufs is None:
        shape = (desc.batch, desc.hkv, nb, desc.d, desc.d)
        bufs = RlaPrefillBuffers(
            states=torch.empty(shape, dtype=torch.float32, device=q.device),
            states_perm=torch.empty(shape, dtype=torch.float32, device=q.device) if perm is not None else None,
            o_rla=torch.empty(desc.batch, desc.hq, desc.q_len, desc.d, dtype=torch.float32, device=q.device))
    spot_rla_block_states(desc, k, v, perm, bufs.states, bufs.states_perm)
    spot_rla_prefill(desc, q, bufs.states, bufs.states_perm, idx, cnt, bufs.o_rla)
    return bufs


def rla_decode_state(desc: spot_desc, k_cache, v_cache):
    """State of the whole cache for decode residual linear attention:
    fp32 (batch, hkv, d, d) = sum over the cache of exp(k) v^T."""
    _require(k_cache, "k_cache", dtype=torch.bfloat16)
    _require(v_cache, "v_cache", dtype=torch.bfloat16)
    ws = torch.empty(max(spot_workspace_size(desc, SPOT_OP_RLA_DECODE_STATE), 1), dtype=torch.uint8,
                     device=k_cache.device)
    state = torch.empty(desc.batch, desc.hkv, desc.d, desc.d, dtype=torch.float32, device=k_cache.device)
    spot_rla_decode_state(desc, k_cache, v_cache, state, ws)
    return state


def rla_decode(desc: spot_desc, q, k_cache, v_cache, state, idx, cnt, o_rla=None, workspace=None):
    """Residual linear attention of the decode queries: fp32 (batch, hq, d)."""
    if o_rla is None:
        o_rla = torch.empty(desc.batch, desc.hq, desc.d, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(spot_workspace_size(desc, SPOT_OP_RLA_DECODE), 1), dtype=torch.uint8,
                                device=q.device)
    spot_rla_decode(desc, q, k_cache, v_cache, state, idx, cnt, o_rla, workspace)
    return o_rla


@dataclass
class DecodeBuffers:
    scores: torch.Tensor
    idx: torch.Tensor
    cnt: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    workspace: torch.Tensor


def decode_desc(q, k_cache, block: int, top_p: float, h_idx: int, d_idx: int, *, n_sink: int = 1, n_recent: int = 1,
                k_min: int = 0, sm_scale: float = 0.0) -> spot_desc:
    b, hq, d = q.shape
    return make_desc(dtype=torch_dtype_code(q), batch=b, hq=hq, hkv=k_cache.shape[1], d=d, q_len=1,
                     kv_len=k_cache.shape[2], block=block, n_sink=n_sink, n_recent=n_recent, k_min=k_min,
                     top_p=top_p, sm_scale=sm_scale, score_kind=SPOT_SCORE_RELU_INDEXER, h_idx=h_idx, d_idx=d_idx)


def alloc_decode(desc: spot_desc, device) -> DecodeBuffers:
    nk = -(-desc.kv_len // desc.block)
    ws = spot_workspace_size(desc, SPOT_OP_DECODE)
    return DecodeBuffers(
        scores=torch.empty(desc.batch, 1, 1, nk, dtype=torch.float32, device=device),
        idx=torch.empty(desc.batch, 1, 1, nk, dtype=torch.int32, device=device),
        cnt=torch.empty(desc.batch, 1, 1, dtype=torch.int32, device=device),
        o=torch.empty(desc.batch, desc.hq, desc.d, dtype=torch.bfloat16, device=device),
        lse=torch.empty(desc.batch, desc.hq, dtype=torch.float32, device=device),
        workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device),
    )


def quantize_indexer_keys(idx_k, block: int, kv_len: int):
    """MXFP4 encoding of the indexer keys idx_k (batch, nT, h_idx, d_idx) bf16.
    Returns (codes uint8 (batch, nT, h_idx*d_idx/2), scales uint8 (batch, nT, h_idx*d_idx/32))."""
    _require(idx_k, "idx_k", dtype=torch.bfloat16)
    b, nt, h_idx, d_idx = idx_k.shape
    desc = make_desc(dtype=SPOT_BF16, batch=b, hq=1, hkv=1, d=128, q_len=1, kv_len=kv_len, block=block,
                     score_kind=SPOT_SCORE_RELU_INDEXER, h_idx=h_idx, d_idx=d_idx)
    codes = torch.empty(b, nt, h_idx * d_idx // 2, dtype=torch.uint8, device=idx_k.device)
    scales = torch.empty(b, nt, h_idx * d_idx // 32, dtype=torch.uint8, device=idx_k.device)
    spot_quantize_indexer_keys(desc, idx_k, codes, scales)
    return codes, scales


def quantize_indexer_keys_int4(idx_k, block: int, kv_len: int):
    """INT4 encoding of the indexer keys idx_k (batch, nT, h_idx, d_idx) bf16.
    Returns (codes uint8 (batch, nT, h_idx*d_idx/2), scales bf16 (batch, nT, h_idx*d_idx/32))."""
    _require(idx_k, "idx_k", dtype=torch.bfloat16)
    b, nt, h_idx, d_idx = idx_k.shape
    desc = make_desc(dtype=SPOT_BF16, batch=b, hq=1, hkv=1, d=128, q_len=1, kv_len=kv_len, block=block,
                     score_kind=SPOT_SCORE_RELU_INDEXER, h_idx=h_idx, d_idx=d_idx)
    codes = torch.empty(b, nt, h_idx * d_idx // 2, dtype=torch.uint8, device=idx_k.device)
    scales = torch.empty(b, nt, h_idx * d_idx // 32, dtype=torch.bfloat16, device=idx_k.device)
    spot_quantize_indexer_keys_int4(desc, idx_k, codes, scales)
    return codes, scales


def decode(q, k_cache, v_cache, idx_q, idx_w, idx_k, block: int, top_p: float, *, n_sink: int = 1,
           n_recent: int = 1, k_min: int = 0, sm_scale: float = 0.0,
           bufs: DecodeBuffers | None = None) -> DecodeBuffers:
    """Whole decode step: indexer scores -> top-p selection -> sparse attention.

    q (batch, hq, d) bf16; k_cache/v_cache (batch, hkv, T, d) bf16;
    idx_q (batch, h_idx, d_idx) bf16; idx_w (batch, h_idx) fp32;
    idx_k (batch, nT, h_idx, d_idx) bf16, or an encoding of it as the pair
    (codes, scales): uint8 scales are MXFP4 (quantize_indexer_keys), bf16
    scales INT4 (quantize_indexer_keys_int4).
    """
    h_idx, d_idx = idx_q.shape[1], idx_q.shape[2]
    desc = decode_desc(q, k_cache, block, top_p, h_idx, d_idx, n_sink=n_sink, n_recent=n_recent, k_min=k_min,
                       sm_scale=sm_scale)
    mx = isinstance(idx_k, tuple)
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("idx_q", idx_q)):
        _require(t, name, dtype=torch.bfloat16)
    if mx:
        _require(idx_k[0], "k_codes", dtype=torch.uint8)
        if idx_k[1].dtype != torch.bfloat16:
            _require(idx_k[1], "k_scales", dtype=torch.uint8)
    else:
        _require(idx_k, "idx_k", dtype=torch.bfloat16)
    _require(idx_w, "idx_w", dtype=torch.float32)
    if bufs is None:
        bufs = alloc_decode(desc, q.device)
    if mx and idx_k[1].dtype == torch.bfloat16:
        _require(idx_k[1], "k_scales", dtype=torch.bfloat16)
        spot_indexer_score_int4(desc, idx_q, idx_w, idx_k[0], idx_k[1], bufs.scores)
    elif mx:
        spot_indexer_score_mxfp4(desc, idx_q, idx_w, idx_k[0], idx_k[1], bufs.scores)
    else:
        spot_block_score(desc, None, None, None, idx_q, idx_w, idx_k, bufs.scores)
    spot_select_topp(desc, bufs.scores, bufs.idx, bufs.cnt)
    spot_sparse_attn_decode(desc, q, k_cache, v_cache, bufs.idx, bufs.cnt, bufs.o, bufs.lse, bufs.workspace)
    return bufs


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
