// C ABI of libspot: host-side validation, workspace sizing and dispatch.
// Nothing here allocates, frees or synchronises; kernels are enqueued on the
// caller's stream.  Every check happens before the first launch, so a failed
// call enqueues nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/spot.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("SPOT_LOG");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPOT_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  if (log_enabled()) std::fprintf(stderr, "[spot] %s launched\n", what);
  g_err.clear();
  return SPOT_OK;
}

bool pow2_block(int b) { return b == 16 || b == 32 || b == 64 || b == 128; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks shared by all calls.
int check_common(const spot_desc* d) {
  if (!d) return fail(SPOT_ERR_INVALID, "desc is NULL");
  if (d->version != SPOT_ABI_VERSION) return fail(SPOT_ERR_INVALID, "desc.version %d != %d", d->version, SPOT_ABI_VERSION);
  if (d->dtype != SPOT_F32 && d->dtype != SPOT_BF16) return fail(SPOT_ERR_INVALID, "unknown dtype %d", d->dtype);
  if (d->batch < 1 || d->hq < 1 || d->hkv < 1) return fail(SPOT_ERR_INVALID, "batch, hq and hkv must be >= 1");
  if (d->hq % d->hkv) return fail(SPOT_ERR_INVALID, "hq (%d) not a multiple of hkv (%d)", d->hq, d->hkv);
  if (d->d != 64 && d->d != 128) return fail(SPOT_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d->d);
  if (!pow2_block(d->block)) return fail(SPOT_ERR_UNSUPPORTED, "block %d (supported: 16, 32, 64, 128)", d->block);
  if (d->q_len < 1 || d->kv_len < 1) return fail(SPOT_ERR_INVALID, "q_len and kv_len must be >= 1");
  if (d->kv_len > (int64_t(1) << 30)) return fail(SPOT_ERR_UNSUPPORTED, "kv_len %lld too long", (long long)d->kv_len);
  if (!(std::isfinite(d->sm_scale)) || d->sm_scale < 0.f) return fail(SPOT_ERR_INVALID, "sm_scale must be finite and >= 0");
  return SPOT_OK;
}

bool is_decode(const spot_desc* d) { return d->q_len == 1 && d->score_kind == SPOT_SCORE_RELU_INDEXER; }

int check_prefill_shape(const spot_desc* d) {
  if (d->q_len != d->kv_len) return fail(SPOT_ERR_INVALID, "prefill needs q_len == kv_len");
  if (d->segment < 0) return fail(SPOT_ERR_INVALID, "segment must be >= 0");
  if (d->segment > 0 && d->segment % d->block) return fail(SPOT_ERR_INVALID, "segment %d not a multiple of block %d", d->segment, d->block);
  const int64_t nb = ceil_div64(d->q_len, d->block);
  if (nb > 65536) return fail(SPOT_ERR_UNSUPPORTED, "%lld blocks per sequence (max 65536)", (long long)nb);
  return SPOT_OK;
}

int check_selection_params(const spot_desc* d) {
  if (d->n_sink < 0 || d->n_recent < 0 || d->k_min < 0) return fail(SPOT_ERR_INVALID, "n_sink, n_recent, k_min must be >= 0");
  if (d->n_sink + d->n_recent < 1) return fail(SPOT_ERR_INVALID, "n_sink + n_recent must be >= 1");
  if (std::isnan(d->top_p)) return fail(SPOT_ERR_INVALID, "top_p is NaN");
  return SPOT_OK;
}

float effective_scale(const spot_desc* d) {
  return d->sm_scale > 0.f ? d->sm_scale : 1.0f / std::sqrt(float(d->d));
}

bool is_pooled(const spot_desc* d) {
  return d->score_kind == SPOT_SCORE_MEANPOOL || d->score_kind == SPOT_SCORE_TAYLOR;
}

// pooled statistics: qbar, kbar natural, kbar permuted (+ K variances natural and permuted for TAYLOR)
size_t meanpool_ws_bytes(const spot_desc* d) {
  const size_t nb = size_t(ceil_div64(d->q_len, d->block));
  const size_t slabs = d->score_kind == SPOT_SCORE_TAYLOR ? 5 : 3;
  return slabs * d->batch * d->hkv * nb * d->d * sizeof(float);
}

// 16-byte vector loads and stores need 16-byte aligned bases (hipMalloc and torch give 256)
int check_aligned16(const char* what, const void* p) {
  if (p && (reinterpret_cast<uintptr_t>(p) & 15u))
    return fail(SPOT_ERR_INVALID, "%s must be 16-byte aligned", what);
  return SPOT_OK;
}

// The bf16 attention kernels read q in 16-byte pieces and k, v with 16-byte
// buffer-to-LDS loads, and write o in 8-byte pieces.
int check_mfma_operands(const void* q, const void* k, const void* v, const void* o) {
  int st;
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("k", k)) || (st = check_aligned16("v", v))) return st;
  if (reinterpret_cast<uintptr_t>(o) & 7u) return fail(SPOT_ERR_INVALID, "o must be 8-byte aligned");
  return SPOT_OK;
}

int check_workspace(size_t need, const void* ws, size_t have) {
  if (need == 0) return SPOT_OK;
  if (!ws || have < need) return fail(SPOT_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? have : size_t(0), need);
  return SPOT_OK;
}

int check_indexer(const spot_desc* d) {
  if (d->d_idx != 16 && d->d_idx != 32 && d->d_idx != 64 && d->d_idx != 128)
    return fail(SPOT_ERR_UNSUPPORTED, "d_idx %d (supported: 16, 32, 64, 128)", d->d_idx);
  if (d->h_idx < 1 || d->h_idx * d->d_idx > 256) return fail(SPOT_ERR_UNSUPPORTED, "h_idx*d_idx must be in [1, 256]");
  return SPOT_OK;
}

}  // namespace

extern "C" {

int spot_version(void) { return SPOT_ABI_VERSION; }

const char* spot_status_string(int status) {
  switch (status) {
    case SPOT_OK: return "ok";
    case SPOT_ERR_INVALID: return "invalid argument";
    case SPOT_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SPOT_ERR_WORKSPACE: return "workspace too small";
    case SPOT_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* spot_last_error(void) { return g_err.c_str(); }

int spot_workspace_size(const spot_desc* desc, int op, size_t* bytes) {
  if (!bytes) return fail(SPOT_ERR_INVALID, "bytes is NULL");
  *bytes = 0;
  int st = check_common(desc);
  if (st) return st;
  switch (op) {
    case SPOT_OP_BLOCK_SCORE:
      if (is_pooled(desc)) {
        if ((st = check_prefill_shape(desc))) return st;
        *bytes = meanpool_ws_bytes(desc);
      } else if (desc->score_kind != SPOT_SCORE_RELU_INDEXER) {
        return fail(SPOT_ERR_INVALID, "unknown score_kind %d", desc->score_kind);
      }
      break;
    case SPOT_OP_SELECT_TOPP:
    case SPOT_OP_PREFILL:
    case SPOT_OP_ORDER_HISTORY:
    case SPOT_OP_PREFILL_EARLY_STOP:
      break;
    case SPOT_OP_HISTORY_MAP: {
      if ((st = check_prefill_shape(desc))) return st;
      if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
      const int nseg = int(ceil_div64(desc->q_len, desc->segment));
      *bytes = spot::hist_workspace_bytes(desc->batch, desc->hkv, nseg, desc->segment, desc->d);
      break;
    }
    case SPOT_OP_KEY_PERMUTATION: {
      if ((st = check_prefill_shape(desc))) return st;
      const int nb = int(ceil_div64(desc->q_len, desc->block));
      const int nr = int(desc->q_len - int64_t(nb - 1) * desc->block);
      *bytes = spot::perm_workspace_bytes(desc->batch, desc->hkv, int(desc->q_len), desc->hq / desc->hkv, nr);
      break;
    }
    case SPOT_OP_RLA_DECODE_STATE: {
      const size_t nr = size_t(ceil_div64(desc->kv_len, spot::kRlaDecodeSpan));
      *bytes = size_t(desc->batch) * desc->hkv * nr * desc->d * desc->d * sizeof(float);
      break;
    }
    case SPOT_OP_DECODE_RLA: {
      const int nk = int(ceil_div64(desc->kv_len, desc->block));
      const int ns = spot::decode_num_splits(desc->batch, desc->hkv, nk);
      *bytes = spot::decode_partials_bytes(desc->batch, desc->hq, desc->d, ns) +
               size_t(desc->batch) * desc->hq * ns * desc->d * sizeof(float);
      break;
    }
    case SPOT_OP_RLA_DECODE: {
      const size_t ns = size_t(spot::rla_decode_num_splits(desc->batch, desc->hkv));
      *bytes = size_t(desc->batch) * desc->hq * ns * desc->d * sizeof(float);
      break;
    }
    case SPOT_OP_DECODE: {
      const int nk = int(ceil_div64(desc->kv_len, desc->block));
      const int ns = spot::decode_num_splits(desc->batch, desc->hkv, nk);
      *bytes = spot::decode_partials_bytes(desc->batch, desc->hq, desc->d, ns);
      break;
    }
    default:
      return fail(SPOT_ERR_INVALID, "unknown op %d", op);
  }
  g_err.clear();
  return SPOT_OK;
}

int spot_block_score(const spot_desc* desc, const void* q, const void* k, const int32_t* perm, const void* idx_q,
                     const float* idx_w, const void* idx_k, float* scores, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if (!scores) return fail(SPOT_ERR_INVALID, "scores is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (is_pooled(desc)) {
    if ((st = check_prefill_shape(desc))) return st;
    if (!q || !k) return fail(SPOT_ERR_INVALID, "q and k are required for MEANPOOL and TAYLOR");
    if ((st = check_aligned16("q", q)) || (st = check_aligned16("k", k))) return st;   // 16-byte row loads
    if (perm && desc->segment <= 0) return fail(SPOT_ERR_INVALID, "perm given but segment is 0");
    const size_t need = meanpool_ws_bytes(desc);
    if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
    const int nb = int(ceil_div64(desc->q_len, desc->block));
    const size_t slab = size_t(desc->batch) * desc->hkv * nb * desc->d;
    float* ws = static_cast<float*>(workspace);
    const bool taylor = desc->score_kind == SPOT_SCORE_TAYLOR;
    spot::PoolArgs pa{q, k, perm, ws, ws + slab, ws + 2 * slab, desc->dtype == SPOT_BF16, desc->batch, desc->hq,
                      desc->hkv, desc->d, int(desc->q_len), desc->block, nb};
    if (taylor) {
      pa.kvar_nat = ws + 3 * slab;
      pa.kvar_perm = ws + 4 * slab;
    }
    hipError_t e = spot::launch_pool_blocks(pa, s);
    if (e != hipSuccess) return launched(e, "pool_blocks");
    spot::MeanpoolScoreArgs sa{ws, ws + slab, perm ? ws + 2 * slab : nullptr, scores, desc->batch, desc->hkv,
                               desc->d, nb, desc->block, desc->segment, effective_scale(desc)};
    if (taylor) {
      sa.var_nat = ws + 3 * slab;
      sa.var_perm = perm ? ws + 4 * slab : nullptr;
    }
    return launched(spot::launch_meanpool_score(sa, s), "meanpool_score");
  }
  if (desc->score_kind == SPOT_SCORE_RELU_INDEXER) {
    if ((st = check_indexer(desc))) return st;
    if (!idx_q || !idx_w || !idx_k) return fail(SPOT_ERR_INVALID, "idx_q, idx_w and idx_k are required for RELU_INDEXER");
    if ((st = check_aligned16("idx_q", idx_q)) || (st = check_aligned16("idx_k", idx_k))) return st;
    const int nk = int(ceil_div64(desc->kv_len, desc->block));
    spot::IndexerScoreArgs ia{static_cast<const uint16_t*>(idx_q), idx_w, static_cast<const uint16_t*>(idx_k), scores,
                              desc->batch, nk, desc->h_idx, desc->d_idx};
    return launched(spot::launch_indexer_score(ia, s), "indexer_score");
  }
  return fail(SPOT_ERR_INVALID, "unknown score_kind %d", desc->score_kind);
}

int spot_select_topp(const spot_desc* desc, const float* scores, int32_t* idx, int32_t* cnt, void* workspace,
                     size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_selection_params(desc))) return st;
  if (!scores || !idx || !cnt) return fail(SPOT_ERR_INVALID, "scores, idx and cnt are required");
  const int64_t nk = ceil_div64(desc->kv_len, desc->block);
  if (nk > spot::kSelectMaxCandidates)
    return fail(SPOT_ERR_UNSUPPORTED, "%lld candidate blocks per row (max %d)", (long long)nk, spot::kSelectMaxCandidates);
  spot::SelectArgs a{};
  a.scores = scores;
  a.idx = idx;
  a.cnt = cnt;
  a.nk = int(nk);
  if (is_decode(desc)) {
    a.nq = 1;
    a.rows = desc->batch;
  } else {
    if ((st = check_prefill_shape(desc))) return st;
    a.nq = int(nk);
    a.rows = desc->batch * desc->hkv * int(nk);
  }
  a.n_sink = desc->n_sink;
  a.n_recent = desc->n_recent;
  a.k_min = desc->k_min;
  a.top_p = desc->top_p;
  return launched(spot::launch_select_topp(a, static_cast<hipStream_t>(stream)), "select_topp");
}

int spot_sparse_attn_prefill(const spot_desc* desc, const void* q, const void* k, const void* v, const int32_t* perm,
                             const int32_t* idx, const int32_t* cnt, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!q || !k || !v || !idx || !cnt || !o) return fail(SPOT_ERR_INVALID, "q, k, v, idx, cnt and o are required");
  if (perm && desc->segment <= 0) return fail(SPOT_ERR_INVALID, "perm given but segment is 0");
  const int nb = int(ceil_div64(desc->q_len, desc->block));
  if (desc->dtype == SPOT_BF16) {
    if ((st = check_mfma_operands(q, k, v, o))) return st;
    const int G = desc->hq / desc->hkv;
    const long long units = (long long)desc->batch * desc->hkv * nb * ((G * desc->block + 255) / 256);
    if (units > 0x7fffffffLL) return fail(SPOT_ERR_UNSUPPORTED, "too many work units");
  }
  spot::PrefillArgs a{q, k, v, perm, idx, cnt, o, lse, desc->dtype == SPOT_BF16, desc->batch, desc->hq, desc->hkv,
                      desc->d, int(desc->q_len), desc->block, desc->segment, nb, effective_scale(desc)};
  return launched(spot::launch_prefill(a, static_cast<hipStream_t>(stream)), "sparse_attn_prefill");
}

static int check_grouped_indexer(const spot_desc* desc) {
  int st = check_common(desc);
  if (st) return st;
  if (desc->score_kind != SPOT_SCORE_RELU_INDEXER) return fail(SPOT_ERR_INVALID, "score_kind must be RELU_INDEXER");
  if ((st = check_indexer(desc))) return st;
  if (desc->d_idx % 32)
    return fail(SPOT_ERR_UNSUPPORTED, "32-element key groups need d_idx a multiple of 32 (got %d)", desc->d_idx);
  return SPOT_OK;
}

int spot_quantize_indexer_keys(const spot_desc* desc, const void* idx_k, uint8_t* k_codes, uint8_t* k_scales,
                               void* stream) {
  int st = check_grouped_indexer(desc);
  if (st) return st;
  if (!idx_k || !k_codes || !k_scales) return fail(SPOT_ERR_INVALID, "idx_k, k_codes and k_scales are required");
  if ((st = check_aligned16("idx_k", idx_k)) || (st = check_aligned16("k_codes", k_codes))) return st;
  const long long nk = ceil_div64(desc->kv_len, desc->block);
  const long long groups = (long long)desc->batch * nk * (desc->h_idx * desc->d_idx / 32);
  return launched(spot::launch_quantize_mxfp4(static_cast<const uint16_t*>(idx_k), k_codes, k_scales, groups,
                                              static_cast<hipStream_t>(stream)),
                  "quantize_indexer_keys");
}

int spot_indexer_score_mxfp4(const spot_desc* desc, const void* idx_q, const float* idx_w, const uint8_t* k_codes,
                             const uint8_t* k_scales, float* scores, void* stream) {
  int st = check_grouped_indexer(desc);
  if (st) return st;
  if (!idx_q || !idx_w || !k_codes || !k_scales || !scores)
    return fail(SPOT_ERR_INVALID, "idx_q, idx_w, k_codes, k_scales and scores are required");
  if ((st = check_aligned16("idx_q", idx_q)) || (st = check_aligned16("k_codes", k_codes))) return st;
  spot::IndexerFp4Args a{static_cast<const uint16_t*>(idx_q), idx_w, k_codes, k_scales, scores, desc->batch,
                         int(ceil_div64(desc->kv_len, desc->block)), desc->h_idx, desc->d_idx};
  return launched(spot::launch_indexer_score_mxfp4(a, static_cast<hipStream_t>(stream)), "indexer_score_mxfp4");
}

int spot_quantize_indexer_keys_int4(const spot_desc* desc, const void* idx_k, uint8_t* k_codes, void* k_scales,
                                    void* stream) {
  int st = check_grouped_indexer(desc);
  if (st) return st;
  if (!idx_k || !k_codes || !k_scales) return fail(SPOT_ERR_INVALID, "idx_k, k_codes and k_scales are required");
  if ((st = check_aligned16("idx_k", idx_k)) || (st = check_aligned16("k_codes", k_codes))) return st;
  if (reinterpret_cast<uintptr_t>(k_scales) & 1u) return fail(SPOT_ERR_INVALID, "k_scales must be 2-byte aligned");
  const long long nk = ceil_div64(desc->kv_len, desc->block);
  const long long groups = (long long)desc->batch * nk * (desc->h_idx * desc->d_idx / 32);
  return launched(spot::launch_quantize_int4(static_cast<const uint16_t*>(idx_k), k_codes,
                                             static_cast<uint16_t*>(k_scales), groups,
                                             static_cast<hipStream_t>(stream)),
                  "quantize_indexer_keys_int4");
}

int spot_indexer_score_int4(const spot_desc* desc, const void* idx_q, const float* idx_w, const uint8_t* k_codes,
                            const void* k_scales, float* scores, void* stream) {
  int st = check_grouped_indexer(desc);
  if (st) return st;
  if (!idx_q || !idx_w || !k_codes || !k_scales || !scores)
    return fail(SPOT_ERR_INVALID, "idx_q, idx_w, k_codes, k_scales and scores are required");
  if ((st = check_aligned16("idx_q", idx_q)) || (st = check_aligned16("k_codes", k_codes))) return st;
  if (reinterpret_cast<uintptr_t>(k_scales) & 1u) return fail(SPOT_ERR_INVALID, "k_scales must be 2-byte aligned");
  spot::IndexerInt4Args a{static_cast<const uint16_t*>(idx_q), idx_w, k_codes, static_cast<const uint16_t*>(k_scales),
                          scores, desc->batch, int(ceil_div64(desc->kv_len, desc->block)), desc->h_idx, desc->d_idx};
  return launched(spot::launch_indexer_score_int4(a, static_cast<hipStream_t>(stream)), "indexer_score_int4");
}

int spot_history_map(const spot_desc* desc, const void* q, const void* k, int32_t* hmap, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!q || !k || !hmap) return fail(SPOT_ERR_INVALID, "q, k and hmap are required");
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("k", k))) return st;
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "history maps support bf16 only");
  if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
  const int L = int(desc->q_len);
  const int nseg = int(ceil_div64(L, desc->segment));
  if (nseg > spot::kHistMaxSegments)
    return fail(SPOT_ERR_UNSUPPORTED, "%d segments (max %d)", nseg, spot::kHistMaxSegments);
  if (int64_t(nseg - 1) * desc->segment > spot::kHistMaxPrefix)
    return fail(SPOT_ERR_UNSUPPORTED, "history of %lld positions (max %d)", (long long)(nseg - 1) * desc->segment,
                spot::kHistMaxPrefix);
  const size_t need = spot::hist_workspace_bytes(desc->batch, desc->hkv, nseg, desc->segment, desc->d);
  if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
  spot::HistMapArgs a{};
  spot::hist_workspace_split(workspace, desc->batch, desc->hkv, nseg, desc->segment, desc->d, a.qrep, a.qpart,
                             a.keys);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.hmap = hmap;
  a.batch = desc->batch;
  a.hq = desc->hq;
  a.hkv = desc->hkv;
  a.d = desc->d;
  a.L = L;
  a.segment = desc->segment;
  a.nseg = nseg;
  a.kcap = spot::hist_key_cap(nseg, desc->segment);
  a.sm_scale = effective_scale(desc);
  return launched(spot::launch_history_map(a, static_cast<hipStream_t>(stream)), "history_map");
}

int spot_sparse_attn_prefill_history_map(const spot_desc* desc, float tau, const void* q, const void* k,
                                         const void* v, const int32_t* hmap, void* o, float* lse, int32_t* nused,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!q || !k || !v || !hmap || !o) return fail(SPOT_ERR_INVALID, "q, k, v, hmap and o are required");
  if ((st = check_mfma_operands(q, k, v, o))) return st;
  if (!std::isfinite(tau) || tau < 0.f) return fail(SPOT_ERR_INVALID, "tau must be finite and >= 0");
  if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "early stopping supports bf16 only");
  if (desc->block != 64 && desc->block != 128)
    return fail(SPOT_ERR_UNSUPPORTED, "early stopping needs block 64 or 128 (got %d)", desc->block);
  const int nb = int(ceil_div64(desc->q_len, desc->block));
  if (nb > spot::kEsMaxBlocks)
    return fail(SPOT_ERR_UNSUPPORTED, "%d blocks per sequence (max %d for early stopping)", nb, spot::kEsMaxBlocks);
  spot::PrefillArgs a{q, k, v, hmap, nullptr, nullptr, o, lse, 1, desc->batch, desc->hq, desc->hkv,
                      desc->d, int(desc->q_len), desc->block, desc->segment, nb, effective_scale(desc)};
  a.es = 1;
  a.tau = tau;
  a.nused = nused;
  a.es_hmap = 1;
  a.nseg = int(ceil_div64(desc->q_len, desc->segment));
  return launched(spot::launch_prefill(a, static_cast<hipStream_t>(stream)), "sparse_attn_prefill_history_map");
}

int spot_order_history(const spot_desc* desc, const float* scores, int32_t* order, int32_t* cnt, void* workspace,
                       size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!scores || !order || !cnt) return fail(SPOT_ERR_INVALID, "scores, order and cnt are required");
  if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
  const int64_t nb = ceil_div64(desc->q_len, desc->block);
  if (nb > spot::kOrderMaxBlocks)
    return fail(SPOT_ERR_UNSUPPORTED, "%lld blocks per sequence (max %d)", (long long)nb, spot::kOrderMaxBlocks);
  spot::OrderArgs a{scores, order, cnt, desc->batch * desc->hkv * int(nb), int(nb), desc->block, desc->segment};
  return launched(spot::launch_order_history(a, static_cast<hipStream_t>(stream)), "order_history");
}

int spot_sparse_attn_prefill_early_stop(const spot_desc* desc, float tau, const void* q, const void* k, const void* v,
                                        const int32_t* perm, const int32_t* order, const int32_t* cnt, void* o,
                                        float* lse, int32_t* nused, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!q || !k || !v || !order || !cnt || !o) return fail(SPOT_ERR_INVALID, "q, k, v, order, cnt and o are required");
  if ((st = check_mfma_operands(q, k, v, o))) return st;
  if (!std::isfinite(tau) || tau < 0.f) return fail(SPOT_ERR_INVALID, "tau must be finite and >= 0");
  if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "early stopping supports bf16 only");
  if (desc->block != 64 && desc->block != 128)
    return fail(SPOT_ERR_UNSUPPORTED, "early stopping needs block 64 or 128 (got %d)", desc->block);
  const int nb = int(ceil_div64(desc->q_len, desc->block));
  if (nb > spot::kEsMaxBlocks)
    return fail(SPOT_ERR_UNSUPPORTED, "%d blocks per sequence (max %d for early stopping)", nb, spot::kEsMaxBlocks);
  spot::PrefillArgs a{q, k, v, perm, order, cnt, o, lse, 1, desc->batch, desc->hq, desc->hkv,
                      desc->d, int(desc->q_len), desc->block, desc->segment, nb, effective_scale(desc)};
  a.es = 1;
  a.tau = tau;
  a.nused = nused;
  return launched(spot::launch_prefill(a, static_cast<hipStream_t>(stream)), "sparse_attn_prefill_early_stop");
}

int spot_sparse_attn_decode(const spot_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* idx, const int32_t* cnt, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if (desc->q_len != 1) return fail(SPOT_ERR_INVALID, "decode needs q_len == 1");
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "decode supports bf16 only");
  const int G = desc->hq / desc->hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(SPOT_ERR_UNSUPPORTED, "hq/hkv = %d (supported: 1, 2, 4, 8)", G);
  if (!q || !k_cache || !v_cache || !idx || !cnt || !o) return fail(SPOT_ERR_INVALID, "q, k_cache, v_cache, idx, cnt and o are required");
  const int nk = int(ceil_div64(desc->kv_len, desc->block));
  const int ns = spot::decode_num_splits(desc->batch, desc->hkv, nk);
  const size_t need = spot::decode_partials_bytes(desc->batch, desc->hq, desc->d, ns);
  if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("k_cache", k_cache)) ||
      (st = check_aligned16("v_cache", v_cache)) || (st = check_aligned16("workspace", workspace)))
    return st;
  spot::DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), idx, cnt, static_cast<uint16_t*>(o), lse,
                     static_cast<float*>(workspace), desc->batch, desc->hq, desc->hkv, desc->d, int(desc->kv_len),
                     desc->block, nk, ns, effective_scale(desc)};
  return launched(spot::launch_decode(a, static_cast<hipStream_t>(stream)), "sparse_attn_decode");
}

int spot_sparse_attn_decode_rla(const spot_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* idx, const int32_t* cnt, const float* rla_state, void* o, float* lse,
                                float* o_rla, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if (desc->q_len != 1) return fail(SPOT_ERR_INVALID, "decode needs q_len == 1");
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "decode supports bf16 only");
  const int G = desc->hq / desc->hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(SPOT_ERR_UNSUPPORTED, "hq/hkv = %d (supported: 1, 2, 4, 8)", G);
  if (!q || !k_cache || !v_cache || !idx || !cnt || !rla_state || !o || !o_rla)
    return fail(SPOT_ERR_INVALID, "q, k_cache, v_cache, idx, cnt, rla_state, o and o_rla are required");
  const int nk = int(ceil_div64(desc->kv_len, desc->block));
  const int ns = spot::decode_num_splits(desc->batch, desc->hkv, nk);
  const size_t att = spot::decode_partials_bytes(desc->batch, desc->hq, desc->d, ns);
  const size_t need = att + size_t(desc->batch) * desc->hq * ns * desc->d * sizeof(float);
  if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("k_cache", k_cache)) ||
      (st = check_aligned16("v_cache", v_cache)) || (st = check_aligned16("workspace", workspace)))
    return st;
  if (reinterpret_cast<uintptr_t>(rla_state) & 3u) return fail(SPOT_ERR_INVALID, "rla_state must be 4-byte aligned");
  spot::DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), idx, cnt, static_cast<uint16_t*>(o), lse,
                     static_cast<float*>(workspace), desc->batch, desc->hq, desc->hkv, desc->d, int(desc->kv_len),
                     desc->block, nk, ns, effective_scale(desc), rla_state,
                     reinterpret_cast<float*>(static_cast<char*>(workspace) + att), o_rla};
  return launched(spot::launch_decode(a, static_cast<hipStream_t>(stream)), "sparse_attn_decode_rla");
}

int spot_sparse_attn_decode_noalloc(const spot_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* idx, const int32_t* cnt, void* o, float* lse, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if (desc->q_len != 1) return fail(SPOT_ERR_INVALID, "decode needs q_len == 1");
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "decode supports bf16 only");
  const int G = desc->hq / desc->hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(SPOT_ERR_UNSUPPORTED, "hq/hkv = %d (supported: 1, 2, 4, 8)", G);
  if (!q || !k_cache || !v_cache || !idx || !cnt || !o) return fail(SPOT_ERR_INVALID, "q, k_cache, v_cache, idx, cnt and o are required");
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("k_cache", k_cache)) ||
      (st = check_aligned16("v_cache", v_cache)))
    return st;
  const int nk = int(ceil_div64(desc->kv_len, desc->block));
  const int ns = spot::decode_num_splits(desc->batch, desc->hkv, nk);
  const size_t need = spot::decode_partials_bytes(desc->batch, desc->hq, desc->d, ns);
  if (need > spot::kDecodeScratchBytes)
    return fail(SPOT_ERR_UNSUPPORTED, "decode partials of %zu bytes exceed the built-in scratch of %zu bytes "
                "(batch * hq too large for the allocation-free call)", need, spot::kDecodeScratchBytes);
  float* scratch = nullptr;
  hipError_t e = spot::decode_scratch(&scratch);
  if (e != hipSuccess) return fail(SPOT_ERR_LAUNCH, "decode scratch address: %s", hipGetErrorString(e));
  spot::DecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), idx, cnt, static_cast<uint16_t*>(o), lse, scratch,
                     desc->batch, desc->hq, desc->hkv, desc->d, int(desc->kv_len), desc->block, nk, ns,
                     effective_scale(desc)};
  return launched(spot::launch_decode(a, static_cast<hipStream_t>(stream)), "sparse_attn_decode_noalloc");
}

int spot_key_permutation(const spot_desc* desc, const void* q, const void* k, int32_t* perm, float* importance,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!q || !k || !perm) return fail(SPOT_ERR_INVALID, "q, k and perm are required");
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("k", k))) return st;
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "key permutation supports bf16 only");
  if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
  if (desc->segment > spot::kPermMaxSegment)
    return fail(SPOT_ERR_UNSUPPORTED, "segment %d (max %d)", desc->segment, spot::kPermMaxSegment);
  const int L = int(desc->q_len);
  const int nb = int(ceil_div64(L, desc->block));
  const int nr = L - (nb - 1) * desc->block;
  const int G = desc->hq / desc->hkv;
  const size_t need = spot::perm_workspace_bytes(desc->batch, desc->hkv, L, G, nr);
  if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
  spot::PermArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.perm = perm;
  a.importance = importance;
  a.nchunks = spot::perm_num_chunks(L);
  a.ngroups = spot::perm_num_groups(G, nr);
  a.ws_lse = static_cast<float*>(workspace);
  a.ws_imp = a.ws_lse + size_t(desc->batch) * desc->hkv * a.nchunks * a.ngroups * spot::kPermRowsPerGroup * 2;
  a.batch = desc->batch;
  a.hq = desc->hq;
  a.hkv = desc->hkv;
  a.d = desc->d;
  a.L = L;
  a.block = desc->block;
  a.nb = nb;
  a.segment = desc->segment;
  a.sm_scale = effective_scale(desc);
  return launched(spot::launch_key_permutation(a, static_cast<hipStream_t>(stream)), "key_permutation");
}

int spot_validate_perm(const spot_desc* desc, const int32_t* perm, int32_t* bad, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!perm || !bad) return fail(SPOT_ERR_INVALID, "perm and bad are required");
  if (desc->segment <= 0) return fail(SPOT_ERR_INVALID, "segment must be > 0");
  if (desc->segment > spot::kPermMaxSegment)
    return fail(SPOT_ERR_UNSUPPORTED, "segment %d (max %d)", desc->segment, spot::kPermMaxSegment);
  spot::PermCheckArgs a{perm, bad, int(desc->q_len), desc->segment, desc->batch * desc->hkv};
  return launched(spot::launch_perm_check(a, static_cast<hipStream_t>(stream)), "validate_perm");
}

// ---------------------------------------------------------------- residual linear attention
int spot_rla_block_states(const spot_desc* desc, const void* k, const void* v, const int32_t* perm, float* states,
                          float* states_perm, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!k || !v || !states) return fail(SPOT_ERR_INVALID, "k, v and states are required");
  if (perm && (desc->segment <= 0 || !states_perm))
    return fail(SPOT_ERR_INVALID, "perm needs segment > 0 and states_perm");
  if (!perm && states_perm) return fail(SPOT_ERR_INVALID, "states_perm given without perm");
  if ((st = check_aligned16("k", k)) || (st = check_aligned16("v", v)) || (st = check_aligned16("states", states)) ||
      (st = check_aligned16("states_perm", states_perm)))
    return st;
  const int pairs = desc->batch * desc->hkv;
  if (pairs > 65535) return fail(SPOT_ERR_UNSUPPORTED, "batch * hkv = %d (max 65535)", pairs);
  const int nb = int(ceil_div64(desc->q_len, desc->block));
  spot::RlaStateArgs a{k, v, nullptr, states, desc->dtype == SPOT_BF16, pairs, desc->d, int(desc->q_len),
                       desc->block, nb};
  if ((st = launched(spot::launch_rla_states(a, static_cast<hipStream_t>(stream)), "rla_block_states"))) return st;
  if (!perm) return SPOT_OK;
  a.perm = perm;
  a.states = states_perm;
  return launched(spot::launch_rla_states(a, static_cast<hipStream_t>(stream)), "rla_block_states (permuted)");
}

int spot_rla_prefill(const spot_desc* desc, const void* q, const float* states, const float* states_perm,
                     const int32_t* idx, const int32_t* cnt, float* o_rla, void* stream) {
  int st = check_common(desc);
  if (st) return st;
  if ((st = check_prefill_shape(desc))) return st;
  if (!q || !states || !idx || !cnt || !o_rla) return fail(SPOT_ERR_INVALID, "q, states, idx, cnt and o_rla are required");
  if (states_perm && desc->segment <= 0) return fail(SPOT_ERR_INVALID, "states_perm given but segment is 0");
  if (desc->n_recent < 1)
    return fail(SPOT_ERR_UNSUPPORTED, "residual linear attention needs n_recent >= 1 (each query block keeps its own block)");
  const int nb = int(ceil_div64(desc->q_len, desc->block));
  if (nb > spot::kRlaMaxBlocks) return fail(SPOT_ERR_UNSUPPORTED, "%d blocks per sequence (max %d)", nb, spot::kRlaMaxBlocks);
  const long long units = (long long)desc->batch * desc->hkv * nb;
  if (units > 0x7fffffffLL) return fail(SPOT_ERR_UNSUPPORTED, "too many work units");
  if ((st = check_aligned16("q", q)) || (st = check_aligned16("states", states)) ||
      (st = check_aligned16("states_perm", states_perm)))
    return st;
  spot::RlaPrefillArgs a{q, states, states_perm, idx, cnt, o_rla, desc->dtype == SPOT_BF16, desc->batch, desc->hq,
                         desc->hkv, desc->d, int(desc->q_len), desc->block, desc->segment, nb};
  return launched(spot::launch_rla_prefill(a, static_cast<hipStream_t>(stream)), "rla_prefill");
}

static int check_rla_decode(const spot_desc* desc) {
  int st = check_common(desc);
  if (st) return st;
  if (desc->q_len != 1) return fail(SPOT_ERR_INVALID, "decode needs q_len == 1");
  if (desc->dtype != SPOT_BF16) return fail(SPOT_ERR_UNSUPPORTED, "decode supports bf16 only");
  const int G = desc->hq / desc->hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(SPOT_ERR_UNSUPPORTED, "hq/hkv = %d (supported: 1, 2, 4, 8)", G);
  if (desc->batch * desc->hkv > 65535) return fail(SPOT_ERR_UNSUPPORTED, "batch * hkv = %d (max 65535)", desc->batch * desc->hkv);
  return SPOT_OK;
}

int spot_rla_decode_state(const spot_desc* desc, const void* k_cache, const void* v_cache, float* state,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_rla_decode(desc);
  if (st) return st;
  if (!k_cache || !v_cache || !state) return fail(SPOT_ERR_INVALID, "k_cache, v_cache and state are required");
  const int pairs = desc->batch * desc->hkv;
  const int nr = int(ceil_div64(desc->kv_len, spot::kRlaDecodeSpan));
  const size_t need = size_t(pairs) * nr * desc->d * desc->d * sizeof(float);
  if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
  if ((st = check_aligned16("k_cache", k_cache)) || (st = check_aligned16("v_cache", v_cache)) ||
      (st = check_aligned16("state", state)) || (st = check_aligned16("workspace", workspace)))
    return st;
  spot::RlaStateArgs a{k_cache, v_cache, nullptr, static_cast<float*>(workspace), 1, pairs, desc->d,
                       int(desc->kv_len), spot::kRlaDecodeSpan, nr};
  if ((st = launched(spot::launch_rla_states(a, static_cast<hipStream_t>(stream)), "rla_decode_state (chunks)")))
    return st;
  return launched(spot::launch_rla_reduce(static_cast<const float*>(workspace), state, nr, desc->d, pairs,
                                          static_cast<hipStream_t>(stream)),
                  "rla_decode_state (sum)");
}

int spot_rla_decode(const spot_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                    const float* state, const int32_t* idx, const int32_t* cnt, float* o_rla, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_rla_decode(desc);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !state || !idx || !cnt || !o_rla)
    return fail(SPOT_ERR_INVALID, "q, k_cache, v_cache, state, idx, cnt and o_rla are required");
  const int ns = spot::rla_decode_num_splits(desc->batch, desc->hkv);
  const size_t need = size_t(desc->batch) * desc->hq * ns * desc->d * sizeof(float);
  if ((st = check_workspace(need, workspace, workspace_bytes))) return st;
  if ((st = check_aligned16("k_cache", k_cache)) || (st = check_aligned16("v_cache", v_cache)))
    return st;
  if (reinterpret_cast<uintptr_t>(q) & 1u) return fail(SPOT_ERR_INVALID, "q must be 2-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(SPOT_ERR_INVALID, "workspace must be 4-byte aligned");
  const int nk = int(ceil_div64(desc->kv_len, desc->block));
  spot::RlaDecodeArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                        static_cast<const uint16_t*>(v_cache), state, idx, cnt, o_rla,
                        static_cast<float*>(workspace), desc->batch, desc->hq, desc->hkv, desc->d,
                        int(desc->kv_len), desc->block, nk, ns};
  return launched(spot::launch_rla_decode(a, static_cast<hipStream_t>(stream)), "rla_decode");
}

}  // extern "C"
