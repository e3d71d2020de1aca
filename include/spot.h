/*
 * spot.h - C ABI of the block-sparse causal attention library (libspot.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The library implements one hot path in four calls, plus the key permutation
 * that feeds its permuted variant:
 *
 *   spot_block_score         score every (query block, key block) pair
 *   spot_select_topp         keep blocks by cumulative-mass top-p
 *   spot_sparse_attn_prefill online-softmax attention over the kept blocks (GQA prefill)
 *   spot_sparse_attn_decode  the same for one decode query per sequence
 *   spot_key_permutation     the intra-segment key permutation the prefill gathers through
 *   spot_validate_perm       debug check that a permutation maps every segment onto itself
 *
 * the selector key cache in FP4 microscaling for the decode scan:
 *
 *   spot_quantize_indexer_keys  encode the indexer keys as MXFP4
 *   spot_indexer_score_mxfp4    the RELU_INDEXER scores from that encoding
 *
 * and an early-stopped variant of selection + prefill attention:
 *
 *   spot_order_history                  visiting order of each query block's history blocks
 *   spot_sparse_attn_prefill_early_stop attention that stops taking history blocks per row
 *   spot_history_map                    per-segment maps of the history by a representative query
 *   spot_sparse_attn_prefill_history_map the early-stopped attention walking those maps
 *
 * Conventions shared by every call
 * --------------------------------
 * Ownership.  Every tensor pointer is caller-owned DEVICE memory.  The library
 *   never allocates, frees or synchronises; each call only enqueues kernels on
 *   `stream` (a hipStream_t; NULL means the null stream) and returns.  Scratch
 *   memory is a caller-provided workspace whose size spot_workspace_size reports.
 * Layouts (all contiguous, row-major):
 *   Q, O            [batch, hq,  q_len,  d]
 *   K, V            [batch, hkv, kv_len, d]
 *   perm            int32 [batch, hkv, q_len]   logical -> physical key row
 *   scores          float [batch, hsel, nq, nk]
 *   idx             int32 [batch, hsel, nq, nk] kept block ids, ascending, -1 padded
 *   cnt             int32 [batch, hsel, nq]     number of kept blocks
 *   idx_q (q^I)     bf16  [batch, h_idx, d_idx]
 *   idx_w (w)       float [batch, h_idx]
 *   idx_k (K^I)     bf16  [batch, nk, h_idx, d_idx]
 *   lse             float [batch, hq, q_len]    natural-log sum of exp of the logits
 *   with nk = ceil(kv_len / block); for prefill nq = nk, hsel = hkv; for decode
 *   nq = 1, hsel = 1 (one list per sequence, shared by all heads).
 * dtype.  SPOT_F32 or SPOT_BF16 for Q, K, V and O (O takes Q's dtype).
 *   Scores, lse and all accumulation are fp32.
 * Errors.  Every call returns SPOT_OK (0) or a negative status; arguments are
 *   validated on the host before anything is launched, so a failed call
 *   enqueues nothing.  spot_last_error() gives a thread-local message.
 *   A launch failure reported by the HIP runtime returns SPOT_ERR_LAUNCH.
 * State.  None across calls; the library is thread-safe.
 *
 * Sources (titles of the summarised papers):
 *   [Spot] SpotAttention: Plug-In Block-Sparse Routing for Pretrained
 *          Long-Context Transformers
 *   [PBS]  PBS-Attn, "Sparsere Blok-Sparse Attention via Tokenpermutatie"
 *   [S2O]  "S2O - Vroege Stoppering voor Sparse Attention via Online Permutatie"
 *   [SPLA] "SPLA - Block Sparse Plus Linear Attention voor Long Context Modeling"
 */
#ifndef SPOT_H
#define SPOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPOT_ABI_VERSION 1

enum spot_status {
  SPOT_OK = 0,
  SPOT_ERR_INVALID = -1,      /* null required pointer, inconsistent sizes, bad parameter */
  SPOT_ERR_UNSUPPORTED = -2,  /* valid but outside the built kernels (dtype, d, block, length) */
  SPOT_ERR_WORKSPACE = -3,    /* workspace smaller than spot_workspace_size reports */
  SPOT_ERR_LAUNCH = -4        /* the HIP runtime rejected a kernel launch */
};

enum spot_dtype { SPOT_F32 = 0, SPOT_BF16 = 1 };

enum spot_score_kind {
  SPOT_SCORE_MEANPOOL = 0,     /* prefill: sm_scale * <mean q, mean k>           ([PBS] §4) */
  SPOT_SCORE_RELU_INDEXER = 1, /* decode: sum_h w_h ReLU(q^I_h . k^I_{h,t})       ([Spot] §1) */
  SPOT_SCORE_TAYLOR = 2        /* prefill: log of the second-order block mass      ([SPLA] §2.1) */
};

enum spot_op {
  SPOT_OP_BLOCK_SCORE = 0,
  SPOT_OP_SELECT_TOPP = 1,
  SPOT_OP_PREFILL = 2,
  SPOT_OP_DECODE = 3,
  SPOT_OP_KEY_PERMUTATION = 4,
  SPOT_OP_ORDER_HISTORY = 5,
  SPOT_OP_PREFILL_EARLY_STOP = 6,
  SPOT_OP_HISTORY_MAP = 7,
  SPOT_OP_RLA_DECODE_STATE = 8,
  SPOT_OP_RLA_DECODE = 9,
  SPOT_OP_DECODE_RLA = 10
};

/* Problem descriptor.  `version` must be SPOT_ABI_VERSION. */
typedef struct spot_desc {
  int32_t version;
  int32_t dtype;                  /* enum spot_dtype */
  int32_t batch, hq, hkv, d;      /* hq % hkv == 0; d in {64, 128} */
  int64_t q_len, kv_len;          /* prefill: q_len == kv_len == L; decode: q_len == 1, kv_len == T */
  int32_t block;                  /* B in {16, 32, 64, 128}: query and key block size */
  int32_t segment;                /* S, a multiple of B, when a permutation is used; else 0 */
  int32_t n_sink, n_recent;       /* forced blocks: the first n_sink and the last n_recent (>= 1 together) */
  int32_t k_min;                  /* floor on the number of residual blocks kept */
  float top_p;                    /* >= 1 keeps every candidate; <= 0 keeps the forced blocks only */
  float sm_scale;                 /* softmax scale; 0 selects 1/sqrt(d) */
  int32_t score_kind;             /* enum spot_score_kind */
  int32_t h_idx, d_idx;           /* indexer heads and width (RELU_INDEXER) */
} spot_desc;

/* Library version (SPOT_ABI_VERSION). */
int spot_version(void);

/* Text for a status code (static storage). */
const char* spot_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* spot_last_error(void);

/* Workspace bytes that `op` needs for `desc` (0 is possible).  Host only. */
int spot_workspace_size(const spot_desc* desc, int op, size_t* bytes);

/*
 * Block scores.
 *
 * MEANPOOL (prefill, [PBS] §4; scale as attention): for KV head g, query
 * block i and key block j <= i
 *     scores[b,g,i,j] = sm_scale * < qbar[g,i], kbar[g,j] >
 *   qbar[g,i] = mean of Q over the G = hq/hkv heads of group g and the rows of
 *   block i; kbar[g,j] = mean of the K rows of block j, taken through `perm`
 *   (rows perm[b,g,t], t in block j) when perm != NULL and block j lies in an
 *   earlier segment than block i, else in natural order.  j > i gets -inf.
 *   Uses q, k, perm (nullable); idx_q, idx_w, idx_k must be NULL or are ignored.
 *   Workspace: the pooled means (spot_workspace_size).
 *
 * TAYLOR (prefill, [SPLA] §2.1 second-order Taylor block selection with a
 * diagonal covariance): with x = sm_scale * qbar[g,i],
 *     scores[b,g,i,j] = < x, kbar[g,j] > + ln(1 + 1/2 * sum_c x_c^2 var[g,j,c])
 *   the logarithm of the estimated attention mass of block j, so the softmax
 *   over blocks is the normalised estimate.  var[g,j,c] is the population
 *   variance of coordinate c over the block's K rows (the same rows as kbar:
 *   through perm for history blocks).  Same inputs as MEANPOOL; workspace:
 *   five pooled slabs instead of three (spot_workspace_size).
 *
 * RELU_INDEXER (decode, [Spot] §1 scoring equation): for sequence b and key
 * block t < nk
 *     scores[b,0,0,t] = sum_h idx_w[b,h] * max(0, < idx_q[b,h], idx_k[b,t,h] >)
 *   Uses idx_q, idx_w, idx_k; q, k, perm are ignored.
 *
 * Alignment: q and k (pooled scores) or idx_q and idx_k (indexer) must be
 * 16-byte aligned (the kernels read rows in 16-byte pieces; SPOT_ERR_INVALID
 * otherwise).
 */
int spot_block_score(const spot_desc* desc, const void* q, const void* k, const int32_t* perm,
                     const void* idx_q, const float* idx_w, const void* idx_k, float* scores,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dual top-p selection ([Spot] §3), one row per (b, g, i) (prefill) or per b
 * (decode).  Candidates are key blocks 0..i (prefill) or 0..nk-1 (decode).
 * Forced: j < n_sink and j > last - n_recent (last = i, or nk-1).  The
 * residual candidates are ordered by (score desc, block id asc); their
 * softmax masses are accumulated (fp64) until the sum reaches top_p
 * (inclusive); at least min(k_min, #residual) are kept; top_p >= 1 keeps all.
 * Output: kept ids ascending in idx, padded with -1 to nk, count in cnt.
 * Rows longer than 16384 candidates are unsupported.
 */
int spot_select_topp(const spot_desc* desc, const float* scores, int32_t* idx, int32_t* cnt,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse prefill attention ([PBS] Problem and §2, [S2O] §1 and §3).
 * For query head h (group g = h / G) and row r of query block i:
 *     O[b,h,r] = sum_t softmax_t(sm_scale * q.k_t) v_t
 * over the keys of the kept blocks idx[b,g,i,0..cnt): a block of an earlier
 * segment contributes rows perm[b,g,t] (t in the block), all visible; a block
 * of the query's own segment (or every block when perm == NULL) contributes
 * its natural rows t <= r.  lse (nullable) receives ln(sum exp(logits)).
 * Kept lists must be ascending, with block ids < nk; every row must see at
 * least one key (guaranteed when the diagonal or block 0 is kept).  bf16:
 * q, k and v 16-byte aligned, o 8-byte aligned (the kernel's vector loads
 * and stores; SPOT_ERR_INVALID otherwise).
 */
int spot_sparse_attn_prefill(const spot_desc* desc, const void* q, const void* k, const void* v,
                             const int32_t* perm, const int32_t* idx, const int32_t* cnt, void* o,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse decode attention ([Spot] Problem and §3 at decode time): one query
 * per (sequence b, head h) at position kv_len - 1 attends every key of the
 * kept blocks idx[b,0,0,0..cnt) (shared by all heads; all visible).
 * q: [batch, hq, d]; k_cache, v_cache: [batch, hkv, kv_len, d];
 * o: [batch, hq, d]; lse (nullable): [batch, hq].
 * Work is split over the kept list; partial (max, sum, accumulator) triples go
 * to the workspace and are merged in a fixed order (deterministic).  A
 * sequence with cnt = 0 attends no key: its O is 0 and its lse -inf.
 * q, k_cache, v_cache and workspace must be 16-byte aligned (SPOT_ERR_INVALID
 * otherwise).
 */
int spot_sparse_attn_decode(const spot_desc* desc, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* idx, const int32_t* cnt, void* o,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of spot_sparse_attn_decode, for callers that cannot
 * allocate device memory (code under stream/graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, layouts, result
 * and errors as spot_sparse_attn_decode, without the workspace: the partials
 * live in a device array built into the library (8 MiB on each GPU the
 * library runs on, held until the process ends).  Inputs whose partials do
 * not fit (batch * hq * nsplit * (d + 2) * 4 bytes above 8 MiB; nsplit is at
 * most 32) return SPOT_ERR_UNSUPPORTED before anything is enqueued.  The call
 * allocates nothing.  Every call on one GPU shares that GPU's array: calls
 * that may overlap on one GPU (several streams, several threads) race and
 * must be serialised by the caller.  The first call on each device looks up
 * the array's address on that device (the device current at the call).
 */
int spot_sparse_attn_decode_noalloc(const spot_desc* desc, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* idx, const int32_t* cnt, void* o,
                                    float* lse, void* stream);

/*
 * Key permutation by global importance ([PBS] §3; index arrays as in [S2O] §1).
 * For KV head g, importance[t] = the causal softmax probability
 * softmax_{t' <= r}(sm_scale * q_{h,r} . k_{t'})[t], averaged over the query
 * rows r of the last query block and the G query heads h of the group (keys
 * after r receive 0).  Inside each segment [sS, (s+1)S) the positions are
 * sorted by importance descending, ties by position ascending:
 * perm[b,g,sS + j] = the j-th of them (logical position -> physical row).
 * q: [batch, hq, L, d] bf16; k: [batch, hkv, L, d] bf16; perm: int32
 * [batch, hkv, L] (output); importance: float [batch, hkv, L] (nullable
 * output).  Requires dtype bf16, segment > 0, a multiple of block and at most
 * 16384, and q, k 16-byte aligned.  Workspace:
 * spot_workspace_size(SPOT_OP_KEY_PERMUTATION).
 */
int spot_key_permutation(const spot_desc* desc, const void* q, const void* k, int32_t* perm, float* importance,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Debug check of a permutation handed to the prefill calls, which trust it:
 * inside each segment [sS, min((s+1)S, L)) of every (batch, KV head), perm
 * must be a bijection of the segment's positions ([PBS] §2: the permutation
 * stays inside segments so that causality between segments holds).
 * perm: int32 [batch, hkv, q_len]; bad: one int32 of device memory that the
 * call sets to the number of violations (a value outside its position's
 * segment, or a value seen before in the segment); 0 means valid.  The result
 * is ready when the stream reaches it (the call does not synchronise).
 * Requires segment > 0 and at most 16384.
 */
int spot_validate_perm(const spot_desc* desc, const int32_t* perm, int32_t* bad, void* stream);

/*
 * Selector key cache in FP4 microscaling ([Spot] §4 quantisation: the
 * selector's K-cache held as INT4/FP4 microscale).  The format is OCP
 * Microscaling (MX) v1.0 MXFP4: every 32 consecutive elements of an indexer
 * key row (h_idx * d_idx elements, so d_idx must be a multiple of 32) share
 * one E8M0 scale byte e (scale 2^(e-127)); each element is a 4-bit E2M1 code
 * (bit 3 sign, bits 0-2 index into 0, 0.5, 1, 1.5, 2, 3, 4, 6), two codes per
 * byte with the even element in the low nibble.
 * Layouts: k_codes uint8 [batch, nk, h_idx*d_idx/2]; k_scales uint8
 * [batch, nk, h_idx*d_idx/32]; nk = ceil(kv_len / block).
 *
 * spot_quantize_indexer_keys: idx_k bf16 [batch, nk, h_idx, d_idx] (finite)
 *   -> codes and scales.  Per group: e = floor(log2(max |x|)) - 2 clamped to
 *   [-127, 127] (-127 for an all-zero group); each x / 2^e is rounded to the
 *   nearest E2M1 value, ties to the even code, saturating at 6; the sign bit
 *   is the input's.  Deterministic and exact (scales are powers of two).
 * spot_indexer_score_mxfp4: as spot_block_score with RELU_INDEXER, with the
 *   keys read from the encoding (decoded value = E2M1 value * 2^(e-127)):
 *     scores[b,0,0,t] = sum_h idx_w[b,h] * max(0, < idx_q[b,h], key[b,t,h] >)
 * Both need score_kind RELU_INDEXER and the indexer limits of
 * spot_block_score, and idx_k, idx_q and k_codes 16-byte aligned; no
 * workspace.
 */
int spot_quantize_indexer_keys(const spot_desc* desc, const void* idx_k, uint8_t* k_codes, uint8_t* k_scales,
                               void* stream);
int spot_indexer_score_mxfp4(const spot_desc* desc, const void* idx_q, const float* idx_w, const uint8_t* k_codes,
                             const uint8_t* k_scales, float* scores, void* stream);

/*
 * Selector key cache in INT4 microscaling ([Spot] §4 quantisation: the
 * selector's K-cache held as INT4/FP4 microscale).  Every 32 consecutive
 * elements of an indexer key row (d_idx a multiple of 32) share one bf16
 * scale s = max|x| / 7 (rounded to nearest, ties to even); each element is
 * x / s rounded to the nearest integer (ties to the even one), clamped to
 * [-7, 7], and stored as a 4-bit two's-complement code, two per byte with the
 * even element in the low nibble; an all-zero group has s = 0 and codes 0.
 * 4.5 bits per element: 3.56x smaller than bf16.
 * Layouts: k_codes uint8 [batch, nk, h_idx*d_idx/2]; k_scales bf16
 * [batch, nk, h_idx*d_idx/32]; nk = ceil(kv_len / block).
 *
 * spot_quantize_indexer_keys_int4: idx_k bf16 [batch, nk, h_idx, d_idx]
 *   (finite) -> codes and scales (deterministic, equal to the exact rule).
 * spot_indexer_score_int4: as spot_block_score with RELU_INDEXER, with the
 *   keys read from the encoding (decoded value = code * s).
 * Both need score_kind RELU_INDEXER and the indexer limits of
 * spot_block_score, idx_k, idx_q and k_codes 16-byte aligned and k_scales
 * 2-byte aligned; no workspace.
 */
int spot_quantize_indexer_keys_int4(const spot_desc* desc, const void* idx_k, uint8_t* k_codes, void* k_scales,
                                    void* stream);
int spot_indexer_score_int4(const spot_desc* desc, const void* idx_q, const float* idx_w, const uint8_t* k_codes,
                            const void* k_scales, float* scores, void* stream);

/*
 * Visiting order for early stopping ([S2O] §2: candidate blocks are processed
 * in descending estimated importance).  For each row (b, g, i) of the MEANPOOL
 * scores [batch, hkv, nb, nb]: the history blocks of query block i, i.e. the
 * blocks j of segments before i's segment (j < floor(i*B/S)*S/B), ordered by
 * scores[b,g,i,j] descending, ties by j ascending.
 * Output: order [batch, hkv, nb, nb] int32 (the ordered ids, -1 padded to nb)
 * and cnt [batch, hkv, nb] int32 (the number of history blocks).
 * Requires segment > 0 (a multiple of block) and nb <= 4096.  No workspace.
 */
int spot_order_history(const spot_desc* desc, const float* scores, int32_t* order, int32_t* cnt,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Early-stopped sparse prefill attention ([S2O] §2 early-stopping rule, §3
 * two passes).  For query head h (group g) and row r of query block i, with
 * s0 = floor(i*B/S)*S the start of i's segment:
 *   pass 1: keys s0..r in natural order (dense causal own segment);
 *   pass 2: the history blocks order[b,g,i,0..cnt) one at a time, their rows
 *           taken through perm (natural rows when perm == NULL), all visible.
 *   After each pass-2 block, gain = the softmax mass (sum of exp(logit - m))
 *   its keys add and acc = the mass accumulated so far including them; the
 *   row takes no further block once gain < tau * acc.
 *   O[b,h,r] = softmax attention over the keys taken; lse (nullable) as in
 *   spot_sparse_attn_prefill; nused (nullable) int32 [batch, hq, q_len]
 *   receives the number of history blocks the row took.
 * tau = 0 takes every history block (dense causal attention).  The
 * comparison runs on the kernel's fp32 sums, so a row whose ratio lies
 * within rounding of tau may stop one block earlier or later than an exact
 * evaluation.  Requires dtype bf16, d in {64, 128}, block in {64, 128},
 * segment > 0 (a multiple of block), nb <= 2048, tau finite and >= 0, and
 * the alignment of q, k, v and o that spot_sparse_attn_prefill needs in bf16.
 * No workspace.
 */
int spot_sparse_attn_prefill_early_stop(const spot_desc* desc, float tau, const void* q, const void* k,
                                        const void* v, const int32_t* perm, const int32_t* order,
                                        const int32_t* cnt, void* o, float* lse, int32_t* nused,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * History maps by a representative query ([S2O] §1 historical KV
 * permutation: the historical keys are scored against a representative
 * query of the segment, prefix tokens only, and the sorted indices form a
 * logical map).  For KV head g and segment s >= 1 (segments of S positions,
 * the last one possibly partial):
 *   qrep = mean of Q over the G query heads of the group and the rows of s;
 *   hmap[b,g,s,j], j < s*S = the positions t < s*S sorted by
 *     sm_scale * < qrep, k_t > descending, ties by t ascending;
 *   hmap[b,g,s,j] = -1 for j >= s*S, and all of segment 0.
 * q: [batch, hq, L, d] bf16; k: [batch, hkv, L, d] bf16; hmap: int32
 * [batch, hkv, nseg, L] (output), nseg = ceil(L / S).  Requires segment > 0,
 * nseg <= 64, (nseg - 1) * S <= 32768 and q, k 16-byte aligned.  Workspace:
 * spot_workspace_size(SPOT_OP_HISTORY_MAP).  Scores are fp32, so keys whose
 * scores agree to fp32 rounding may be ordered differently from an exact
 * evaluation.
 */
int spot_history_map(const spot_desc* desc, const void* q, const void* k, int32_t* hmap, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Early-stopped prefill on history maps ([S2O] §1-3): as
 * spot_sparse_attn_prefill_early_stop, with pass 2 visiting, for a query in
 * segment s, the history blocks hmap[b,g,s, jB .. (j+1)B) for j = 0, 1, ...
 * (all visible) instead of ordered key blocks; the same per-row stopping
 * rule with threshold tau; nused counts the runs taken.  Same requirements
 * as spot_sparse_attn_prefill_early_stop plus segment > 0 (a multiple of
 * block).  No workspace.
 */
int spot_sparse_attn_prefill_history_map(const spot_desc* desc, float tau, const void* q, const void* k,
                                         const void* v, const int32_t* hmap, void* o, float* lse, int32_t* nused,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Residual linear attention ([SPLA] §2.2: the blocks outside the selection
 * enter through linear attention, evaluated as the all-blocks estimate minus
 * the selected-blocks estimate; §2.3: parameter-free exponential feature
 * map).  For a query row q with kept key set K(q) and visible key set A(q):
 *   o_rla = sum over t in A(q) \ K(q) of (phi(q) . phi(k_t)) v_t,
 *   phi(x) = exp(x) elementwise on the raw q and k rows, no normaliser
 * (the page normalises the branch afterwards with a trained RMS norm and
 * gates it into the output; those trained parts are not in this library).
 * Prefill: A = {t <= r}, K = the keys of the row's kept blocks (earlier
 * segments through the permutation, as in spot_sparse_attn_prefill).
 * Decode: A = the whole cache, K = the keys of the kept blocks.
 * Linear attention is evaluated through d x d fp32 states
 * S = sum_t phi(k_t) v_t^T of key ranges; every sum runs in a fixed order in
 * fp32, so results are deterministic.  Outputs are fp32.
 *
 * spot_rla_block_states: prefill descriptor.  states [batch, hkv, nb, d, d]:
 *   the state of each key block j (rows jB .. min((j+1)B, L)); with perm (and
 *   segment > 0) also states_perm, the state of the rows perm[b,g,t] for t in
 *   block j.  k, v: [batch, hkv, L, d] (bf16 or fp32), 16-byte aligned;
 *   states 16-byte aligned.  perm entries outside [0, L) are clamped (wrong
 *   sums, never out-of-range reads).  No workspace.
 * spot_rla_prefill: prefill descriptor.  q [batch, hq, L, d], the states
 *   above (states_perm non-NULL: blocks of earlier segments use it; requires
 *   segment > 0), the kept lists idx/cnt of spot_select_topp ->
 *   o_rla fp32 [batch, hq, L, d].  Each query block's own block must be in
 *   its list, which n_recent >= 1 guarantees: n_recent = 0 returns
 *   SPOT_ERR_UNSUPPORTED.  nb <= 4096.  q and the states 16-byte aligned.
 *   No workspace.
 * spot_rla_decode_state: decode descriptor (bf16).  state [batch, hkv, d, d]
 *   = the state of the whole cache [0, kv_len), built from chunk states in
 *   the workspace (spot_workspace_size(SPOT_OP_RLA_DECODE_STATE)).  Run when
 *   the cache changes, not per step.  k_cache, v_cache, state and workspace
 *   16-byte aligned.
 * spot_rla_decode: decode descriptor (bf16, hq/hkv in 1, 2, 4, 8).  q
 *   [batch, hq, d], the caches, the state above and the kept lists of
 *   spot_select_topp -> o_rla fp32 [batch, hq, d] = phi(q)^T state minus the
 *   linear attention over the kept keys (only the kept blocks are read; list
 *   entries outside the cache add nothing).  The kept keys are split over
 *   several workgroups whose partial sums sit in the workspace
 *   (spot_workspace_size(SPOT_OP_RLA_DECODE)) and are subtracted in a fixed
 *   order.  k_cache, v_cache 16-byte aligned, workspace 4-byte aligned.
 */
/*
 * Decode attention with the residual linear attention in the same pass
 * ([SPLA] §2.2: the selected blocks' linear-attention term is computed in the
 * fused kernel from the kept tiles the attention already reads).  Exactly
 * spot_sparse_attn_decode (o and lse, the same arithmetic), plus o_rla fp32
 * [batch, hq, d] = exp(q)^T rla_state minus the kept keys' sum of
 * (exp(q) . exp(k)) v, with rla_state from spot_rla_decode_state.  Same
 * requirements as spot_sparse_attn_decode; rla_state 4-byte aligned;
 * workspace: spot_workspace_size(SPOT_OP_DECODE_RLA).
 */
int spot_sparse_attn_decode_rla(const spot_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* idx, const int32_t* cnt, const float* rla_state, void* o, float* lse,
                                float* o_rla, void* workspace, size_t workspace_bytes, void* stream);

int spot_rla_block_states(const spot_desc* desc, const void* k, const void* v, const int32_t* perm, float* states,
                          float* states_perm, void* stream);
int spot_rla_prefill(const spot_desc* desc, const void* q, const float* states, const float* states_perm,
                     const int32_t* idx, const int32_t* cnt, float* o_rla, void* stream);
int spot_rla_decode_state(const spot_desc* desc, const void* k_cache, const void* v_cache, float* state,
                          void* workspace, size_t workspace_bytes, void* stream);
int spot_rla_decode(const spot_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                    const float* state, const int32_t* idx, const int32_t* cnt, float* o_rla, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPOT_H */
