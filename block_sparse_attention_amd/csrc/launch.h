// Host-side launchers of the gfx950 kernels (one definition per kernel file).
// Arguments are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spot {

struct PoolArgs {
  const void* q;
  const void* k;
  const int32_t* perm;   // nullable
  float* qbar;           // [batch, hkv, nb, d]
  float* kbar_nat;
  float* kbar_perm;      // written only when perm != nullptr
  int bf16, batch, hq, hkv, d, L, block, nb;
  float* kvar_nat;       // nullable: per-dimension block variances of K (natural)
  float* kvar_perm;      // and through perm (written only when perm != nullptr)
};
hipError_t launch_pool_blocks(const PoolArgs& a, hipStream_t s);

struct MeanpoolScoreArgs {
  const float* qbar;
  const float* kbar_nat;
  const float* kbar_perm;  // nullable
  float* scores;           // [batch, hkv, nb, nb]
  int batch, hkv, d, nb, block, segment;
  float scale;
  const float* var_nat;    // nullable: Taylor score with these block variances
  const float* var_perm;
};
hipError_t launch_meanpool_score(const MeanpoolScoreArgs& a, hipStream_t s);

struct IndexerScoreArgs {
  const uint16_t* idx_q;  // [batch, h_idx, d_idx] bf16
  const float* idx_w;     // [batch, h_idx]
  const uint16_t* idx_k;  // [batch, nk, h_idx, d_idx] bf16
  float* scores;          // [batch, nk]
  int batch, nk, h_idx, d_idx;
};
hipError_t launch_indexer_score(const IndexerScoreArgs& a, hipStream_t s);

struct IndexerFp4Args {
  const uint16_t* idx_q;  // [batch, h_idx, d_idx] bf16
  const float* idx_w;     // [batch, h_idx]
  const uint8_t* codes;   // [batch, nk, h_idx * d_idx / 2] packed E2M1 pairs
  const uint8_t* scales;  // [batch, nk, h_idx * d_idx / 32] E8M0
  float* scores;          // [batch, nk]
  int batch, nk, h_idx, d_idx;
};
hipError_t launch_indexer_score_mxfp4(const IndexerFp4Args& a, hipStream_t s);
hipError_t launch_quantize_mxfp4(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long ngroups,
                                 hipStream_t s);

struct IndexerInt4Args {
  const uint16_t* idx_q;   // [batch, h_idx, d_idx] bf16
  const float* idx_w;      // [batch, h_idx]
  const uint8_t* codes;    // [batch, nk, h_idx * d_idx / 2] packed 4-bit two's-complement pairs
  const uint16_t* scales;  // [batch, nk, h_idx * d_idx / 32] bf16
  float* scores;           // [batch, nk]
  int batch, nk, h_idx, d_idx;
};
hipError_t launch_indexer_score_int4(const IndexerInt4Args& a, hipStream_t s);
hipError_t launch_quantize_int4(const uint16_t* x, uint8_t* codes, uint16_t* scales, long long ngroups,
                                hipStream_t s);

struct SelectArgs {
  const float* scores;  // [rows, nk]
  int32_t* idx;         // [rows, nk]
  int32_t* cnt;         // [rows]
  int rows, nk, nq;     // nq == 1: decode rows (candidates 0..nk-1); else row % nq = query block i
  int n_sink, n_recent, k_min;
  float top_p;
};
hipError_t launch_select_topp(const SelectArgs& a, hipStream_t s);
constexpr int kSelectMaxCandidates = 16384;

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* perm;  // nullable
  const int32_t* idx;   // [batch, hkv, nb, nb]
  const int32_t* cnt;   // [batch, hkv, nb]
  void* o;
  float* lse;           // nullable
  int bf16, batch, hq, hkv, d, L, block, segment, nb;
  float sm_scale;
  // early stopping: idx holds the visiting order of the history blocks and
  // cnt their number; the own segment is implied
  int es;
  float tau;
  int32_t* nused;       // [batch, hq, L] history blocks taken per row, nullable
  // early stopping on per-segment history maps: perm points at maps
  // [batch, hkv, nseg, L] and the history is visited in map order
  int es_hmap;
  int nseg;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
constexpr int kEsMaxBlocks = 2048;     // blocks per sequence for early stopping (visiting list staged in LDS)

struct HistMapArgs {
  const uint16_t* q;   // [batch, hq, L, d] bf16
  const uint16_t* k;   // [batch, hkv, L, d] bf16
  int32_t* hmap;       // [batch, hkv, nseg, L]
  float* qrep;         // workspace: [batch, hkv, nseg, d] representative queries
  float* qpart;        // workspace: partial sums of the segment means
  uint64_t* keys;      // workspace: [batch, hkv, nseg, kcap] sort keys
  int batch, hq, hkv, d, L, segment, nseg, kcap;
  float sm_scale;
};
hipError_t launch_history_map(const HistMapArgs& a, hipStream_t s);
int hist_key_cap(int nseg, int segment);
size_t hist_workspace_bytes(int batch, int hkv, int nseg, int segment, int d);
void hist_workspace_split(void* ws, int batch, int hkv, int nseg, int segment, int d, float*& qrep, float*& qpart,
                          uint64_t*& keys);
constexpr int kHistMaxPrefix = 32768;   // history positions per segment map
constexpr int kHistMaxSegments = 64;    // representative queries held in LDS by the key pass

struct OrderArgs {
  const float* scores;  // [rows, nb]
  int32_t* order;       // [rows, nb]
  int32_t* cnt;         // [rows]
  int rows, nb, block, segment;
};
hipError_t launch_order_history(const OrderArgs& a, hipStream_t s);
constexpr int kOrderMaxBlocks = 4096;

struct DecodeArgs {
  const uint16_t* q;   // [batch, hq, d]
  const uint16_t* k;   // [batch, hkv, T, d]
  const uint16_t* v;
  const int32_t* idx;  // [batch, nk]
  const int32_t* cnt;  // [batch]
  uint16_t* o;         // [batch, hq, d]
  float* lse;          // nullable
  float* partials;     // workspace: [batch, hkv, nsplit, G, d + 2] fp32 (acc, max, sum)
  int batch, hq, hkv, d, T, block, nk, nsplit;
  float sm_scale;
  // residual linear attention beside the attention (all three set, or none)
  const float* rla_state;   // [batch, hkv, d, d] state of the whole cache
  float* rla_partials;      // workspace: [batch, hkv, nsplit, G, d] kept-key terms
  float* o_rla;             // [batch, hq, d]
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
int decode_num_splits(int batch, int hkv, int nk);
size_t decode_partials_bytes(int batch, int hq, int d, int nsplit);
// allocation-free decode: a file-scope device array of this size holds the partials; decode_scratch gives
// its address on the current device (looked up once per device)
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
hipError_t decode_scratch(float** ptr);

struct PermArgs {
  const uint16_t* q;   // [batch, hq, L, d] bf16
  const uint16_t* k;   // [batch, hkv, L, d] bf16
  int32_t* perm;       // [batch, hkv, L]
  float* importance;   // [batch, hkv, L] or nullptr
  float* ws_lse;       // workspace: per-chunk (max, sum) of every last-block query row
  float* ws_imp;       // workspace: per-row-group importance partials
  int batch, hq, hkv, d, L, block, nb, segment, nchunks, ngroups;
  float sm_scale;
};
hipError_t launch_key_permutation(const PermArgs& a, hipStream_t s);
int perm_num_chunks(int L);
int perm_num_groups(int G, int nr);
size_t perm_workspace_bytes(int batch, int hkv, int L, int G, int nr);
constexpr int kPermMaxSegment = 16384;

struct PermCheckArgs {
  const int32_t* perm;   // [pairs, L]
  int32_t* bad;          // one int32: violations found
  int L, segment, pairs;
};
hipError_t launch_perm_check(const PermCheckArgs& a, hipStream_t s);
constexpr int kPermRowsPerGroup = 256;   // query rows per workgroup in the permutation passes

// residual linear attention (feature map exp, no normaliser)
struct RlaStateArgs {
  const void* k;         // [pairs, L, d]
  const void* v;
  const int32_t* perm;   // [pairs, L] or nullptr: position t of a range reads row perm[t]
  float* states;         // [pairs, nranges, d, d]
  int bf16, pairs, d, L, span, nranges;
};
hipError_t launch_rla_states(const RlaStateArgs& a, hipStream_t s);
hipError_t launch_rla_reduce(const float* chunks, float* out, int nranges, int d, int pairs, hipStream_t s);
constexpr int kRlaMaxBlocks = 4096;     // blocks per sequence (kept and rest lists staged in LDS)
constexpr int kRlaDecodeSpan = 4096;    // keys per chunk state of the cache

struct RlaPrefillArgs {
  const void* q;              // [batch, hq, L, d]
  const float* states;        // [batch, hkv, nb, d, d] natural blocks
  const float* states_perm;   // same, blocks through the permutation; nullptr: natural everywhere
  const int32_t* idx;         // [batch, hkv, nb, nb] ascending kept lists
  const int32_t* cnt;         // [batch, hkv, nb]
  float* o;                   // [batch, hq, L, d]
  int bf16, batch, hq, hkv, d, L, block, segment, nb;
};
hipError_t launch_rla_prefill(const RlaPrefillArgs& a, hipStream_t s);

struct RlaDecodeArgs {
  const uint16_t* q;     // [batch, hq, d] bf16
  const uint16_t* k;     // [batch, hkv, T, d]
  const uint16_t* v;
  const float* state;    // [batch, hkv, d, d] state of the whole cache
  const int32_t* idx;    // [batch, nk]
  const int32_t* cnt;    // [batch]
  float* o;              // [batch, hq, d]
  float* partials;       // workspace: [batch, hkv, nsplit, G, d]
  int batch, hq, hkv, d, T, block, nk, nsplit;
};
hipError_t launch_rla_decode(const RlaDecodeArgs& a, hipStream_t s);
int rla_decode_num_splits(int batch, int hkv);

}  // namespace spot
