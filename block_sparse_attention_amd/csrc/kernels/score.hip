// Block scoring kernels for gfx950.
//
// pool_blocks      per-block means of Q (over the heads of a KV group and the
//                  rows of the block) and of K (natural, and through the key
//                  permutation): mean pooling for block selection as in PBS-Attn
//                  section 4 ("Implementatie", block selection on permuted keys).
//                  With variance outputs it also writes the per-dimension
//                  variance of each block's K rows (SPLA section 2.1 block
//                  statistics), from a second pass over the rows.
// meanpool_score   sm_scale * <qbar_i, kbar_j> for every key block j <= i
//                  (SpotAttention section 1: all previous blocks are scored in
//                  one contraction); j > i is -inf.  Taylor variant (SPLA
//                  section 2.1): x . kbar_j + log(1 + 1/2 sum_d x_d^2 var_jd)
//                  with x = sm_scale * qbar_i, the log of the second-order
//                  estimate of the block's attention mass.
// indexer_score    SpotAttention section 1 scoring equation:
//                  sum_h w_h ReLU(q^I_h . k^I_{h,t}), one streaming pass over the
//                  indexer key cache.
//
// quantize_mxfp4   SpotAttention section 4: the selector's key cache in FP4
//                  microscaling (OCP MX MXFP4: E2M1 elements, one E8M0
//                  power-of-two scale per 32 elements).
// indexer_score_mxfp4  the ReLU indexer score over that cache: the E2M1 pairs
//                  are widened to bf16 by the gfx950 conversion instruction and
//                  multiplied with the bf16 query by v_dot2; the group sum is
//                  scaled by its power of two.
//
// All of them are HBM- or latency-bound; they use plain fp32 VALU arithmetic.
#include "../launch.h"
#include "common.h"

namespace spot {

// ---------------------------------------------------------------- pooling
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
  x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Reduce per-thread column partials (rows_par row slots x d columns) through
// LDS and store sum * inv_count for the d columns.
// With `keep`, the result is also left in LDS for a following pass.
__device__ __forceinline__ void reduce_cols_store(float (&acc)[8], float* red, int lr, int rp, int rows_par,
                                                  int d, float inv_count, float* out, float* keep = nullptr) {
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rp * d + lr * 8 + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float s = 0.f;
    for (int r = 0; r < rows_par; ++r) s += red[r * d + c];
    out[c] = s * inv_count;
    if (keep) keep[c] = s * inv_count;
  }
  __syncthreads();
}

// Second pass over a block's K rows: sum of squared deviations from the mean
// kept in LDS, stored divided by the row count.
template <typename T, bool PERM>
__device__ __forceinline__ void block_variance(const PoolArgs& a, const T* K, size_t kv_row0, int r0, int nr,
                                               int lr, int rp, int rows_par, float* red, const float* mean,
                                               float* out) {
  float acc[8];
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = mean[lr * 8 + e];
#pragma unroll 4
  for (int rr = rp; rr < nr; rr += rows_par) {
    const int row = PERM ? a.perm[kv_row0 + r0 + rr] : r0 + rr;
    float x[8];
    load8<T>(K + (kv_row0 + row) * a.d + lr * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dx = x[e] - mu[e];
      acc[e] = fmaf(dx, dx, acc[e]);
    }
  }
  reduce_cols_store(acc, red, lr, rp, rows_par, a.d, 1.0f / float(nr), out);
}

template <typename T>
__global__ __launch_bounds__(256) void pool_blocks_kernel(PoolArgs a) {
  __shared__ float red[256 * 8];
  __shared__ float mean_s[128];
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int d = a.d, L = a.L, B = a.block;
  const int G = a.hq / a.hkv;
  const int lpr = d / 8;              // lanes per row
  const int rows_par = 256 / lpr;     // rows in flight per pass
  const int lr = threadIdx.x % lpr, rp = threadIdx.x / lpr;
  const int r0 = i * B;
  const int nr = min(B, L - r0);
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const size_t out_off = ((size_t(b) * a.hkv + g) * a.nb + i) * d;

  float acc[8];
  // Q: G heads x nr rows
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int rr = rp; rr < G * nr; rr += rows_par) {
    const int h = g * G + rr / nr, r = r0 + rr % nr;
    float x[8];
    load8<T>(Q + ((size_t(b) * a.hq + h) * L + r) * d + lr * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
  reduce_cols_store(acc, red, lr, rp, rows_par, d, 1.0f / float(G * nr), a.qbar + out_off);

  const size_t kv_row0 = (size_t(b) * a.hkv + g) * L;
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int rr = rp; rr < nr; rr += rows_par) {
    float x[8];
    load8<T>(K + (kv_row0 + r0 + rr) * d + lr * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
  reduce_cols_store(acc, red, lr, rp, rows_par, d, 1.0f / float(nr), a.kbar_nat + out_off, mean_s);
  if (a.kvar_nat)
    block_variance<T, false>(a, K, kv_row0, r0, nr, lr, rp, rows_par, red, mean_s, a.kvar_nat + out_off);

  if (a.perm) {
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int rr = rp; rr < nr; rr += rows_par) {
      const int phys = a.perm[kv_row0 + r0 + rr];
      float x[8];
      load8<T>(K + (kv_row0 + phys) * d + lr * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
    reduce_cols_store(acc, red, lr, rp, rows_par, d, 1.0f / float(nr), a.kbar_perm + out_off, mean_s);
    if (a.kvar_nat)
      block_variance<T, true>(a, K, kv_row0, r0, nr, lr, rp, rows_par, red, mean_s, a.kvar_perm + out_off);
  }
}

hipError_t launch_pool_blocks(const PoolArgs& a, hipStream_t s) {
  dim3 grid(a.nb, a.hkv, a.batch);
  if (a.bf16)
    pool_blocks_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    pool_blocks_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- mean-pool score
// Score tile (query blocks x key blocks).  16 x 16 tiles give 512 workgroups
// at 128 blocks and 8 KV heads, against 128 for 32 x 32 tiles (7.2 -> 5.2 us;
// the Taylor score 11.8 -> 7.3 us on MI355X).
#ifndef SPOT_SCORE_TILE
#define SPOT_SCORE_TILE 16
#endif
constexpr int kST = SPOT_SCORE_TILE;
constexpr int kSR = kST / 16;         // each of the 16 x 16 threads scores a kSR x kSR block
static_assert(kSR >= 1 && kST % 16 == 0, "16 x 16 threads per tile");

// Tiles of pooled rows sit in LDS with rows padded by 4 floats: 16-byte
// accesses stay aligned and the 16 key rows a wave reads start on distinct
// 4-bank groups.  Each thread accumulates a kSR x kSR block of scores over d
// in ascending order, four dims per LDS read.
constexpr int kSPad = 4;

template <bool TAYLOR>
__global__ __launch_bounds__(256) void meanpool_score_kernel(MeanpoolScoreArgs a) {
  extern __shared__ float4 sm4[];
  float* sm = reinterpret_cast<float*>(sm4);
  const int d = a.d, nb = a.nb;
  const int ld = d + kSPad;
  float* qs = sm;
  float* kn = qs + kST * ld;
  float* kp = kn + kST * ld;
  float* vns = kp + kST * ld;   // TAYLOR: block variances (natural, permuted)
  float* vps = vns + kST * ld;
  const int i0 = blockIdx.y * kST, j0 = blockIdx.x * kST;
  const size_t bg = blockIdx.z;
  float* out = a.scores + bg * size_t(nb) * nb;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;

  if (j0 > i0 + kST - 1) {  // entirely above the diagonal
    for (int e = threadIdx.x; e < kST * kST; e += 256) {
      const int i = i0 + e / kST, j = j0 + e % kST;
      if (i < nb && j < nb) out[size_t(i) * nb + j] = -kInf;
    }
    return;
  }
  const float* qb = a.qbar + bg * size_t(nb) * d;
  const float* knb = a.kbar_nat + bg * size_t(nb) * d;
  const float* kpb = a.kbar_perm ? a.kbar_perm + bg * size_t(nb) * d : nullptr;
  const float* vnb = TAYLOR ? a.var_nat + bg * size_t(nb) * d : nullptr;
  const float* vpb = TAYLOR && kpb ? a.var_perm + bg * size_t(nb) * d : nullptr;
  auto stage = [&](float* dst, const float* src, int row0, int r, int c) {
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dst + r * ld + c) =
        (row0 + r < nb) ? *reinterpret_cast<const float4*>(src + size_t(row0 + r) * d + c) : zero;
  };
  for (int e = threadIdx.x; e < kST * d / 4; e += 256) {
    const int r = e / (d / 4), c = (e % (d / 4)) * 4;
    stage(qs, qb, i0, r, c);
    stage(kn, knb, j0, r, c);
    if (kpb) stage(kp, kpb, j0, r, c);
    if constexpr (TAYLOR) {
      stage(vns, vnb, j0, r, c);
      if (vpb) stage(vps, vpb, j0, r, c);
    }
  }
  __syncthreads();
  float sn[kSR][kSR], sp[kSR][kSR], tn[kSR][kSR], tp[kSR][kSR];   // tn, tp (TAYLOR): sum qbar_c^2 var_c
#pragma unroll
  for (int u = 0; u < kSR; ++u)
#pragma unroll
    for (int w = 0; w < kSR; ++w) sn[u][w] = sp[u][w] = tn[u][w] = tp[u][w] = 0.f;
  auto ld4 = [&](const float* base, int row, int c) { return *reinterpret_cast<const float4*>(base + row * ld + c); };
  auto acc4 = [](float& s, const float4& x, const float4& y) {
    s = fmaf(x.x, y.x, s);
    s = fmaf(x.y, y.y, s);
    s = fmaf(x.z, y.z, s);
    s = fmaf(x.w, y.w, s);
  };
  auto sq4 = [](const float4& x) { return make_float4(x.x * x.x, x.y * x.y, x.z * x.z, x.w * x.w); };
#pragma unroll 4
  for (int c = 0; c < d; c += 4) {
    float4 q[kSR], kk[kSR];
#pragma unroll
    for (int u = 0; u < kSR; ++u) {
      q[u] = ld4(qs, ty * kSR + u, c);
      kk[u] = ld4(kn, tx * kSR + u, c);
    }
#pragma unroll
    for (int u = 0; u < kSR; ++u)
#pragma unroll
      for (int w = 0; w < kSR; ++w) acc4(sn[u][w], q[u], kk[w]);
    if (kpb) {
#pragma unroll
      for (int w = 0; w < kSR; ++w) kk[w] = ld4(kp, tx * kSR + w, c);
#pragma unroll
      for (int u = 0; u < kSR; ++u)
#pragma unroll
        for (int w = 0; w < kSR; ++w) acc4(sp[u][w], q[u], kk[w]);
    }
    if constexpr (TAYLOR) {
#pragma unroll
      for (int u = 0; u < kSR; ++u) q[u] = sq4(q[u]);
#pragma unroll
      for (int w = 0; w < kSR; ++w) kk[w] = ld4(vns, tx * kSR + w, c);
#pragma unroll
      for (int u = 0; u < kSR; ++u)
#pragma unroll
        for (int w = 0; w < kSR; ++w) acc4(tn[u][w], q[u], kk[w]);
      if (vpb) {
#pragma unroll
        for (int w = 0; w < kSR; ++w) kk[w] = ld4(vps, tx * kSR + w, c);
#pragma unroll
        for (int u = 0; u < kSR; ++u)
#pragma unroll
          for (int w = 0; w < kSR; ++w) acc4(tp[u][w], q[u], kk[w]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kSR; ++u)
#pragma unroll
    for (int w = 0; w < kSR; ++w) {
      const int i = i0 + ty * kSR + u, j = j0 + tx * kSR + w;
      if (i >= nb || j >= nb) continue;
      float v = -kInf;
      if (j <= i) {
        const bool hist = kpb && a.segment > 0 && (j * a.block) / a.segment < (i * a.block) / a.segment;
        v = a.scale * (hist ? sp[u][w] : sn[u][w]);
        if constexpr (TAYLOR) v += log1pf(0.5f * a.scale * a.scale * (hist ? tp[u][w] : tn[u][w]));
      }
      out[size_t(i) * nb + j] = v;
    }
}

hipError_t launch_meanpool_score(const MeanpoolScoreArgs& a, hipStream_t s) {
  const int nt = (a.nb + kST - 1) / kST;
  dim3 grid(nt, nt, a.batch * a.hkv);
  if (a.var_nat) {
    const size_t lds = size_t(5) * kST * (a.d + kSPad) * sizeof(float);
    meanpool_score_kernel<true><<<grid, 256, lds, s>>>(a);
  } else {
    const size_t lds = size_t(3) * kST * (a.d + kSPad) * sizeof(float);
    meanpool_score_kernel<false><<<grid, 256, lds, s>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- ReLU indexer score
// A row (one key block: h_idx x d_idx bf16) is spread over LPR lanes, 8
// elements (16 bytes) per lane; lanes of one indexer head sum their dot
// products, the head leaders add w_h * ReLU(dot), and the row's lanes sum the
// heads.  Each lane keeps kIdxUnroll rows in flight; one grid row per sequence.
#ifndef SPOT_INDEXER_UNROLL
#define SPOT_INDEXER_UNROLL 4         // rows in flight per lane (tuning knob)
#endif
#ifndef SPOT_INDEXER_MAX_BLOCKS
#define SPOT_INDEXER_MAX_BLOCKS 256   // workgroups per sequence: enough that each takes one round of rows (tuning knob)
#endif
constexpr int kIdxUnroll = SPOT_INDEXER_UNROLL;
constexpr int kIdxMaxBlocks = SPOT_INDEXER_MAX_BLOCKS;
constexpr int kFp4Unroll = 4;       // the same for the MXFP4 scan
constexpr int kFp4MaxBlocks = 64;

template <int LPR>
__global__ __launch_bounds__(256) void indexer_score_kernel(IndexerScoreArgs a) {
  constexpr int RPW = 64 / LPR;   // rows per wave per load
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int R = a.h_idx * a.d_idx;
  const int lph = a.d_idx / 8;    // lanes per indexer head
  const int e0 = li * 8;
  const bool act = e0 < R;
  const int head = act ? e0 / a.d_idx : 0;
  uint4 qv = make_uint4(0u, 0u, 0u, 0u);
  float w = 0.f;
  if (act) {
    qv = *reinterpret_cast<const uint4*>(a.idx_q + size_t(b) * R + e0);
    w = a.idx_w[size_t(b) * a.h_idx + head];
  }
  const uint16_t* kb = a.idx_k + size_t(b) * a.nk * R;
  const int step = gridDim.x * 4 * RPW * kIdxUnroll;
  for (int t0 = (blockIdx.x * 4 + wave) * RPW * kIdxUnroll; t0 < a.nk; t0 += step) {
    uint4 kv[kIdxUnroll];
#pragma unroll
    for (int u = 0; u < kIdxUnroll; ++u) {
      const int t = t0 + u * RPW + sub;
      kv[u] = (act && t < a.nk) ? *reinterpret_cast<const uint4*>(kb + size_t(t) * R + e0)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kIdxUnroll; ++u) {
      float dp = dot2_bf16(kv[u].x, qv.x, dot2_bf16(kv[u].y, qv.y, dot2_bf16(kv[u].z, qv.z,
                           dot2_bf16(kv[u].w, qv.w, 0.f))));
      for (int o = 1; o < lph; o <<= 1) dp += __shfl_xor(dp, o);
      float val = (act && (li % lph) == 0) ? w * fmaxf(dp, 0.f) : 0.f;
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1)
        if (o >= lph) val += __shfl_xor(val, o);
      const int t = t0 + u * RPW + sub;
      if (li == 0 && t < a.nk) a.scores[size_t(b) * a.nk + t] = val;
    }
  }
}

template <int LPR>
static void launch_idx(const IndexerScoreArgs& a, hipStream_t s) {
  const int per_block = 4 * (64 / LPR) * kIdxUnroll;
  int blocks = (a.nk + per_block - 1) / per_block;
  if (blocks > kIdxMaxBlocks) blocks = kIdxMaxBlocks;
  indexer_score_kernel<LPR><<<dim3(blocks, a.batch), 256, 0, s>>>(a);
}

hipError_t launch_indexer_score(const IndexerScoreArgs& a, hipStream_t s) {
  const int lanes = (a.h_idx * a.d_idx) / 8;   // 16-byte chunks per row (R <= 256)
  if (lanes <= 2) launch_idx<2>(a, s);
  else if (lanes <= 4) launch_idx<4>(a, s);
  else if (lanes <= 8) launch_idx<8>(a, s);
  else if (lanes <= 16) launch_idx<16>(a, s);
  else launch_idx<32>(a, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- MXFP4 indexer keys
// Magnitude code of |y| on the E2M1 grid (0, 0.5, 1, 1.5, 2, 3, 4, 6), rounded
// to nearest with ties to the even code and saturating at 6: every midpoint
// below an even code counts with >=, every midpoint below an odd code with >.
__device__ __forceinline__ uint32_t e2m1_code(uint16_t bits, float inv_scale) {
  const float a = fabsf(bf16_to_f32(bits) * inv_scale);
  const uint32_t m = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
  return ((uint32_t(bits) >> 12) & 8u) | m;
}

// One thread per group of 32 consecutive elements: shared exponent from the
// largest magnitude (compared as bit patterns), then 16 packed code bytes
// (element 2k in the low nibble) and one scale byte.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, long long ngroups) {
  const long long gi = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gi >= ngroups) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + gi * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  int e = -127;
  if (amax) {
    const int ef = int(amax >> 7);
    const int fl = ef > 0 ? ef - 127 : (31 - __builtin_clz(amax & 0x7fu)) - 133;   // floor(log2 max)
    e = min(max(fl - 2, -127), 127);
  }
  scales[gi] = uint8_t(e + 127);
  const float inv = __uint_as_float(uint32_t(127 - e) << 23);   // 2^-e, a normal float for finite inputs
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t word = w[4 * i + j];
      const uint32_t byte = e2m1_code(uint16_t(word & 0xffffu), inv) | (e2m1_code(uint16_t(word >> 16), inv) << 4);
      r |= byte << (8 * j);
    }
    out[i] = r;
  }
  *reinterpret_cast<uint4*>(codes + gi * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_quantize_mxfp4(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long ngroups,
                                 hipStream_t s) {
  const long long blocks = (ngroups + 255) / 256;
  quantize_mxfp4_kernel<<<dim3(unsigned(blocks)), 256, 0, s>>>(x, codes, scales, ngroups);
  return hipGetLastError();
}

// A row (one key block: h_idx x d_idx codes) is spread over LPR lanes, one
// 32-element group (16 code bytes + its scale byte) per lane.
template <int LPR>
__global__ __launch_bounds__(256) void indexer_score_mxfp4_kernel(IndexerFp4Args a) {
  constexpr int RPW = 64 / LPR;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int R = a.h_idx * a.d_idx;
  const int lph = a.d_idx / 32;   // lanes per indexer head
  const int e0 = li * 32;
  const bool act = e0 < R;        // LPR rounds R / 32 up to a power of two: the extra lanes hold no group
  const int head = act ? e0 / a.d_idx : 0;
  uint32_t qw[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.idx_q + size_t(b) * R + (act ? e0 : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = qp[i];
      qw[4 * i] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
    }
  }
  const float w = act ? a.idx_w[size_t(b) * a.h_idx + head] : 0.f;
  // codes and scales of sequence b as buffer resources: a lane without a row reads out of range (zero), so
  // every load of the round is issued unconditionally and all are in flight together
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.codes + size_t(b) * a.nk * (R / 2)), 0, a.nk * (R / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.scales + size_t(b) * a.nk * (R / 32)), 0, a.nk * (R / 32), 0x00020000);
  const int step = gridDim.x * 4 * RPW * kFp4Unroll;
  for (int t0 = (blockIdx.x * 4 + wave) * RPW * kFp4Unroll; t0 < a.nk; t0 += step) {
    uint4 cv[kFp4Unroll];
    int ex[kFp4Unroll];
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const int t = t0 + u * RPW + sub;
      const bool in = act && t < a.nk;
      cv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rc, in ? uint32_t(t * (R / 2) + li * 16) : 0x80000000u, 0, 0));
      ex[u] = __builtin_amdgcn_raw_buffer_load_b8(rsc, in ? uint32_t(t * (R / 32) + li) : 0x80000000u, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const uint32_t cw[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
      float dp = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // byte j of word i holds elements 8i+2j (low nibble) and 8i+2j+1
        dp = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[i], 1.0f, 0)),
                       qw[4 * i + 0], dp);
        dp = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[i], 1.0f, 1)),
                       qw[4 * i + 1], dp);
        dp = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[i], 1.0f, 2)),
                       qw[4 * i + 2], dp);
        dp = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[i], 1.0f, 3)),
                       qw[4 * i + 3], dp);
      }
      dp = ldexpf(dp, ex[u] - 127);
      for (int o = 1; o < lph; o <<= 1) dp += __shfl_xor(dp, o);
      float val = (act && (li % lph) == 0) ? w * fmaxf(dp, 0.f) : 0.f;
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1)
        if (o >= lph) val += __shfl_xor(val, o);
      const int t = t0 + u * RPW + sub;
      if (li == 0 && t < a.nk) a.scores[size_t(b) * a.nk + t] = val;
    }
  }
}

template <int LPR>
static void launch_idx_fp4(const IndexerFp4Args& a, hipStream_t s) {
  const int per_block = 4 * (64 / LPR) * kFp4Unroll;
  int blocks = (a.nk + per_block - 1) / per_block;
  if (blocks > kFp4MaxBlocks) blocks = kFp4MaxBlocks;
  indexer_score_mxfp4_kernel<LPR><<<dim3(blocks, a.batch), 256, 0, s>>>(a);
}

hipError_t launch_indexer_score_mxfp4(const IndexerFp4Args& a, hipStream_t s) {
  const int lanes = (a.h_idx * a.d_idx) / 32;   // one 32-element group per lane (R <= 256)
  if (lanes <= 1) launch_idx_fp4<1>(a, s);
  else if (lanes <= 2) launch_idx_fp4<2>(a, s);
  else if (lanes <= 4) launch_idx_fp4<4>(a, s);
  else launch_idx_fp4<8>(a, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- INT4 indexer keys
// SpotAttention section 4 (selector K-cache as INT4 microscale): every 32
// consecutive elements share one bf16 scale s = max|x| / 7 (rounded to
// nearest even); each element is x / s rounded to the nearest integer (ties
// to even) and clamped to [-7, 7], stored as a 4-bit two's-complement code,
// two per byte with the even element in the low nibble.  An all-zero group
// gets scale 0 and codes 0.  The division is IEEE fp32: for bf16 x and s the
// exact quotient is either a half-integer or at least 2^-9 relative away
// from one, so the rounded quotient takes the same integer as the exact one.
__global__ __launch_bounds__(256) void quantize_int4_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ scales, long long ngroups) {
  const long long gi = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gi >= ngroups) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + gi * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  uint32_t amax = 0;   // largest magnitude, compared as bf16 bit patterns (exact for finite values)
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  const uint32_t sbits = pack_bf16x2(bf16_to_f32(uint16_t(amax)) / 7.0f, 0.f) & 0xFFFFu;
  const float sc = bf16_to_f32(uint16_t(sbits));
  scales[gi] = uint16_t(sbits);
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t word = w[4 * i + j / 2];
      const float v = (j & 1) ? bf16_hi(word) : bf16_lo(word);
      const int c = sc > 0.f ? int(fminf(fmaxf(rintf(v / sc), -7.f), 7.f)) : 0;
      r |= (uint32_t(c) & 15u) << (4 * j);
    }
    out[i] = r;
  }
  *reinterpret_cast<uint4*>(codes + gi * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_quantize_int4(const uint16_t* x, uint8_t* codes, uint16_t* scales, long long ngroups,
                                hipStream_t s) {
  const long long blocks = (ngroups + 255) / 256;
  quantize_int4_kernel<<<dim3(unsigned(blocks)), 256, 0, s>>>(x, codes, scales, ngroups);
  return hipGetLastError();
}

// A row (one key block: h_idx x d_idx codes) is spread over LPR lanes, one
// 32-element group (16 code bytes + its bf16 scale) per lane; codes widen to
// fp32 and multiply the bf16 query (exact products), the group sum is scaled
// once.
template <int LPR>
__global__ __launch_bounds__(256) void indexer_score_int4_kernel(IndexerInt4Args a) {
  constexpr int RPW = 64 / LPR;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int R = a.h_idx * a.d_idx;
  const int lph = a.d_idx / 32;   // lanes per indexer head
  const int e0 = li * 32;
  const bool act = e0 < R;        // LPR rounds R / 32 up to a power of two: the extra lanes hold no group
  const int head = act ? e0 / a.d_idx : 0;
  float qf[32];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.idx_q + size_t(b) * R + (act ? e0 : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = qp[i];
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qf[8 * i + 2 * k] = bf16_lo(vw[k]);
        qf[8 * i + 2 * k + 1] = bf16_hi(vw[k]);
      }
    }
  }
  const float w = act ? a.idx_w[size_t(b) * a.h_idx + head] : 0.f;
  // as in the MXFP4 scan: out-of-range buffer reads (zero) for lanes without a row, every load in flight
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.codes + size_t(b) * a.nk * (R / 2)), 0, a.nk * (R / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.scales + size_t(b) * a.nk * (R / 32)), 0, a.nk * (R / 32) * 2, 0x00020000);
  const int step = gridDim.x * 4 * RPW * kFp4Unroll;
  for (int t0 = (blockIdx.x * 4 + wave) * RPW * kFp4Unroll; t0 < a.nk; t0 += step) {
    uint4 cv[kFp4Unroll];
    uint32_t scb[kFp4Unroll];   // scale bits, widened where they are used
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const int t = t0 + u * RPW + sub;
      const bool in = act && t < a.nk;
      cv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rc, in ? uint32_t(t * (R / 2) + li * 16) : 0x80000000u, 0, 0));
      scb[u] = __builtin_amdgcn_raw_buffer_load_b16(rsc, in ? uint32_t((t * (R / 32) + li) * 2) : 0x80000000u, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const uint32_t cw[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
      // v_cvt_off_f32_i4 turns the low nibble of a byte (selected in the
      // instruction) into c / 16: the even elements from the word, the odd
      // ones from the word shifted by a nibble.  The sum is 1/16 of the sum of
      // c * q taken in the same order, exactly (a power-of-two scaling), and
      // the factor 16 goes back with the scale.
      float dp = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = cw[i];
        uint32_t hi = cw[i] >> 4;
        asm volatile("" : "+v"(hi));   // one shift per word, then byte selects (not a field extract per element)
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // byte j of word i: elements 8i + 2j (low nibble) and 8i + 2j + 1
          dp = fmaf(__builtin_amdgcn_cvt_off_f32_i4((lo >> (8 * j)) & 0xffu), qf[8 * i + 2 * j], dp);
          dp = fmaf(__builtin_amdgcn_cvt_off_f32_i4((hi >> (8 * j)) & 0xffu), qf[8 * i + 2 * j + 1], dp);
        }
      }
      dp = (dp * 16.0f) * bf16_to_f32(uint16_t(scb[u]));
      for (int o = 1; o < lph; o <<= 1) dp += __shfl_xor(dp, o);
      float val = (act && (li % lph) == 0) ? w * fmaxf(dp, 0.f) : 0.f;
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1)
        if (o >= lph) val += __shfl_xor(val, o);
      const int t = t0 + u * RPW + sub;
      if (li == 0 && t < a.nk) a.scores[size_t(b) * a.nk + t] = val;
    }
  }
}

template <int LPR>
static void launch_idx_int4(const IndexerInt4Args& a, hipStream_t s) {
  const int per_block = 4 * (64 / LPR) * kFp4Unroll;
  int blocks = (a.nk + per_block - 1) / per_block;
  if (blocks > kFp4MaxBlocks) blocks = kFp4MaxBlocks;
  indexer_score_int4_kernel<LPR><<<dim3(blocks, a.batch), 256, 0, s>>>(a);
}

hipError_t launch_indexer_score_int4(const IndexerInt4Args& a, hipStream_t s) {
  const int lanes = (a.h_idx * a.d_idx) / 32;   // one 32-element group per lane (R <= 256)
  if (lanes <= 1) launch_idx_int4<1>(a, s);
  else if (lanes <= 2) launch_idx_int4<2>(a, s);
  else if (lanes <= 4) launch_idx_int4<4>(a, s);
  else launch_idx_int4<8>(a, s);
  return hipGetLastError();
}

}  // namespace spot
