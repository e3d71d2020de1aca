// Dual top-p block selection for gfx950 (SpotAttention section 3, "Dual Top-p
// Selectieregel"): reserved sink and recency blocks, nucleus selection on the
// residual distribution until the cumulative mass reaches p, floor K_min.
//
// One workgroup per row; each thread owns a contiguous run of candidate ids.
// The residual candidates that can be kept are ordered exactly in LDS on
// 64-bit keys (inverted order-preserving score bits above the id rank, so
// ascending keys are score-descending with ties to the lower id): small sets
// by counting each key's rank against all the others, larger ones by a
// bitonic network;
// their masses are prefix-summed in fp64 in that order and the first prefix
// reaching p ends the kept set.  On rows longer than the sort buffer only the
// candidates above a mass bound enter the sort: if the mass first reaches p
// at the k-th sorted block, the blocks from k on carry more than (1-p)Z
// between at most n_res of them, so every kept block has mass above
// (1-p)Z/n_res.  If even that set is too large, the cutoff is searched
// instead: with key = order-preserving score bits, the kept set is
// {key > K} plus the first ties in id order, where K is the largest key whose
// upper set still holds mass >= p (binary search over the key space).  Every
// mass is a fixed-order fp64 reduction, so the result is deterministic.
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kSelMaxPerThread = 16;   // candidates per thread (16384 / 1024)
#ifndef SPOT_SELECT_PER_THREAD
#define SPOT_SELECT_PER_THREAD 16
#endif
constexpr int kSelTargetPerThread = SPOT_SELECT_PER_THREAD;   // launch as few threads as keep at most this many per thread
static_assert(kSelTargetPerThread <= kSelMaxPerThread, "per-thread runs are register arrays");
static_assert(kSelMaxPerThread % 4 == 0, "runs are loaded in 16-byte groups");
constexpr int kSortMax = 2048;         // candidates sorted exactly in LDS
constexpr int kRankReads = 512;        // rank by counting while each thread compares at most this many keys
constexpr int kRankMax = 512;          // ... which bounds the set to 512 candidates (nthr <= 1024)
constexpr int kRankRounds = 3;         // and gives each thread at most 3 of them (nthr >= 64)
static_assert(kRankMax < kSortMax, "the key after a counted set pads an odd count");
constexpr int kRefineMin = 128;        // long rows: above this many candidates, narrow them by a score histogram
constexpr int kHistBins = 64;          // histogram bins of width 1/kHistScale in score units below the row max
constexpr float kHistScale = 4.0f;

__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s) == 0x80000000u ? 0u : __float_as_uint(s);   // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---- wave64 reductions and scans on DPP row operations (rows of 16 lanes)
// plus v_readlane across the four rows; no LDS crossbar round trips.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowRor8 = 0x128, kDppRowRor4 = 0x124, kDppQuad2301 = 0x4E, kDppQuad1032 = 0xB1;

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {   // lanes without a source in their row read 0
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, dpp_i32<CTRL>(__builtin_bit_cast(int, x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = uint32_t(dpp_i32<CTRL>(int(uint32_t(u)))), hi = uint32_t(dpp_i32<CTRL>(int(uint32_t(u >> 32))));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), l));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ float readlane_f32(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// totals over the wave (same value in every lane); rows first, then the four row totals in order
__device__ __forceinline__ double wave_total_f64(double x) {
  x += dpp_f64<kDppRowRor8>(x);
  x += dpp_f64<kDppRowRor4>(x);
  x += dpp_f64<kDppQuad2301>(x);
  x += dpp_f64<kDppQuad1032>(x);
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}
__device__ __forceinline__ int wave_total_i32(int x) {
  x += dpp_i32<kDppRowRor8>(x);
  x += dpp_i32<kDppRowRor4>(x);
  x += dpp_i32<kDppQuad2301>(x);
  x += dpp_i32<kDppQuad1032>(x);
  return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
         (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
  x = fmaxf(x, dpp_f32<kDppQuad2301>(x));
  x = fmaxf(x, dpp_f32<kDppQuad1032>(x));
  return fmaxf(fmaxf(readlane_f32(x, 0), readlane_f32(x, 16)), fmaxf(readlane_f32(x, 32), readlane_f32(x, 48)));
}
// inclusive prefix over the lanes: Hillis-Steele inside each row, then the earlier rows' totals
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += dpp_i32<kDppRowShr1>(x);
  x += dpp_i32<kDppRowShr2>(x);
  x += dpp_i32<kDppRowShr4>(x);
  x += dpp_i32<kDppRowShr8>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
  x += dpp_f64<kDppRowShr1>(x);
  x += dpp_f64<kDppRowShr2>(x);
  x += dpp_f64<kDppRowShr4>(x);
  x += dpp_f64<kDppRowShr8>(x);
  const double r0 = readlane_f64(x, 15), r1 = readlane_f64(x, 31), r2 = readlane_f64(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  double before = 0.0;
  if (row >= 1) before = r0;
  if (row >= 2) before += r1;
  if (row >= 3) before += r2;
  return before + x;
}

// ---- workgroup reductions: one value per wave in LDS, one barrier.  Two
// scratch slots alternate between successive calls; a slot is rewritten two
// calls later, after every thread has passed the barrier of the call between.
constexpr int kSelMaxWaves = 16;
struct SelScratch {
  double d[2][kSelMaxWaves];
  int i[2][kSelMaxWaves];
  float f[2][kSelMaxWaves];
};
struct BlockOps {
  SelScratch& s;
  int ph;   // slot of the next call (the same in every thread: calls are workgroup-uniform)
};

__device__ double block_sum_f64(double x, BlockOps& b) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_total_f64(x);
  double* slot = b.s.d[b.ph];
  b.ph ^= 1;
  if (lane == 0) slot[w] = x;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < nw; ++k) t += slot[k];
  return t;
}

__device__ int block_sum_i32(int x, BlockOps& b) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_total_i32(x);
  int* slot = b.s.i[b.ph];
  b.ph ^= 1;
  if (lane == 0) slot[w] = x;
  __syncthreads();
  int t = 0;
  for (int k = 0; k < nw; ++k) t += slot[k];
  return t;
}

__device__ float block_max_f32(float x, BlockOps& b) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_max_f32(x);
  float* slot = b.s.f[b.ph];
  b.ph ^= 1;
  if (lane == 0) slot[w] = x;
  __syncthreads();
  float t = -kInf;
  for (int k = 0; k < nw; ++k) t = fmaxf(t, slot[k]);
  return t;
}

// exclusive prefix (in thread order) of one int per thread, plus the total
__device__ int block_excl_scan_i32(int x, BlockOps& b, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const int incl = wave_incl_scan_i32(x);
  int* slot = b.s.i[b.ph];
  b.ph ^= 1;
  if (lane == 63) slot[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int k = 0; k < nw; ++k) {
    if (k < w) before += slot[k];
    tot += slot[k];
  }
  total = tot;
  return before + incl - x;
}

__device__ double block_excl_scan_f64(double x, BlockOps& b, double& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const double incl = wave_incl_scan_f64(x);
  double* slot = b.s.d[b.ph];
  b.ph ^= 1;
  if (lane == 63) slot[w] = incl;
  __syncthreads();
  double before = 0.0, tot = 0.0;
  for (int k = 0; k < nw; ++k) {
    if (k < w) before += slot[k];
    tot += slot[k];
  }
  total = tot;
  return before + (incl - x);
}

// kept ids ascending (thread runs are contiguous and in order), -1 padding, count
__device__ void write_row(const SelectArgs& a, int row, uint32_t keepm, int c0, BlockOps& sc) {
  int total_kept;
  int pos = block_excl_scan_i32(__popc(keepm), sc, total_kept);
  int32_t* irow = a.idx + size_t(row) * a.nk;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e)
    if (keepm & (1u << e)) irow[pos++] = c0 + e;
  // -1 padding: up to three words to a 16-byte boundary, then 16-byte stores
  const int c1 = min(a.nk, total_kept + int((4u - uint32_t((reinterpret_cast<uintptr_t>(irow + total_kept) >> 2) & 3u)) & 3u));
  if (int(threadIdx.x) < c1 - total_kept) irow[total_kept + threadIdx.x] = -1;
  const int n4 = (a.nk - c1) >> 2;
  int4* irow4 = reinterpret_cast<int4*>(irow + c1);
  for (int k = threadIdx.x; k < n4; k += blockDim.x) irow4[k] = make_int4(-1, -1, -1, -1);
  for (int c = c1 + 4 * n4 + threadIdx.x; c < a.nk; c += blockDim.x) irow[c] = -1;
  if (threadIdx.x == 0) a.cnt[row] = total_kept;
}

// Rank of each of the n keys k[0..n) = the number of smaller keys (all keys
// differ in their id word).  Thread t ranks keys t, t + nthr, ... (at most R);
// every key pair is read from LDS once and compared with all of them.
// k[n] must hold ~0 when n is odd.
template <int R>
__device__ void rank_by_count(const uint64_t* k, int n, uint16_t* rank, uint64_t* ranked) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  uint64_t x[R];
  int r[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int i = tid + t * nthr;
    x[t] = i < n ? k[i] : 0ull;
    r[t] = 0;
  }
#pragma unroll 4
  for (int j = 0; j < n; j += 2) {
    const uint64_t y0 = k[j], y1 = k[j + 1];
#pragma unroll
    for (int t = 0; t < R; ++t) r[t] += int(y0 < x[t]) + int(y1 < x[t]);
  }
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int i = tid + t * nthr;
    if (i < n) {
      rank[i] = uint16_t(r[t]);
      ranked[r[t]] = x[t];
    }
  }
}

__global__ __launch_bounds__(1024) void select_topp_kernel(SelectArgs a) {
  __shared__ SelScratch s_red;
  BlockOps sc{s_red, 0};
  __shared__ __align__(16) uint64_t s_sort[kSortMax];   // counting reads pairs: s_sort[ncand] pads an odd count (ncand <= kRankMax < kSortMax)
  __shared__ uint16_t s_rank[kSortMax];
  __shared__ uint64_t s_ranked[kRankMax];
  __shared__ int s_kstar;
  __shared__ int s_hcnt[kHistBins];
  __shared__ float s_hmass[kHistBins];
  __shared__ int s_bcut;
  const int nk = a.nk;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const bool decode = a.nq == 1;
  const int n = decode ? nk : (row % a.nq) + 1;   // candidates 0..n-1
  const int last = n - 1;
  const int per = (n + nthr - 1) / nthr;          // <= kSelMaxPerThread
  const int c0 = min(tid * per, n);
  const float* srow = a.scores + size_t(row) * nk;

  // this thread's run: candidate c0 + e, e < per
  uint32_t key[kSelMaxPerThread];
  double ex[kSelMaxPerThread];
  float sv[kSelMaxPerThread];
  // Every load in flight before any is used.  When the runs are whole
  // 16-byte groups of a 16-byte aligned row, 16-byte buffer loads: a wave's
  // 4-byte loads of contiguous runs touch one 64-byte segment per lane and
  // instruction, which the vector cache serves a segment per cycle (with 16
  // candidates per thread that alone took 3 of the 15 us of a decode row).
  // Reads past the row return 0 (they belong to no candidate).
  if ((per & 3) == 0 && (nk & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15u) == 0) {
    const __amdgpu_buffer_rsrc_t rrow =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(srow), 0, nk * 4, 0x00020000);
#pragma unroll
    for (int j = 0; j < kSelMaxPerThread / 4; ++j) {
      const uint32_t off = (4 * j < per) ? uint32_t(c0 + 4 * j) * 4u : 0x80000000u;
      const float4 v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rrow, off, 0, 0));
      sv[4 * j] = v.x;
      sv[4 * j + 1] = v.y;
      sv[4 * j + 2] = v.z;
      sv[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      const int c = c0 + e;
      sv[e] = srow[(e < per && c < n) ? c : 0];
    }
  }
  uint32_t resid = 0, forcedm = 0;   // bit masks over the run
  float smax = -kInf;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e) {
    key[e] = 0u;
    ex[e] = 0.0;
    const int c = c0 + e;
    if (e < per && c < n) {
      const bool f = c < a.n_sink || c > last - a.n_recent;
      if (f) {
        forcedm |= 1u << e;
      } else {
        resid |= 1u << e;
        key[e] = score_key(sv[e]);
        smax = fmaxf(smax, sv[e]);
      }
    }
  }
  // forced blocks: the first n_sink and the last n_recent of the n candidates (they may overlap)
  const int n_res = n - min(n, min(n, max(a.n_sink, 0)) + min(n, max(a.n_recent, 0)));

  if (a.top_p >= 1.0f) {   // every residual block
    write_row(a, row, forcedm | resid, c0, sc);
    return;
  }
  const int kfloor = min(a.k_min, n_res);
  const bool by_mass = a.top_p > 0.0f && n_res > 0;
  if (!by_mass && kfloor == 0) {   // forced blocks only
    write_row(a, row, forcedm, c0, sc);
    return;
  }

  // ---- exact sort of the candidates that can be kept
  float gmax = 0.f;
  double target = 0.0;
  uint32_t candm = resid;
  if (by_mass) {
    gmax = block_max_f32(smax, sc);
    double local = 0.0;
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e)
      if (resid & (1u << e)) {
        ex[e] = double(__expf(key_score(key[e]) - gmax));
        local += ex[e];
      }
    const double z = block_sum_f64(local, sc);
    target = double(a.top_p) * z;
    if (n_res > kSortMax) {
      const double bound = (1.0 - double(a.top_p)) * z / double(n_res) * (1.0 - 1e-6);
      candm = 0;
#pragma unroll
      for (int e = 0; e < kSelMaxPerThread; ++e)
        if ((resid & (1u << e)) && ex[e] > bound) candm |= 1u << e;
    }
  }
  bool filtered = candm != resid || n_res > kSortMax;
  if (by_mass && n_res > kRefineMin) {
    // Narrow the candidates with a histogram of their masses over score bins
    // below the row max: keep the bins down to one past the bin where the
    // (fp32, any-order) cumulative mass first reaches the target.  The kept
    // set is still decided by the exact scan below over a prefix of the
    // sorted order; if the narrowed set falls short of the target, that scan
    // finds no crossing and the cutoff search runs instead.
    if (tid < kHistBins) {
      s_hcnt[tid] = 0;
      s_hmass[tid] = 0.f;
    }
    __syncthreads();
    uint8_t bin[kSelMaxPerThread];
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      bin[e] = 0;
      if (candm & (1u << e)) {
        const float dsc = (gmax - key_score(key[e])) * kHistScale;
        const int bi = dsc < float(kHistBins - 1) ? int(dsc) : kHistBins - 1;
        bin[e] = uint8_t(bi);
        atomicAdd(&s_hcnt[bi], 1);
        atomicAdd(&s_hmass[bi], float(ex[e]));
      }
    }
    __syncthreads();
    static_assert(kHistBins == 64, "one wave scans the bins, lane b holding bin b");
    if (tid < 64) {
      const float goal = float(target) * 1.001f;
      float cum = s_hmass[tid];
      int cnt = s_hcnt[tid];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(cum, o);
        const int z = __shfl_up(cnt, o);
        if (tid >= o) {
          cum += y;
          cnt += z;
        }
      }
      const int total = __shfl(cnt, 63);
      const unsigned long long hit = __ballot(cum >= goal);
      const int b = hit ? __ffsll((long long)hit) - 1 : kHistBins;   // first bin reaching the goal
      const int bcut = min(b + 1, kHistBins - 1);
      const int upto = __shfl(cnt, bcut);                               // candidates in bins 0..bcut
      if (tid == 0)
        s_bcut = (total > kRefineMin && b < kHistBins && upto < total && upto >= kfloor) ? bcut : kHistBins;
    }
    __syncthreads();
    const int bcut = s_bcut;   // kHistBins: keep all
    if (bcut < kHistBins) {
#pragma unroll
      for (int e = 0; e < kSelMaxPerThread; ++e)
        if ((candm & (1u << e)) && int(bin[e]) > bcut) candm &= ~(1u << e);
      filtered = true;
    }
  }
  int ncand;
  const int off = block_excl_scan_i32(__popc(candm), sc, ncand);
  if (ncand <= kSortMax && ncand >= kfloor) {
    int w = off;
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e)
      if (candm & (1u << e)) {
        s_sort[w] = (uint64_t(~key[e]) << 32) | uint32_t(w);   // ascending: score desc, then id asc
        ++w;
      }
    const uint64_t* ord;   // the candidates in ascending key order
    const int rounds = (ncand + nthr - 1) / nthr;
    if (ncand <= kRankMax && rounds <= kRankRounds && rounds * ncand <= kRankReads) {
      if (tid == 0) s_sort[ncand] = ~0ull;   // pads an odd count; never below a key
      __syncthreads();
      if (rounds == 1) rank_by_count<1>(s_sort, ncand, s_rank, s_ranked);
      else rank_by_count<kRankRounds>(s_sort, ncand, s_rank, s_ranked);
      __syncthreads();
      ord = s_ranked;
    } else {
      int cap = 2;
      while (cap < ncand) cap <<= 1;
      for (int k = ncand + tid; k < cap; k += nthr) s_sort[k] = ~0ull;
      __syncthreads();
      for (int k = 2; k <= cap; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int e = tid; e < cap; e += nthr) {
            const int p = e ^ j;
            if (p > e) {
              const uint64_t x = s_sort[e], y = s_sort[p];
              if ((x > y) == ((e & k) == 0)) {
                s_sort[e] = y;
                s_sort[p] = x;
              }
            }
          }
          __syncthreads();
        }
      }
      for (int k = tid; k < ncand; k += nthr) s_rank[uint32_t(s_sort[k])] = uint16_t(k);
      ord = s_sort;
    }
    int kstar = 0;
    if (by_mass) {
      if (tid == 0) s_kstar = 0x7fffffff;
      const int rper = (ncand + nthr - 1) / nthr;
      const int k0 = min(tid * rper, ncand), k1 = min(k0 + rper, ncand);
      double part = 0.0;
      for (int kk = k0; kk < k1; ++kk) part += double(__expf(key_score(~uint32_t(ord[kk] >> 32)) - gmax));
      double tot;
      double cum = block_excl_scan_f64(part, sc, tot);
      for (int kk = k0; kk < k1; ++kk) {
        const double prev = cum;
        cum += double(__expf(key_score(~uint32_t(ord[kk] >> 32)) - gmax));
        if (cum >= target && !(prev >= target)) {
          atomicMin(&s_kstar, kk + 1);
          break;
        }
      }
      __syncthreads();
      kstar = s_kstar;
      if (kstar == 0x7fffffff) kstar = filtered ? -1 : ncand;   // rounding at p close to 1: keep all
    } else {
      __syncthreads();
    }
    if (kstar >= 0) {
      const int kfinal = max(kstar, kfloor);
      uint32_t keepm = forcedm;
      int pidx = off;
#pragma unroll
      for (int e = 0; e < kSelMaxPerThread; ++e)
        if (candm & (1u << e)) {
          if (s_rank[pidx] < kfinal) keepm |= 1u << e;
          ++pidx;
        }
      write_row(a, row, keepm, c0, sc);
      return;
    }
  }

  // kept residual: key > kcut, plus the first mtie candidates with key == kcut
  uint32_t kcut = 0u;
  int mtie = 0;
  bool keep_all = false, keep_none = false;
  if (a.top_p >= 1.0f) {
    keep_all = true;
  } else {
    int kstar = 0;
    if (a.top_p > 0.0f && n_res > 0) {
      const float gmax = block_max_f32(smax, sc);
      double local = 0.0;
#pragma unroll
      for (int e = 0; e < kSelMaxPerThread; ++e)
        if (resid & (1u << e)) {
          ex[e] = double(__expf(key_score(key[e]) - gmax));
          local += ex[e];
        }
      const double z = block_sum_f64(local, sc);
      const double target = double(a.top_p) * z;
      // largest K with mass(key >= K) >= target (K = 0 always qualifies)
      uint32_t lo = 0u, hi = 0xffffffffu;
      while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < kSelMaxPerThread; ++e)
          if ((resid & (1u << e)) && key[e] >= mid) part += ex[e];
        if (block_sum_f64(part, sc) >= target) lo = mid;
        else hi = mid - 1u;
      }
      kcut = lo;
      double above = 0.0;
      int n_above = 0, n_tie = 0;
#pragma unroll
      for (int e = 0; e < kSelMaxPerThread; ++e)
        if (resid & (1u << e)) {
          if (key[e] > kcut) { above += ex[e]; ++n_above; }
          else if (key[e] == kcut) ++n_tie;
        }
      above = block_sum_f64(above, sc);
      n_above = block_sum_i32(n_above, sc);
      n_tie = block_sum_i32(n_tie, sc);
      // ties share one mass; take the fewest (in id order) that reach the target
      const double e_tie = double(__expf(key_score(kcut) - gmax));
      const double need = ceil((target - above) / e_tie);
      mtie = need < 1.0 ? 1 : (need > double(n_tie) ? n_tie : int(need));
      kstar = n_above + mtie;
    }
    const int kfloor = min(a.k_min, n_res);
    if (kstar < kfloor) {
      // floor K_min: largest K with count(key >= K) >= kfloor, ties by id
      uint32_t lo = 0u, hi = 0xffffffffu;
      while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;
        int part = 0;
#pragma unroll
        for (int e = 0; e < kSelMaxPerThread; ++e)
          if ((resid & (1u << e)) && key[e] >= mid) ++part;
        if (block_sum_i32(part, sc) >= kfloor) lo = mid;
        else hi = mid - 1u;
      }
      kcut = lo;
      int n_above = 0;
#pragma unroll
      for (int e = 0; e < kSelMaxPerThread; ++e)
        if ((resid & (1u << e)) && key[e] > kcut) ++n_above;
      n_above = block_sum_i32(n_above, sc);
      mtie = kfloor - n_above;
      kstar = kfloor;
    }
    keep_none = kstar == 0;
  }

  // rank of this thread's ties in id order
  int my_ties = 0;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e)
    if ((resid & (1u << e)) && key[e] == kcut) ++my_ties;
  int tie_total;
  int tie_rank = block_excl_scan_i32(my_ties, sc, tie_total);

  uint32_t keepm = forcedm;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e) {
    if (!(resid & (1u << e))) continue;
    bool k;
    if (keep_all) {
      k = true;
    } else if (keep_none) {
      k = false;
    } else if (key[e] == kcut) {
      k = tie_rank < mtie;
      ++tie_rank;
    } else {
      k = key[e] > kcut;
    }
    if (k) keepm |= 1u << e;
  }
  write_row(a, row, keepm, c0, sc);
}

// Visiting order of the history blocks for early-stopped attention (S2O
// section 2: candidates are processed in descending estimated importance).
// One workgroup per (batch, KV head, query block) row: the blocks of earlier
// segments are sorted in LDS by a bitonic network on 64-bit keys (inverted
// order-preserving score bits above the block id: ascending keys are
// score-descending with ties to the lower id).
constexpr int kOrderThreads = 256;
__global__ __launch_bounds__(kOrderThreads) void order_history_kernel(OrderArgs a) {
  __shared__ uint64_t s_key[kOrderMaxBlocks];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int i = row % a.nb;
  const int n = ((i * a.block) / a.segment) * a.segment / a.block;
  const float* sc = a.scores + size_t(row) * a.nb;
  int cap = 2;
  while (cap < n) cap <<= 1;
  for (int k = tid; k < cap; k += kOrderThreads)
    s_key[k] = k < n ? ((uint64_t(~score_key(sc[k])) << 32) | uint32_t(k)) : ~0ull;
  __syncthreads();
  if (n > 1) {
    for (int k = 2; k <= cap; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int e = tid; e < cap; e += kOrderThreads) {
          const int p = e ^ j;
          if (p > e) {
            const uint64_t x = s_key[e], y = s_key[p];
            if ((x > y) == ((e & k) == 0)) {
              s_key[e] = y;
              s_key[p] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  int32_t* out = a.order + size_t(row) * a.nb;
  for (int k = tid; k < a.nb; k += kOrderThreads) out[k] = k < n ? int32_t(uint32_t(s_key[k])) : -1;
  if (tid == 0) a.cnt[row] = n;
}

hipError_t launch_order_history(const OrderArgs& a, hipStream_t s) {
  order_history_kernel<<<a.rows, kOrderThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_topp(const SelectArgs& a, hipStream_t s) {
  // as few waves as keep every thread at kSelMaxPerThread candidates or fewer:
  // the row is a chain of block-wide steps, and barriers over fewer waves are cheaper
  int threads = 64;
  while (threads < 1024 && threads * kSelTargetPerThread < a.nk) threads <<= 1;
  select_topp_kernel<<<a.rows, threads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace spot
