// Dual top-p block selection for gfx950 (SpotAttention section 3, "Dual Top-p
// Selectieregel"): reserved sink and recency blocks, nucleus selection on the
// residual distribution until the cumulative mass reaches p, floor K_min.
//
// One workgroup per row; each thread owns a contiguous run of candidate ids.
// Rows of at most 2048 candidates are ordered exactly: each residual
// candidate's rank is the number of candidates ahead of it (higher score, or
// equal score and lower id), the masses are prefix-summed in fp64 in rank
// order and the first prefix reaching p ends the kept set.  Longer rows
// (decode) search the cutoff instead of sorting: with
// key(s) = order-preserving bits of the score, the kept residual set of the
// rule (scores descending, ties to the lower block id, shortest prefix whose
// mass reaches p) is {key > K} plus the first m candidates with key == K in
// id order, where K is the largest key whose upper set {key >= K} still holds
// mass >= p.  K is found by binary search over the 32-bit key space; every
// mass is a fixed-order fp64 reduction (per-thread runs, then wave
// butterflies, then waves in order), so the result is deterministic.
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kSelMaxPerThread = 16;   // candidates per thread (16384 / 1024)
constexpr int kRankMax = 2048;         // rows up to this length are ranked exactly

__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct SelScratch {
  double d[32];
  int i[32];
  uint32_t u[32];
  float f[32];
};

__device__ double block_sum_f64(double x, SelScratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if (lane == 0) sc.d[w] = x;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < nw; ++k) t += sc.d[k];
  __syncthreads();
  return t;
}

__device__ int block_sum_i32(int x, SelScratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if (lane == 0) sc.i[w] = x;
  __syncthreads();
  int t = 0;
  for (int k = 0; k < nw; ++k) t += sc.i[k];
  __syncthreads();
  return t;
}

__device__ float block_max_f32(float x, SelScratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_max(x);
  if (lane == 0) sc.f[w] = x;
  __syncthreads();
  float t = -kInf;
  for (int k = 0; k < nw; ++k) t = fmaxf(t, sc.f[k]);
  __syncthreads();
  return t;
}

// exclusive prefix (in thread order) of one int per thread, plus the total
__device__ int block_excl_scan_i32(int x, SelScratch& sc, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sc.i[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int k = 0; k < nw; ++k) {
    if (k < w) before += sc.i[k];
    tot += sc.i[k];
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

__device__ double block_excl_scan_f64(double x, SelScratch& sc, double& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  double incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sc.d[w] = incl;
  __syncthreads();
  double before = 0.0, tot = 0.0;
  for (int k = 0; k < nw; ++k) {
    if (k < w) before += sc.d[k];
    tot += sc.d[k];
  }
  __syncthreads();
  total = tot;
  return before + (incl - x);
}

// kept ids ascending (thread runs are contiguous and in order), -1 padding, count
__device__ void write_row(const SelectArgs& a, int row, uint32_t keepm, int c0, SelScratch& sc) {
  int total_kept;
  int pos = block_excl_scan_i32(__popc(keepm), sc, total_kept);
  int32_t* irow = a.idx + size_t(row) * a.nk;
#pragma unroll
  for (int e = 0; e < kSelMaxPerThread; ++e)
    if (keepm & (1u << e)) irow[pos++] = c0 + e;
  for (int c = total_kept + threadIdx.x; c < a.nk; c += blockDim.x) irow[c] = -1;
  if (threadIdx.x == 0) a.cnt[row] = total_kept;
}

__global__ __launch_bounds__(1024) void select_topp_kernel(SelectArgs a) {
  __shared__ SelScratch sc;
  __shared__ uint32_t s_key[kRankMax];
  __shared__ uint16_t s_sorted[kRankMax];
  __shared__ uint8_t s_flag[kRankMax];
  __shared__ int s_kstar;
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
        const float s = srow[c];
        resid |= 1u << e;
        key[e] = score_key(s);
        smax = fmaxf(smax, s);
      }
    }
  }
  const int n_res = block_sum_i32(__popc(resid), sc);

  if (n <= kRankMax) {
    // ---- exact order by rank (rows up to kRankMax candidates)
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      const int c = c0 + e;
      if (e < per && c < n) {
        s_key[c] = (resid & (1u << e)) ? key[e] : 0u;   // 0: not a residual candidate
        s_flag[c] = (forcedm & (1u << e)) ? 1 : 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      if (!(resid & (1u << e))) continue;
      const int c = c0 + e;
      const uint32_t k = key[e];
      int rank = 0;
      for (int o = 0; o < n; ++o) {
        const uint32_t ko = s_key[o];
        rank += (ko > k || (ko == k && o < c)) ? 1 : 0;
      }
      s_sorted[rank] = uint16_t(c);
    }
    __syncthreads();
    int kstar;
    if (a.top_p >= 1.0f) {
      kstar = n_res;
    } else if (a.top_p <= 0.0f || n_res == 0) {
      kstar = 0;
    } else {
      const float gmax = block_max_f32(smax, sc);
      const int rper = (n_res + nthr - 1) / nthr;
      const int k0 = min(tid * rper, n_res), k1 = min(k0 + rper, n_res);
      double local = 0.0;
      for (int kk = k0; kk < k1; ++kk) local += double(__expf(srow[s_sorted[kk]] - gmax));
      double z;
      const double before = block_excl_scan_f64(local, sc, z);
      if (tid == 0) s_kstar = n_res;
      __syncthreads();
      const double target = double(a.top_p) * z;
      double cum = before;
      for (int kk = k0; kk < k1; ++kk) {
        const double prev = cum;
        cum += double(__expf(srow[s_sorted[kk]] - gmax));
        if (cum >= target && !(prev >= target)) {
          atomicMin(&s_kstar, kk + 1);
          break;
        }
      }
      __syncthreads();
      kstar = s_kstar;
    }
    kstar = max(kstar, min(a.k_min, n_res));
    for (int kk = tid; kk < kstar; kk += nthr) s_flag[s_sorted[kk]] = 1;
    __syncthreads();
    uint32_t keepm = 0;
#pragma unroll
    for (int e = 0; e < kSelMaxPerThread; ++e) {
      const int c = c0 + e;
      if (e < per && c < n && s_flag[c]) keepm |= 1u << e;
    }
    write_row(a, row, keepm, c0, sc);
    return;
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

hipError_t launch_select_topp(const SelectArgs& a, hipStream_t s) {
  // enough threads that each owns at most kSelMaxPerThread candidates (and ~4 when possible)
  int threads = 64;
  while (threads < 1024 && threads * 4 < a.nk) threads <<= 1;
  select_topp_kernel<<<a.rows, threads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace spot
