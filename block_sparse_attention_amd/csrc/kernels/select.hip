// Dual top-p block selection for gfx950 (SpotAttention section 3, "Dual Top-p
// Selectieregel"): reserved sink and recency blocks, nucleus selection on the
// residual distribution until the cumulative mass reaches p, floor K_min.
//
// One workgroup per row.  The residual candidates are sorted in LDS (bitonic
// network on 64-bit keys: inverted order-preserving score bits above the
// block id, so ascending keys are score-descending with ties to the lower id),
// their softmax masses are prefix-summed in fp64, the crossing index is found,
// and the kept set is compacted to ascending block ids.
#include "../launch.h"
#include "common.h"

namespace spot {

__device__ __forceinline__ uint32_t score_desc_bits(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// Block-wide exclusive scan of one value per thread (blockDim.x <= 1024).
template <typename V>
__device__ V block_exclusive_scan(V x, V* buf, V& total) {
  const int t = threadIdx.x, n = blockDim.x;
  buf[t] = x;
  __syncthreads();
  for (int o = 1; o < n; o <<= 1) {
    V y = (t >= o) ? buf[t - o] : V(0);
    __syncthreads();
    buf[t] += y;
    __syncthreads();
  }
  const V incl = buf[t];
  total = buf[n - 1];
  __syncthreads();
  return incl - x;
}

__global__ __launch_bounds__(1024) void select_topp_kernel(SelectArgs a) {
  extern __shared__ unsigned char lds[];
  const int nk = a.nk;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const bool decode = a.nq == 1;
  const int n = decode ? nk : (row % a.nq) + 1;  // candidates 0..n-1
  const int last = n - 1;
  int sort_n = 2;
  while (sort_n < n) sort_n <<= 1;

  int cap = 2;
  while (cap < nk) cap <<= 1;
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);                       // [cap >= sort_n]
  double* scan = reinterpret_cast<double*>(lds + sizeof(uint64_t) * cap);  // [1024]
  uint8_t* flag = reinterpret_cast<uint8_t*>(scan + 1024);                 // [nk]
  __shared__ int s_kstar;

  const float* srow = a.scores + size_t(row) * nk;
  auto forced = [&](int c) { return c < a.n_sink || c > last - a.n_recent; };

  for (int c = tid; c < sort_n; c += nthr) {
    uint64_t key = ~0ull;
    if (c < n && !forced(c)) key = (uint64_t(score_desc_bits(srow[c])) << 32) | uint32_t(c);
    keys[c] = key;
  }
  for (int c = tid; c < nk; c += nthr) flag[c] = (c < n && forced(c)) ? 1 : 0;
  int n_forced = 0;
  {
    // |{c < n : c < n_sink or c > last - n_recent}|
    const int lo = min(max(a.n_sink, 0), n);
    const int hi_start = max(last - a.n_recent + 1, 0);
    const int hi = n - max(hi_start, lo);
    n_forced = lo + max(hi, 0);
  }
  const int n_res = n - n_forced;
  __syncthreads();

  // bitonic sort, ascending
  for (int k = 2; k <= sort_n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = tid; e < sort_n; e += nthr) {
        const int p = e ^ j;
        if (p > e) {
          const uint64_t x = keys[e], y = keys[p];
          const bool up = (e & k) == 0;
          if ((x > y) == up) {
            keys[e] = y;
            keys[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  int kstar;
  if (a.top_p >= 1.0f) {
    kstar = n_res;
  } else if (a.top_p <= 0.0f || n_res == 0) {
    kstar = 0;
  } else {
    // masses exp(s_k - s_top) in sorted order, prefix sums in fp64
    const double s_top = double(srow[uint32_t(keys[0])]);
    const int per = (n_res + nthr - 1) / nthr;
    const int k0 = min(tid * per, n_res), k1 = min(k0 + per, n_res);
    double local = 0.0;
    for (int kk = k0; kk < k1; ++kk) local += exp(double(srow[uint32_t(keys[kk])]) - s_top);
    double total;
    const double before = block_exclusive_scan<double>(local, scan, total);
    if (tid == 0) s_kstar = n_res;
    __syncthreads();
    const double target = double(a.top_p) * total;
    double c = before;
    for (int kk = k0; kk < k1; ++kk) {
      const double prev = c;
      c += exp(double(srow[uint32_t(keys[kk])]) - s_top);
      if (c >= target && !(prev >= target)) atomicMin(&s_kstar, kk + 1);
    }
    __syncthreads();
    kstar = s_kstar;
  }
  kstar = max(kstar, min(a.k_min, n_res));

  for (int kk = tid; kk < kstar; kk += nthr) flag[uint32_t(keys[kk])] = 1;
  __syncthreads();

  // compact flags to ascending ids
  const int per = (nk + nthr - 1) / nthr;
  const int c0 = min(tid * per, nk), c1 = min(c0 + per, nk);
  int mine = 0;
  for (int c = c0; c < c1; ++c) mine += flag[c];
  int total_kept;
  int pos = block_exclusive_scan<int>(mine, reinterpret_cast<int*>(scan), total_kept);
  int32_t* irow = a.idx + size_t(row) * nk;
  for (int c = c0; c < c1; ++c)
    if (flag[c]) irow[pos++] = c;
  for (int c = total_kept + tid; c < nk; c += nthr) irow[c] = -1;
  if (tid == 0) a.cnt[row] = total_kept;
}

static size_t select_lds_bytes(int nk) {
  size_t cap = 2;
  while (cap < size_t(nk)) cap <<= 1;
  return sizeof(uint64_t) * cap + sizeof(double) * 1024 + size_t(nk);
}

hipError_t launch_select_topp(const SelectArgs& a, hipStream_t s) {
  int threads = 64;
  while (threads < 1024 && threads * 2 < a.nk) threads <<= 1;
  const size_t lds = select_lds_bytes(a.nk);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_topp_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  select_topp_kernel<<<a.rows, threads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace spot
