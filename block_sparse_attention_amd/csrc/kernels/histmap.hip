// Per-segment history maps for gfx950 (S2O section 1, historical KV
// permutation): for every segment s >= 1 of a (batch, KV head), the prefix
// positions t < s*S sorted by sm_scale * <qrep_s, k_t> descending, ties by
// position; qrep_s is the mean of Q over the group's heads and the segment's
// rows.  The early-stopped prefill walks the map of its query's segment in
// consecutive runs of B positions.
//
// segmean_kernel    qrep: kHmParts workgroups per (batch, KV head, segment)
//                   each sum a slice of the G x S query rows (HBM-bound read
//                   of Q); segmean_finish adds the slices in order.
// histkey_kernel    one 16-lane row per key t (128 keys per workgroup): the key is read once with
//                   16-byte loads and dotted with the representative query of
//                   every later segment (in LDS); writes 64-bit sort keys
//                   (inverted order-preserving score bits above t).
// histsort_kernel   one workgroup per (batch, KV head, segment): bitonic sort
//                   of the segment's keys in LDS (up to 16384), or, for up to
//                   32768 keys, both halves sorted in LDS in opposite
//                   directions, one compare-exchange pass across the halves in
//                   global memory, and each half merged in LDS.
#include "../launch.h"
#include "common.h"

namespace spot {

__device__ __forceinline__ uint32_t hm_score_key(float s) {
  const uint32_t u = __float_as_uint(s) == 0x80000000u ? 0u : __float_as_uint(s);   // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- segment means
constexpr int kHmParts = 32;   // workgroups per segment mean
template <int D>
__global__ __launch_bounds__(256) void segmean_kernel(HistMapArgs a) {
  constexpr int LPR = D / 8;            // lanes per row, 8 elements each
  constexpr int RP = 256 / LPR;         // rows in flight
  __shared__ float red[RP][D];
  const int sg = blockIdx.x / kHmParts, part = blockIdx.x % kHmParts, g = blockIdx.y, b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int r0 = sg * a.segment;
  const int nr = min(a.segment, a.L - r0);
  const int per = (G * nr + kHmParts - 1) / kHmParts;   // rows (head, row) of this slice
  const int lo = part * per, hi = min(G * nr, lo + per);
  const int lr = threadIdx.x % LPR, rp = threadIdx.x / LPR;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int rr = lo + rp; rr < hi; rr += RP) {
    const int h = g * G + rr / nr, r = r0 + rr % nr;
    const uint4 u = *reinterpret_cast<const uint4*>(a.q + ((size_t(b) * a.hq + h) * a.L + r) * D + lr * 8);
    acc[0] += bf16_lo(u.x); acc[1] += bf16_hi(u.x); acc[2] += bf16_lo(u.y); acc[3] += bf16_hi(u.y);
    acc[4] += bf16_lo(u.z); acc[5] += bf16_hi(u.z); acc[6] += bf16_lo(u.w); acc[7] += bf16_hi(u.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rp][lr * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int r = 0; r < RP; ++r) s += red[r][threadIdx.x];
    a.qpart[(((size_t(b) * a.hkv + g) * a.nseg + sg) * kHmParts + part) * D + threadIdx.x] = s;
  }
}

template <int D>
__global__ __launch_bounds__(D) void segmean_finish(HistMapArgs a) {
  const int sg = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t(b) * a.hkv + g) * a.nseg + sg;
  const int nr = min(a.segment, a.L - sg * a.segment);
  float s = 0.f;
  for (int p = 0; p < kHmParts; ++p) s += a.qpart[(row * kHmParts + p) * D + threadIdx.x];
  a.qrep[row * D + threadIdx.x] = s / float((a.hq / a.hkv) * nr);
}

// ---------------------------------------------------------------- sort keys
constexpr int kHkKeysPerWg = 128;
template <int D>
__global__ __launch_bounds__(256) void histkey_kernel(HistMapArgs a) {
  extern __shared__ float qs[];          // [nseg][D] representative queries of this (batch, KV head)
  const int g = blockIdx.y, b = blockIdx.z;
  const size_t bg = size_t(b) * a.hkv + g;
  for (int e = threadIdx.x; e < a.nseg * D; e += 256) qs[e] = a.qrep[bg * a.nseg * D + e];
  __syncthreads();
  constexpr int LPR = 16, EPL = D / LPR;   // 16 lanes per key, EPL elements each
  const int li = threadIdx.x & 15;
  const int n_last = (a.nseg - 1) * a.segment;    // keys that are history of some segment
  for (int it = 0; it < kHkKeysPerWg / 16; ++it) {
  const int t = blockIdx.x * kHkKeysPerWg + it * 16 + (threadIdx.x >> 4);
  const bool valid = t < n_last;
  float kv[EPL];
  {
    const uint16_t* krow = a.k + (bg * a.L + (valid ? t : 0)) * D + li * EPL;
    if constexpr (EPL == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(krow);
      kv[0] = bf16_lo(u.x); kv[1] = bf16_hi(u.x); kv[2] = bf16_lo(u.y); kv[3] = bf16_hi(u.y);
      kv[4] = bf16_lo(u.z); kv[5] = bf16_hi(u.z); kv[6] = bf16_lo(u.w); kv[7] = bf16_hi(u.w);
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(krow);
      kv[0] = bf16_lo(u.x); kv[1] = bf16_hi(u.x); kv[2] = bf16_lo(u.y); kv[3] = bf16_hi(u.y);
    }
  }
  const int s_first = valid ? t / a.segment + 1 : a.nseg;   // segments whose history holds t
  for (int sg = s_first; sg < a.nseg; ++sg) {
    const float* qv = qs + sg * D + li * EPL;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) d = fmaf(kv[e], qv[e], d);
    d = row16_sum(d);
    if (li == 0)
      a.keys[(bg * a.nseg + sg) * a.kcap + t] = (uint64_t(~hm_score_key(d * a.sm_scale)) << 32) | uint32_t(t);
  }
  }
}

// ---------------------------------------------------------------- sort
constexpr int kHmThreads = 1024;
constexpr int kHmLds = 16384;            // keys sorted in LDS at once

// bitonic stages k = k0..kmax, j down to 1, over s[0..n) in LDS; direction of
// element e: ascending iff (e & k) == 0, flipped when `desc`
__device__ void hm_bitonic(uint64_t* s, int n, int k0, int kmax, bool desc) {
  for (int k = k0; k <= kmax; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = threadIdx.x; e < n; e += kHmThreads) {
        const int p = e ^ j;
        if (p > e) {
          const uint64_t x = s[e], y = s[p];
          const bool asc = ((e & k) == 0) != desc;
          if ((x > y) == asc) {
            s[e] = y;
            s[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Bitonic network over the 1024*R keys s[0..1024R) with R consecutive keys
// per thread: strides below R are register swaps, strides below 64R are
// shuffles inside a wave, larger strides go through LDS with workgroup
// barriers.  Stages k = 2..1024R with `desc` flipping every direction (a full
// sort), or, with merge_only, just the stages j = 512R..1 of an ascending
// merge of a bitonic sequence.
template <int R>
__device__ void hm_sort_block(uint64_t* s, bool desc, bool merge_only) {
  const int tid = threadIdx.x;
  const int n = kHmThreads * R;
  uint64_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = s[tid * R + r];
  for (int k = merge_only ? n : 2; k <= n; k <<= 1) {
    int j = k >> 1;
    if (j >= 64 * R) {   // strides across waves: in LDS
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) s[tid * R + r] = x[r];
      __syncthreads();
      for (; j >= 64 * R; j >>= 1) {
        for (int e = tid; e < n; e += kHmThreads) {
          const int p = e ^ j;
          if (p > e) {
            const uint64_t u = s[e], w = s[p];
            const bool asc = ((e & k) == 0) != desc;
            if ((u > w) == asc) {
              s[e] = w;
              s[p] = u;
            }
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = s[tid * R + r];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {   // strides R*d inside a wave
      if (R * d < k && R * d <= j) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int e = tid * R + r;
          const uint64_t y = __shfl_xor(x[r], d);
          const bool asc = ((e & k) == 0) != desc, lower = (tid & d) == 0;
          x[r] = (asc == lower) ? (x[r] < y ? x[r] : y) : (x[r] < y ? y : x[r]);
        }
      }
    }
#pragma unroll
    for (int jj = R / 2; jj >= 1; jj >>= 1) {   // strides inside a thread
      if (jj < k) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if ((r & jj) == 0) {
            const int e = tid * R + r;
            const bool asc = ((e & k) == 0) != desc;
            const uint64_t lo = x[r] < x[r | jj] ? x[r] : x[r | jj];
            const uint64_t hi = x[r] < x[r | jj] ? x[r | jj] : x[r];
            x[r] = asc ? lo : hi;
            x[r | jj] = asc ? hi : lo;
          }
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) s[tid * R + r] = x[r];
  __syncthreads();
}

__device__ void hm_sort_any(uint64_t* s, int cap, bool desc) {
  switch (cap / kHmThreads) {
    case 16: hm_sort_block<16>(s, desc, false); break;
    case 8: hm_sort_block<8>(s, desc, false); break;
    case 4: hm_sort_block<4>(s, desc, false); break;
    case 2: hm_sort_block<2>(s, desc, false); break;
    case 1: hm_sort_block<1>(s, desc, false); break;
    default: hm_bitonic(s, cap, 2, cap, desc);   // fewer keys than threads
  }
}

__global__ __launch_bounds__(kHmThreads) void histsort_kernel(HistMapArgs a) {
  __shared__ uint64_t s[kHmLds];
  const int sg = blockIdx.x + 1, g = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t(b) * a.hkv + g) * a.nseg + sg;
  uint64_t* gk = a.keys + row * a.kcap;
  int32_t* out = a.hmap + row * a.L;
  const int n = sg * a.segment;
  int cap = 2;
  while (cap < n) cap <<= 1;
  if (cap <= kHmLds) {
    for (int e = threadIdx.x; e < cap; e += kHmThreads) s[e] = e < n ? gk[e] : ~0ull;
    __syncthreads();
    hm_sort_any(s, cap, false);
    for (int e = threadIdx.x; e < n; e += kHmThreads) out[e] = int32_t(uint32_t(s[e]));
  } else {
    // cap == 2 * kHmLds: halves sorted ascending / descending make the whole bitonic
    for (int h = 0; h < 2; ++h) {
      for (int e = threadIdx.x; e < kHmLds; e += kHmThreads) {
        const int x = h * kHmLds + e;
        s[e] = x < n ? gk[x] : ~0ull;
      }
      __syncthreads();
      hm_sort_block<kHmLds / kHmThreads>(s, h == 1, false);
      for (int e = threadIdx.x; e < kHmLds; e += kHmThreads) gk[h * kHmLds + e] = s[e];
      __syncthreads();
    }
    // the stage across the halves (j = kHmLds of the final ascending merge)
    for (int e = threadIdx.x; e < kHmLds; e += kHmThreads) {
      const uint64_t x = gk[e], y = gk[e + kHmLds];
      if (x > y) {
        gk[e] = y;
        gk[e + kHmLds] = x;
      }
    }
    __syncthreads();
    for (int h = 0; h < 2; ++h) {
      for (int e = threadIdx.x; e < kHmLds; e += kHmThreads) s[e] = gk[h * kHmLds + e];
      __syncthreads();
      // stages j = kHmLds/2 .. 1 of the ascending merge of size 2*kHmLds
      hm_sort_block<kHmLds / kHmThreads>(s, false, true);
      for (int e = threadIdx.x; e < kHmLds; e += kHmThreads) {
        const int x = h * kHmLds + e;
        if (x < n) out[x] = int32_t(uint32_t(s[e]));
      }
      __syncthreads();
    }
  }
  for (int e = n + threadIdx.x; e < a.L; e += kHmThreads) out[e] = -1;
}

// map of segment 0 (no history): all -1
__global__ __launch_bounds__(256) void histfill_kernel(HistMapArgs a) {
  const size_t row = (size_t(blockIdx.z) * a.hkv + blockIdx.y) * a.nseg;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < a.L; e += gridDim.x * 256) a.hmap[row * a.L + e] = -1;
}

int hist_key_cap(int nseg, int segment) {
  const int n = (nseg - 1) * segment;
  int cap = 2;
  while (cap < n) cap <<= 1;
  return cap;
}

size_t hist_workspace_bytes(int batch, int hkv, int nseg, int segment, int d) {
  const size_t qrep = size_t(batch) * hkv * nseg * d * sizeof(float);
  const size_t qpart = qrep * kHmParts;
  const size_t keys = size_t(batch) * hkv * nseg * hist_key_cap(nseg, segment) * sizeof(uint64_t);
  return ((qrep + 255) / 256) * 256 + ((qpart + 255) / 256) * 256 + keys;
}

void hist_workspace_split(void* ws, int batch, int hkv, int nseg, int segment, int d, float*& qrep, float*& qpart,
                          uint64_t*& keys) {
  const size_t qb = size_t(batch) * hkv * nseg * d * sizeof(float);
  char* p = static_cast<char*>(ws);
  qrep = reinterpret_cast<float*>(p);
  p += ((qb + 255) / 256) * 256;
  qpart = reinterpret_cast<float*>(p);
  p += ((qb * kHmParts + 255) / 256) * 256;
  keys = reinterpret_cast<uint64_t*>(p);
  (void)segment;
}

template <int D>
static hipError_t launch_hist_d(const HistMapArgs& a, hipStream_t s) {
  segmean_kernel<D><<<dim3(a.nseg * kHmParts, a.hkv, a.batch), 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  segmean_finish<D><<<dim3(a.nseg, a.hkv, a.batch), D, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  histfill_kernel<<<dim3((a.L + 255) / 256 < 64 ? (a.L + 255) / 256 : 64, a.hkv, a.batch), 256, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.nseg < 2) return hipSuccess;
  const int n_last = (a.nseg - 1) * a.segment;
  histkey_kernel<D><<<dim3((n_last + kHkKeysPerWg - 1) / kHkKeysPerWg, a.hkv, a.batch), 256,
                      size_t(a.nseg) * D * sizeof(float), s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  histsort_kernel<<<dim3(a.nseg - 1, a.hkv, a.batch), kHmThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_history_map(const HistMapArgs& a, hipStream_t s) {
  if (a.d == 128) return launch_hist_d<128>(a, s);
  if (a.d == 64) return launch_hist_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace spot
