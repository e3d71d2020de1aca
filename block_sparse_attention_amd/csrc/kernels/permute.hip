// Key permutation by global importance for gfx950 (PBS-Attn section 3,
// "Op Globale Belang Gebaseerde Key-Permutatie"): the importance of every key
// is the attention probability it receives from the last block of queries,
// mean-pooled over those query rows and the query heads of the KV group;
// inside each segment the keys are sorted by importance, descending (ties by
// position), which gives the logical -> physical index array the sparse
// attention gathers through (S2O section 1, index-driven loading).
//
// perm_lse_kernel   split over key chunks: per query row of the last block,
//                   running max and sum of exp over the chunk's visible keys
//                   (S^T = K Q^T on MFMA, one query per lane column).
// perm_imp_kernel   merges the chunk partials into each row's log-sum-exp,
//                   then S = Q K^T on MFMA (one key per lane column): the
//                   probabilities of the wave's 32 rows are summed in-lane, the
//                   8 waves in fixed order; one partial per query-row group.
// perm_sort_kernel  one workgroup per segment: sums the row-group partials,
//                   sorts (importance desc, position asc) with a bitonic
//                   network in LDS and writes perm (and the importance).
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kPermChunk = 1024;   // keys per workgroup in the two MFMA passes
constexpr int kPermKT = 64;        // keys per tile
constexpr int kPermNW = 8;         // waves per workgroup (32 query rows each)
constexpr int kPermRows = kPermNW * 32;
static_assert(kPermRows == kPermRowsPerGroup, "row group size shared with the host layer");

__device__ __forceinline__ void perm_row(const PermArgs& a, int group, int wv, int ql, int& h, int& r, bool& valid) {
  const int G = a.hq / a.hkv;
  const int nr = a.L - (a.nb - 1) * a.block;   // rows of the last query block
  const int pr = group * kPermRows + wv * 32 + ql;
  valid = pr < G * nr;
  const int prc = valid ? pr : 0;
  h = prc / nr;               // head within the group
  r = a.L - nr + prc % nr;    // query position
}

// stage one 64-key tile of K (rows c0 .. c0+63, zero beyond L) in LDS
template <int D>
__device__ __forceinline__ void stage_k(const uint16_t* Kg, int c0, int L, uint16_t* ks) {
  constexpr int KLD = D + 8;
  constexpr int CPR = D / 8;
  for (int cid = threadIdx.x; cid < kPermKT * CPR; cid += kPermNW * 64) {
    const int row = cid / CPR, col8 = cid % CPR;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c0 + row < L) v = *reinterpret_cast<const uint4*>(Kg + size_t(c0 + row) * D + col8 * 8);
    *reinterpret_cast<uint4*>(&ks[row * KLD + col8 * 8]) = v;
  }
}

template <int D>
__device__ __forceinline__ void load_q(const PermArgs& a, int b, int g, int h, int r, int hf, bf16x8_t (&qf)[D / 16]) {
  const int G = a.hq / a.hkv;
  const uint16_t* qrow = a.q + ((size_t(b) * a.hq + g * G + h) * a.L + r) * D;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16 + hf * 8));
}

template <int D>
__global__ __launch_bounds__(kPermNW * 64) void perm_lse_kernel(PermArgs a, float scale_log2) {
  constexpr int KLD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kPermKT * KLD];
  const int chunk = blockIdx.x, group = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, ql = lane & 31, hf = lane >> 5;
  int h, r;
  bool valid;
  perm_row(a, group, wv, ql, h, r, valid);
  bf16x8_t qf[D / 16];
  load_q<D>(a, b, g, h, r, hf, qf);
  const uint16_t* Kg = a.k + size_t(bg) * a.L * D;

  float m = -kInf, l = 0.f;
  const int kbeg = chunk * kPermChunk, kend = min(a.L, kbeg + kPermChunk);
  for (int c0 = kbeg; c0 < kend; c0 += kPermKT) {
    __syncthreads();
    stage_k<D>(Kg, c0, a.L, Ks);
    __syncthreads();
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&Ks[(rt * 32 + ql) * KLD + ks * 16 + hf * 8]);
        s[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[rt], 0, 0, 0);
      }
    float mx = -kInf;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = c0 + rt * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        const float x = (t <= r) ? s[rt][e] * scale_log2 : -kInf;   // t <= r < L
        s[rt][e] = x;
        mx = __builtin_fmaxf(mx, x);
      }
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = __builtin_fmaxf(m, mx);
    if (m_new != -kInf) {
      float add = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) add += __builtin_amdgcn_exp2f(s[rt][e] - m_new);
      l = (m == -kInf ? 0.f : l * __builtin_amdgcn_exp2f(m - m_new)) + add;
      m = m_new;
    }
  }
  l += __shfl_xor(l, 32);
  if (valid && hf == 0) {
    float* part = a.ws_lse + ((size_t(bg) * a.nchunks + chunk) * a.ngroups * kPermRows + group * kPermRows +
                              wv * 32 + ql) * 2;
    part[0] = m;
    part[1] = l;
  }
}

template <int D>
__global__ __launch_bounds__(kPermNW * 64) void perm_imp_kernel(PermArgs a, float scale_log2) {
  constexpr int KLD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kPermKT * KLD];
  __shared__ float s_lse[kPermRows];
  __shared__ int s_pos[kPermRows];
  __shared__ float s_col[kPermNW][kPermKT];
  const int chunk = blockIdx.x, group = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, ql = lane & 31, hf = lane >> 5;
  int h, r;
  bool valid;
  perm_row(a, group, wv, ql, h, r, valid);

  // log2-sum-exp of each of the group's rows, merged over all chunks in order
  if (hf == 0) {
    const int row = wv * 32 + ql;
    float M = -kInf, Lsum = 0.f;
    if (valid) {
      for (int c = 0; c < a.nchunks; ++c) {
        const float* p = a.ws_lse + ((size_t(bg) * a.nchunks + c) * a.ngroups * kPermRows + group * kPermRows + row) * 2;
        const float mc = p[0], lc = p[1];
        if (mc == -kInf) continue;
        if (mc > M) {
          Lsum = (M == -kInf ? 0.f : Lsum * __builtin_amdgcn_exp2f(M - mc));
          M = mc;
        }
        Lsum += lc * __builtin_amdgcn_exp2f(mc - M);
      }
    }
    s_lse[row] = valid ? M + __log2f(Lsum) : kInf;   // +inf: contributes exp2(-inf) = 0
    s_pos[row] = valid ? r : -1;
  }
  bf16x8_t qf[D / 16];
  load_q<D>(a, b, g, h, r, hf, qf);
  const uint16_t* Kg = a.k + size_t(bg) * a.L * D;
  float* out = a.ws_imp + (size_t(bg) * a.ngroups + group) * a.L;
  __syncthreads();
  // the 16 query rows this lane's S entries belong to (fixed for the whole pass)
  float lse_r[16];
  int pos_r[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = wv * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
    lse_r[e] = s_lse[row];
    pos_r[e] = s_pos[row];
  }

  const int kbeg = chunk * kPermChunk, kend = min(a.L, kbeg + kPermChunk);
  for (int c0 = kbeg; c0 < kend; c0 += kPermKT) {
    __syncthreads();
    stage_k<D>(Kg, c0, a.L, Ks);
    __syncthreads();
    // S = Q K^T: A = Q fragment (row = query), B = K fragment (column = key)
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&Ks[(rt * 32 + ql) * KLD + ks * 16 + hf * 8]);
        s[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, s[rt], 0, 0, 0);
      }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int t = c0 + rt * 32 + ql;   // this lane's key
      float col = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        col += (t <= pos_r[e]) ? __builtin_amdgcn_exp2f(s[rt][e] * scale_log2 - lse_r[e]) : 0.f;
      col += __shfl_xor(col, 32);
      if (hf == 0) s_col[wv][rt * 32 + ql] = col;
    }
    __syncthreads();
    if (threadIdx.x < kPermKT && c0 + threadIdx.x < a.L) {
      float acc = 0.f;
      for (int w = 0; w < kPermNW; ++w) acc += s_col[w][threadIdx.x];
      out[c0 + threadIdx.x] = acc;
    }
  }
}

__global__ __launch_bounds__(1024) void perm_sort_kernel(PermArgs a, float inv_rows) {
  extern __shared__ uint64_t s_keys[];
  const int seg = blockIdx.x, bg = blockIdx.y;
  const int s0 = seg * a.segment;
  const int n = min(a.segment, a.L - s0);
  int cap = 2;
  while (cap < n) cap <<= 1;
  const float* part = a.ws_imp + size_t(bg) * a.ngroups * a.L;
  for (int k = threadIdx.x; k < cap; k += blockDim.x) {
    uint64_t key = ~0ull;
    if (k < n) {
      float imp = 0.f;
      for (int grp = 0; grp < a.ngroups; ++grp) imp += part[size_t(grp) * a.L + s0 + k];
      imp *= inv_rows;
      if (a.importance) a.importance[size_t(bg) * a.L + s0 + k] = imp;
      // importance >= 0: its bits order like the values; invert for descending
      key = (uint64_t(~__float_as_uint(imp)) << 32) | uint32_t(k);
    }
    s_keys[k] = key;
  }
  __syncthreads();
  for (int k = 2; k <= cap; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = threadIdx.x; e < cap; e += blockDim.x) {
        const int p = e ^ j;
        if (p > e) {
          const uint64_t x = s_keys[e], y = s_keys[p];
          if ((x > y) == ((e & k) == 0)) {
            s_keys[e] = y;
            s_keys[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  int32_t* prow = a.perm + size_t(bg) * a.L + s0;
  for (int k = threadIdx.x; k < n; k += blockDim.x) prow[k] = s0 + int(uint32_t(s_keys[k]));
}

int perm_num_chunks(int L) { return (L + kPermChunk - 1) / kPermChunk; }
int perm_num_groups(int G, int nr) { return (G * nr + kPermRows - 1) / kPermRows; }
size_t perm_workspace_bytes(int batch, int hkv, int L, int G, int nr) {
  const size_t bg = size_t(batch) * hkv;
  const size_t ng = size_t(perm_num_groups(G, nr));
  return bg * perm_num_chunks(L) * ng * kPermRows * 2 * sizeof(float) + bg * ng * size_t(L) * sizeof(float);
}

template <int D>
static hipError_t launch_perm_d(PermArgs a, hipStream_t s) {
  const float scale_log2 = a.sm_scale * kLog2e;
  const dim3 grid(a.nchunks, a.ngroups, a.batch * a.hkv);
  perm_lse_kernel<D><<<grid, kPermNW * 64, 0, s>>>(a, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  perm_imp_kernel<D><<<grid, kPermNW * 64, 0, s>>>(a, scale_log2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.hq / a.hkv;
  const int nr = a.L - (a.nb - 1) * a.block;
  int cap = 2;
  while (cap < a.segment) cap <<= 1;
  const size_t lds = size_t(cap) * sizeof(uint64_t);
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(perm_sort_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(lds));
    if (e != hipSuccess) return e;
  }
  const int nseg = (a.L + a.segment - 1) / a.segment;
  perm_sort_kernel<<<dim3(nseg, a.batch * a.hkv), 1024, lds, s>>>(a, 1.0f / float(G * nr));
  return hipGetLastError();
}

// ---------------------------------------------------------------- bijection check
// Debug check that perm maps each segment onto itself one to one: one
// workgroup per (segment, batch x KV head) marks the values it sees in an LDS
// bitmap; a value outside the position's segment, or one already marked,
// counts as one violation.  As many values as positions are checked, so zero
// violations means a bijection.
constexpr int kCheckThreads = 256;

__global__ void perm_check_zero(int32_t* bad) {
  if (threadIdx.x == 0) *bad = 0;
}

__global__ __launch_bounds__(kCheckThreads) void perm_check_kernel(PermCheckArgs a) {
  __shared__ uint32_t bits[kPermMaxSegment / 32];
  __shared__ int s_bad[kCheckThreads / 64];
  const int seg = blockIdx.x;
  const size_t pair = blockIdx.y;
  const int s0 = seg * a.segment;
  const int n = min(a.segment, a.L - s0);
  for (int w = threadIdx.x; w < (n + 31) / 32; w += kCheckThreads) bits[w] = 0u;
  __syncthreads();
  const int32_t* p = a.perm + pair * a.L + s0;
  int bad = 0;
  for (int i = threadIdx.x; i < n; i += kCheckThreads) {
    const uint32_t v = uint32_t(p[i]) - uint32_t(s0);   // wraps for values below the segment
    if (v >= uint32_t(n)) {
      ++bad;
      continue;
    }
    const uint32_t m = 1u << (v & 31u);
    if (atomicOr(&bits[v >> 5], m) & m) ++bad;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o);
  if ((threadIdx.x & 63) == 0) s_bad[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kCheckThreads / 64; ++w) t += s_bad[w];
    if (t) atomicAdd(a.bad, t);
  }
}

hipError_t launch_perm_check(const PermCheckArgs& a, hipStream_t s) {
  perm_check_zero<<<1, 64, 0, s>>>(a.bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nseg = (a.L + a.segment - 1) / a.segment;
  perm_check_kernel<<<dim3(unsigned(nseg), unsigned(a.pairs)), kCheckThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_key_permutation(const PermArgs& a, hipStream_t s) {
  if (a.d == 128) return launch_perm_d<128>(a, s);
  if (a.d == 64) return launch_perm_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace spot
