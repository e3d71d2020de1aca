// Block-sparse decode attention for gfx950.
//
// One query per (sequence, head) at the last position attends the keys of the
// kept 16-token blocks.  The step is bound by reading the kept part of the KV
// cache (SpotAttention "Probleemstelling": every decode step re-reads a cache
// that grows with the context), so the kernel streams rows with 16-byte
// loads, several blocks in flight per thread, and keeps the arithmetic on the
// VALU (bf16 pair dot products, fp32 accumulation).
//
// decode_split_kernel: workgroup = (split s, KV head g, sequence b).  Split s
//   takes kept blocks s, s + nsplit, s + 2*nsplit, ... of sequence b, so the
//   block ids it needs do not depend on the kept count and their loads
//   overlap the count's.  A row of 16 lanes owns one key slot of every block
//   of the split (lane c holds dims c*D/16 .. +D/16), keeps its own
//   online-softmax state for the G query heads of the group, and the 16 slot
//   streams are merged through LDS into one partial (acc, m, l) per head.
// decode_combine_kernel: merges the partials of the splits in split order
//   (deterministic; all loads issued before the merge) and writes O (bf16)
//   and the natural-log LSE.
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;
constexpr float kDecRescale = 8.0f;
constexpr int kDecMaxSplits = 32;

template <int EPL> struct DVec;
template <> struct DVec<8> {
  using T = uint4;
  static __device__ __forceinline__ T ld(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ T zero() { return make_uint4(0u, 0u, 0u, 0u); }
  static __device__ __forceinline__ uint32_t w(const T& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};
template <> struct DVec<4> {
  using T = uint2;
  static __device__ __forceinline__ T ld(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ T zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ uint32_t w(const T& v, int k) { return k == 0 ? v.x : v.y; }
};

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeArgs a, float scale_log2) {
  constexpr int EPL = D / 16;           // elements per lane
  constexpr int KS = kDecThreads / 16;  // key-slot streams per workgroup
  static_assert(KS == 16, "a round's slot u exists for all streams or none when KS divides the block");
  using V = DVec<EPL>;
  __shared__ float s_m[KS][G], s_l[KS][G];
  __shared__ float s_acc[KS][G][D];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, c = tid & 15, ks = tid >> 4;
  const int B = a.block, T = a.T;
  const int32_t* il = a.idx + size_t(b) * a.nk;
  // this split's first kDecUnroll block ids, loaded beside the count
  int pre[kDecUnroll];
#pragma unroll
  for (int u = 0; u < kDecUnroll; ++u) {
    const int bi = s + u * a.nsplit;
    pre[u] = il[bi < a.nk ? bi : 0];
  }
  const int n = a.cnt[b];
  if (s >= n) return;   // the combine reads splits [0, min(n, nsplit)) only
  const int nmine = (n - s + a.nsplit - 1) / a.nsplit;   // blocks s, s+nsplit, ... below n
  const int nslots = nmine * B;
  const size_t kvbase = (size_t(b) * a.hkv + g) * size_t(T) * D;
  const uint16_t* Kg = a.k + kvbase;
  const uint16_t* Vg = a.v + kvbase;

  typename V::T qv[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) qv[hh] = V::ld(a.q + (size_t(b) * a.hq + g * G + hh) * D + c * EPL);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -kInf;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }

  // slot = (local block k, key j); stream ks walks keys ks, ks + KS, ...
  for (int base = ks; base < nslots; base += KS * kDecUnroll) {
    typename V::T kv[kDecUnroll], vv[kDecUnroll];
    bool ok[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int sl = base + u * KS;
      ok[u] = false;
      kv[u] = V::zero();
      vv[u] = V::zero();
      if (sl < nslots) {
        const int kb = sl / B;
        int blk;
        if (kb < kDecUnroll) {
          blk = pre[0];
#pragma unroll
          for (int u2 = 1; u2 < kDecUnroll; ++u2) blk = (kb == u2) ? pre[u2] : blk;
        } else {
          blk = il[s + kb * a.nsplit];
        }
        const int pos = blk * B + sl % B;
        if (pos < T) {
          ok[u] = true;
          kv[u] = V::ld(Kg + size_t(pos) * D + c * EPL);
          vv[u] = V::ld(Vg + size_t(pos) * D + c * EPL);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      // slot base + u KS exists for every stream or for none (nslots is a
      // multiple of 16 = KS for blocks of 16 or more): skip empty slots whole
      if (base - ks + u * KS >= nslots) break;
      float vf[EPL];
#pragma unroll
      for (int k2 = 0; k2 < EPL / 2; ++k2) {
        const uint32_t w = V::w(vv[u], k2);
        vf[2 * k2] = bf16_lo(w);
        vf[2 * k2 + 1] = bf16_hi(w);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float dp = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < EPL / 2; ++k2) dp = dot2_bf16(V::w(kv[u], k2), V::w(qv[hh], k2), dp);
        dp = row16_sum(dp);
        if (!ok[u]) continue;
        const float x = dp * scale_log2;
        if (x > m[hh] + kDecRescale) {
          const float alpha = __builtin_amdgcn_exp2f(m[hh] - x);
          l[hh] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
          m[hh] = x;
        }
        const float p = __builtin_amdgcn_exp2f(x - m[hh]);
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(p, vf[e], acc[hh][e]);
      }
    }
  }

  // merge the KS slot streams
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (c == 0) {
      s_m[ks][hh] = m[hh];
      s_l[ks][hh] = l[hh];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[ks][hh][c * EPL + e] = acc[hh][e];
  }
  __syncthreads();
  float* part = a.partials + ((size_t(b) * a.hkv + g) * a.nsplit + s) * G * (D + 2);
  for (int o = tid; o < G * D; o += kDecThreads) {
    const int hh = o / D, dd = o % D;
    float M = -kInf;
    for (int q = 0; q < KS; ++q) M = fmaxf(M, s_m[q][hh]);
    float A = 0.f, Lsum = 0.f;
    if (M != -kInf) {
      for (int q = 0; q < KS; ++q) {
        const float f = __builtin_amdgcn_exp2f(s_m[q][hh] - M);
        A = fmaf(s_acc[q][hh][dd], f, A);
        Lsum = fmaf(s_l[q][hh], f, Lsum);
      }
    }
    float* ph = part + hh * (D + 2);
    ph[dd] = A;
    if (dd == 0) {
      ph[D] = M;
      ph[D + 1] = Lsum;
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;
  const int g = h / G, hh = h % G;
  const float* part = a.partials + ((size_t(b) * a.hkv + g) * a.nsplit) * G * (D + 2) + hh * (D + 2);
  const size_t stride = size_t(G) * (D + 2);
  const int ns = min(a.cnt[b], a.nsplit);
  float ms[kDecMaxSplits], ls[kDecMaxSplits], as[kDecMaxSplits];
#pragma unroll
  for (int s = 0; s < kDecMaxSplits; ++s) {
    const bool on = s < ns;
    const float* ps = part + (on ? s : 0) * stride;
    ms[s] = on ? ps[D] : -kInf;
    ls[s] = on ? ps[D + 1] : 0.f;
    as[s] = on ? ps[dd] : 0.f;
  }
  float M = -kInf;
#pragma unroll
  for (int s = 0; s < kDecMaxSplits; ++s) M = fmaxf(M, ms[s]);
  float A = 0.f, Lsum = 0.f;
  if (M != -kInf) {
#pragma unroll
    for (int s = 0; s < kDecMaxSplits; ++s) {
      const float f = __builtin_amdgcn_exp2f(ms[s] - M);   // 0 for empty splits
      A = fmaf(as[s], f, A);
      Lsum = fmaf(ls[s], f, Lsum);
    }
  }
  const float val = Lsum > 0.f ? A / Lsum : 0.f;
  a.o[(size_t(b) * a.hq + h) * D + dd] = uint16_t(pack_bf16x2(val, 0.f) & 0xFFFFu);
  if (a.lse && dd == 0) a.lse[size_t(b) * a.hq + h] = (Lsum > 0.f) ? (M + __log2f(Lsum)) * kLn2 : -kInf;
}

#ifndef SPOT_DECODE_TARGET_WGS
#define SPOT_DECODE_TARGET_WGS 1536   // split workgroups per step: 1280-1792 measured 7% faster than 2048 (tuning knob)
#endif

int decode_num_splits(int batch, int hkv, int nk) {
  const int pairs = batch * hkv;
  int ns = (SPOT_DECODE_TARGET_WGS + pairs - 1) / pairs;
  if (ns > kDecMaxSplits) ns = kDecMaxSplits;
  if (ns > nk) ns = nk;
  return ns < 1 ? 1 : ns;
}

size_t decode_partials_bytes(int batch, int hq, int d, int nsplit) {
  return size_t(batch) * hq * nsplit * (d + 2) * sizeof(float);
}

template <int D, int G>
static hipError_t launch_dg(const DecodeArgs& a, hipStream_t s, float scale_log2) {
  decode_split_kernel<D, G><<<dim3(a.nsplit, a.hkv, a.batch), kDecThreads, 0, s>>>(a, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<D, G><<<dim3(a.hq, a.batch), D, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, hipStream_t s, float scale_log2) {
  switch (a.hq / a.hkv) {
    case 1: return launch_dg<D, 1>(a, s, scale_log2);
    case 2: return launch_dg<D, 2>(a, s, scale_log2);
    case 4: return launch_dg<D, 4>(a, s, scale_log2);
    case 8: return launch_dg<D, 8>(a, s, scale_log2);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const float scale_log2 = a.sm_scale * kLog2e;
  if (a.d == 128) return launch_d<128>(a, s, scale_log2);
  if (a.d == 64) return launch_d<64>(a, s, scale_log2);
  return hipErrorInvalidValue;
}

}  // namespace spot
