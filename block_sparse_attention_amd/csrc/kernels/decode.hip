// Block-sparse decode attention for gfx950.
//
// One query per (sequence, head) at the last position attends the keys of the
// kept 16-token blocks.  The step is bound by reading the kept part of the KV
// cache (SpotAttention "Probleemstelling": every decode step re-reads a cache
// that grows with the context), so the kernel streams rows with 16-byte
// loads, the next round's loads issued before the current round is used, and
// keeps the arithmetic on the VALU (bf16 pair dot products, fp32
// accumulation).
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
// With the residual linear attention (SPLA section 2.2) the split kernel also
// sums (exp(q) . exp(k)) v over the kept keys it reads and takes its share of
// the rows of exp(q)^T S_cache (S_cache = sum over the cache of exp(k) v^T,
// built once per cache; the share's loads overlap those of the kept list);
// the combine adds every split's difference in order.
#include <mutex>

#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kDecThreads = 256;
#ifndef SPOT_DECODE_UNROLL
#define SPOT_DECODE_UNROLL 2      // key slots per stream and load round: 112 VGPRs (4: 150) (tuning knob)
#endif
constexpr int kDecUnroll = SPOT_DECODE_UNROLL;
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

// RLA: the same pass also accumulates the residual linear attention's kept-key
// term (SPLA section 2.2: the selected blocks' linear attention, computed on
// the kept tiles the attention already loads): per head, sum over the kept
// keys of (exp(q) . exp(k)) v, merged over the streams by a plain sum.
template <int D, int G, int NT, bool RLA>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeArgs a, float scale_log2) {
  constexpr int EPL = D / 16;           // elements per lane
  constexpr int KS = NT / 16;           // key-slot streams per workgroup
  constexpr int U = kDecUnroll;         // slots per stream and round
  using V = DVec<EPL>;
  __shared__ float s_m[KS][G], s_l[KS][G];
  __shared__ float s_acc[KS][G][D];
  __shared__ float s_racc[RLA ? KS : 1][G][RLA ? D : 1];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, c = tid & 15, ks = tid >> 4;
  const int B = a.block, T = a.T;
  const int lgB = 31 - __builtin_clz(B);
  const int32_t* il = a.idx + size_t(b) * a.nk;
  // block ids of this split's first round, loaded beside the count (stream ks, slot u of round 0 is
  // key (ks + KS u) mod B of local block (ks + KS u) / B, i.e. kept block s + nsplit (ks + KS u) / B)
  int ids[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bi = s + ((ks + KS * u) >> lgB) * a.nsplit;
    ids[u] = il[bi < a.nk ? bi : 0];
  }
  const size_t pair = size_t(b) * a.hkv + g;
  // residual: this split's rows k0 .. k1 of exp(q)^T S_cache for the outputs (head o / D, column o % D) it
  // writes; it needs neither the count nor the list, so its loads overlap theirs
  constexpr int ROUTS = RLA ? (G * D + NT - 1) / NT : 1;
  float share[ROUTS];
  if constexpr (RLA) {
    const int rows_per = (D + a.nsplit - 1) / a.nsplit;
    const int k0 = min(D, s * rows_per), k1 = min(D, k0 + rows_per);
#pragma unroll
    for (int u = 0; u < ROUTS; ++u) {
      const int o = tid + u * NT;
      share[u] = 0.f;
      if (o < G * D) {
        const uint16_t* qh = a.q + (size_t(b) * a.hq + g * G + o / D) * D;
        const float* S = a.rla_state + pair * D * D + o % D;
#pragma unroll 8
        for (int k = k0; k < k1; ++k) share[u] = fmaf(expf(bf16_to_f32(qh[k])), S[size_t(k) * D], share[u]);
      }
    }
  }
  const int n = a.cnt[b];
  if (s >= n) {   // no kept block of its own: the attention combine reads splits [0, min(n, nsplit)) only
    if constexpr (RLA) {
#pragma unroll
      for (int u = 0; u < ROUTS; ++u) {
        const int o = tid + u * NT;
        if (o < G * D) a.rla_partials[(pair * a.nsplit + s) * G * D + o] = share[u];
      }
    }
    return;
  }
  const int nmine = (n - s + a.nsplit - 1) / a.nsplit;   // blocks s, s + nsplit, ... below n

  {
    const int nslots = nmine * B;
    const int nj = ks < nslots ? (nslots - ks + KS - 1) / KS : 0;   // this stream's slots
    const int nrounds = ((nslots + KS - 1) / KS + U - 1) / U;
    const size_t kvbase = pair * size_t(T) * D;
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
    float fq[RLA ? G : 1][EPL], racc[RLA ? G : 1][EPL];   // exp(q) of the lane's dims; kept-key term
    if constexpr (RLA) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int k2 = 0; k2 < EPL / 2; ++k2) {
          const uint32_t w = V::w(qv[hh], k2);
          fq[hh][2 * k2] = expf(bf16_lo(w));
          fq[hh][2 * k2 + 1] = expf(bf16_hi(w));
          racc[hh][2 * k2] = racc[hh][2 * k2 + 1] = 0.f;
        }
    }

    // slot j of stream ks is slot ks + KS j of the split: key (ks + KS j) mod B of local block (ks + KS j) / B
    auto block_ids = [&](int r, int (&out)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sl = ks + KS * (r * U + u);
        out[u] = sl < nslots ? il[s + (sl >> lgB) * a.nsplit] : 0;
      }
    };
    auto issue = [&](int r, const int (&bid)[U], typename V::T (&kv)[U], typename V::T (&vv)[U], bool (&ok)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sl = ks + KS * (r * U + u);
        const int pos = (bid[u] << lgB) + (sl & (B - 1));
        ok[u] = sl < nslots && pos < T;
        kv[u] = ok[u] ? V::ld(Kg + size_t(pos) * D + c * EPL) : V::zero();
        vv[u] = ok[u] ? V::ld(Vg + size_t(pos) * D + c * EPL) : V::zero();
      }
    };
    auto consume = [&](int r, const typename V::T (&kv)[U], const typename V::T (&vv)[U], const bool (&ok)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // the 16 lanes of a stream agree on whether its slot exists: skip empty slots whole
        if (r * U + u >= nj) break;
        float vf[EPL];
#pragma unroll
        for (int k2 = 0; k2 < EPL / 2; ++k2) {
          const uint32_t w = V::w(vv[u], k2);
          vf[2 * k2] = bf16_lo(w);
          vf[2 * k2 + 1] = bf16_hi(w);
        }
        if constexpr (RLA) {
          float fk[EPL];
#pragma unroll
          for (int k2 = 0; k2 < EPL / 2; ++k2) {
            const uint32_t w = V::w(kv[u], k2);
            fk[2 * k2] = expf(bf16_lo(w));
            fk[2 * k2 + 1] = expf(bf16_hi(w));
          }
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            float wd = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) wd = fmaf(fq[hh][e], fk[e], wd);
            wd = row16_sum(wd);
            if (ok[u]) {
#pragma unroll
              for (int e = 0; e < EPL; ++e) racc[hh][e] = fmaf(wd, vf[e], racc[hh][e]);
            }
          }
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
    };

    // two register sets alternate: round r + 1's loads are in flight while round r is consumed, and round
    // r + 2's block ids while round r + 1's loads are issued
    typename V::T ka[U], va[U], kb2[U], vb[U];
    bool oka[U], okb[U];
    issue(0, ids, ka, va, oka);
    block_ids(1, ids);
    int r = 0;
    for (; r + 1 < nrounds; r += 2) {
      issue(r + 1, ids, kb2, vb, okb);
      block_ids(r + 2, ids);
      consume(r, ka, va, oka);
      if (r + 2 < nrounds) {
        issue(r + 2, ids, ka, va, oka);
        block_ids(r + 3, ids);
      }
      consume(r + 1, kb2, vb, okb);
    }
    if (r < nrounds) consume(r, ka, va, oka);

    // merge the KS slot streams through LDS
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (c == 0) {
        s_m[ks][hh] = m[hh];
        s_l[ks][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[ks][hh][c * EPL + e] = acc[hh][e];
      if constexpr (RLA) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_racc[ks][hh][c * EPL + e] = racc[hh][e];
      }
    }
    __syncthreads();
    float* part = a.partials + (pair * a.nsplit + s) * G * (D + 2);
    for (int o = tid; o < G * D; o += NT) {
      const int hh = o / D, dd = o % D;
      float M = -kInf;
#pragma unroll
      for (int q = 0; q < KS; ++q) M = fmaxf(M, s_m[q][hh]);
      float A = 0.f, Lsum = 0.f;
      if (M != -kInf) {
#pragma unroll
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
      if constexpr (RLA) {   // its share of the state term minus the kept keys' term of its streams
        float R = 0.f;
#pragma unroll
        for (int q = 0; q < KS; ++q) R += s_racc[q][hh][dd];
        a.rla_partials[(pair * a.nsplit + s) * G * D + o] = share[(o - tid) / NT] - R;
      }
    }
  }
}

template <int D, int G, bool RLA>
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
  if constexpr (RLA) {
    // every split's partial (its share of exp(q)^T S_cache minus its kept keys' term), in split order
    const float* rp = a.rla_partials + ((size_t(b) * a.hkv + g) * a.nsplit) * G * D + hh * D + dd;
    float rs[kDecMaxSplits];
#pragma unroll
    for (int s2 = 0; s2 < kDecMaxSplits; ++s2) rs[s2] = s2 < a.nsplit ? rp[size_t(s2) * G * D] : 0.f;
    float r = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kDecMaxSplits; ++s2) r += rs[s2];
    a.o_rla[(size_t(b) * a.hq + h) * D + dd] = r;
  }
}

#ifndef SPOT_DECODE_TARGET_WGS
#define SPOT_DECODE_TARGET_WGS 1024   // split workgroups per step: 512-1536 measured, 1024 best overall (tuning knob)
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

// Device-resident scratch of the allocation-free decode entry point: the
// split partials of one call.  Each GPU the library runs on holds its own
// copy until the process ends; every call on a GPU uses that GPU's copy, so
// calls that overlap on one GPU race.  Nothing in it must start at zero: the
// combine reads only the partials the same call's split workgroups wrote.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the array's name is a host-side stand-in: its device address on this GPU comes from the runtime
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

template <int D, int G>
static hipError_t launch_dg(const DecodeArgs& a, hipStream_t s, float scale_log2) {
  const dim3 grid(a.nsplit, a.hkv, a.batch);
  if (a.o_rla) decode_split_kernel<D, G, kDecThreads, true><<<grid, kDecThreads, 0, s>>>(a, scale_log2);
  else decode_split_kernel<D, G, kDecThreads, false><<<grid, kDecThreads, 0, s>>>(a, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.o_rla) decode_combine_kernel<D, G, true><<<dim3(a.hq, a.batch), D, 0, s>>>(a);
  else decode_combine_kernel<D, G, false><<<dim3(a.hq, a.batch), D, 0, s>>>(a);
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
