// Block-sparse decode attention for gfx950.
//
// One query per (sequence, head) at the last position attends the keys of the
// kept 16-token blocks.  The step re-reads the kept part of the KV cache
// (SpotAttention "Probleemstelling": every decode step re-reads a cache that
// grows with the context); with a few dozen kept blocks per sequence it is
// bound by latency rather than bandwidth, so the work is spread evenly over
// workgroups that are all resident at once, and each wave issues every load
// it needs in as few dependent rounds as possible.
//
// decode_split_kernel: the kept list of each (sequence b, KV head g) is cut
//   into units of kDecUnitBlocks consecutive blocks (more when the list is
//   long, so that a pair never has more than kDecMaxUnits units), and the
//   units of all pairs are numbered in (b, g, unit) order.  Every workgroup
//   derives that numbering from the kept counts and takes units blockIdx.x,
//   blockIdx.x + gridDim.x, ...  Its four waves take the unit's blocks in
//   turn (wave w: blocks w, w + 4, ...).  A wave is four rows of 16 lanes:
//   row r takes key slots r, r + 4, ... and lane c of a row holds dims
//   c*D/16 .. +D/16 of a key, keeping its own online-softmax state for the G
//   query heads of the group.  Rows merge through lane swaps, waves through
//   LDS, and the workgroup writes one partial (acc, m, l) per head and unit.
// decode_combine_kernel: merges the partials of a pair's units in unit order
//   (deterministic) and writes O (bf16) and the natural-log LSE.
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kDecRows = 4;            // key streams (rows of 16 lanes) per wave
constexpr int kDecWaves = 4;           // waves per workgroup
constexpr float kDecRescale = 8.0f;
constexpr int kDecUnitBlocks = 2 * kDecWaves;   // kept blocks per unit while the list is short: two per wave
constexpr int kDecMaxUnits = 32;       // units (partials) per (sequence, KV head)
constexpr int kDecCombineChunk = 16;
#ifndef SPOT_DECODE_KEYS_PER_ROW
#define SPOT_DECODE_KEYS_PER_ROW 8     // key slots per row loaded in one round: two 16-key blocks (tuning knob)
#endif
constexpr int kDecKpr = SPOT_DECODE_KEYS_PER_ROW;
#ifndef SPOT_DECODE_MAX_WGS
#define SPOT_DECODE_MAX_WGS 768        // split workgroups launched: what the GPU holds at once at G = 4 (tuning knob)
#endif

// Units of a kept list of n blocks, and the blocks per unit.
__device__ __forceinline__ int dec_units(int n) { return min(kDecMaxUnits, (n + kDecUnitBlocks - 1) / kDecUnitBlocks); }
__device__ __forceinline__ int dec_unit_blocks(int n, int units) { return units > 0 ? (n + units - 1) / units : 0; }

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

// Value of lane ^ 16 / lane ^ 32 through the gfx950 lane swaps (VALU, no LDS).
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// Merge the online-softmax state of this lane with that of lane ^ X (X = 16 or 32).
template <int G, int EPL, int X>
__device__ __forceinline__ void merge_rows(float (&m)[G], float (&l)[G], float (&acc)[G][EPL]) {
  auto other = [](float x) { return X == 16 ? lane_xor16(x) : lane_xor32(x); };
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float mo = other(m[hh]), lo = other(l[hh]);
    const float M = fmaxf(m[hh], mo);
    const float fs = M == -kInf ? 0.f : __builtin_amdgcn_exp2f(m[hh] - M);
    const float fo = M == -kInf ? 0.f : __builtin_amdgcn_exp2f(mo - M);
    l[hh] = l[hh] * fs + lo * fo;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = acc[hh][e] * fs + other(acc[hh][e]) * fo;
    m[hh] = M;
  }
}

// Partials: acc [batch, hkv, kDecMaxUnits, G, D] fp32, then (m, l) [batch, hkv, kDecMaxUnits, G, 2] fp32.
__device__ __forceinline__ float* part_ml(const DecodeArgs& a, int G) {
  return a.partials + size_t(a.batch) * a.hkv * kDecMaxUnits * G * a.d;
}

// Unit x of the (b, g, unit) numbering -> b, g, unit; false past the last unit.
// Wave-level: lanes hold 64 sequences at a time, an inclusive scan of their
// unit counts (times hkv) locates x.
__device__ bool dec_find_unit(const DecodeArgs& a, int x, int& b, int& g, int& u, int& n) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int bb = b0 + lane;
    const int nb = bb < a.batch ? a.cnt[bb] : 0;
    const int units = bb < a.batch ? dec_units(nb) * a.hkv : 0;
    int incl = units;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const unsigned long long hit = __ballot(before + incl > x);
    if (hit) {
      const int l0 = __ffsll((long long)hit) - 1;
      b = b0 + l0;
      n = __shfl(nb, l0);
      const int first = before + __shfl(incl - units, l0);
      const int per_pair = dec_units(n);
      const int r = x - first;
      g = r / per_pair;
      u = r - g * per_pair;
      return true;
    }
    before += __shfl(incl, 63);
  }
  return false;
}

template <int D, int G>
__global__ __launch_bounds__(64 * kDecWaves) void decode_split_kernel(DecodeArgs a, float scale_log2) {
  constexpr int EPL = D / 16;   // elements per lane
  using V = DVec<EPL>;
  __shared__ float s_acc[kDecWaves][G][D];
  __shared__ float s_ml[kDecWaves][G][2];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c = lane & 15, row = lane >> 4;
  const int B = a.block, T = a.T;

  for (int x = blockIdx.x;; x += gridDim.x) {
    int b, g, u, n;
    if (!dec_find_unit(a, x, b, g, u, n)) return;   // the same answer in every wave
    const int pair = b * a.hkv + g;
    const int upp = dec_units(n), bpu = dec_unit_blocks(n, upp);
    const int p0 = u * bpu, p1 = min(n, p0 + bpu);           // kept-list positions of this unit
    const int nmine = p1 - p0 > w ? (p1 - p0 - w + kDecWaves - 1) / kDecWaves : 0;   // positions p0 + w + 4k
    const int nslots = nmine * B;
    const int32_t* il = a.idx + size_t(b) * a.nk;
    const int pre0 = il[min(p0 + w, a.nk - 1)];
    const int pre1 = il[min(p0 + w + kDecWaves, a.nk - 1)];
    const size_t kvbase = size_t(pair) * size_t(T) * D;
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

    for (int base = 0; base < nslots; base += kDecRows * kDecKpr) {
      typename V::T kv[kDecKpr], vv[kDecKpr];
      bool ok[kDecKpr];
#pragma unroll
      for (int k = 0; k < kDecKpr; ++k) {
        const int sl = base + row + kDecRows * k;   // slot = (local block kb, key sl - kb*B)
        ok[k] = false;
        kv[k] = V::zero();
        vv[k] = V::zero();
        if (sl < nslots) {
          const int kb = sl / B;
          const int blk = kb == 0 ? pre0 : kb == 1 ? pre1 : il[p0 + w + kDecWaves * kb];
          const int pos = blk * B + (sl - kb * B);
          if (pos < T) {
            ok[k] = true;
            kv[k] = V::ld(Kg + size_t(pos) * D + c * EPL);
            vv[k] = V::ld(Vg + size_t(pos) * D + c * EPL);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kDecKpr; ++k) {
        if (base + kDecRows * k >= nslots) break;   // no row has slot k (wave-uniform)
        float vf[EPL];
#pragma unroll
        for (int k2 = 0; k2 < EPL / 2; ++k2) {
          const uint32_t wv = V::w(vv[k], k2);
          vf[2 * k2] = bf16_lo(wv);
          vf[2 * k2 + 1] = bf16_hi(wv);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float dp = 0.f;
#pragma unroll
          for (int k2 = 0; k2 < EPL / 2; ++k2) dp = dot2_bf16(V::w(kv[k], k2), V::w(qv[hh], k2), dp);
          dp = row16_sum(dp);
          const float xs = dp * scale_log2;
          const bool up = ok[k] && xs > m[hh] + kDecRescale;
          if (__ballot(up)) {   // wave-uniform: rare after a row's first key
            const float alpha = up ? __builtin_amdgcn_exp2f(m[hh] - xs) : 1.f;
            l[hh] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
            m[hh] = up ? xs : m[hh];
          }
          const float p = ok[k] ? __builtin_amdgcn_exp2f(xs - m[hh]) : 0.f;
          l[hh] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(p, vf[e], acc[hh][e]);
        }
      }
    }

    merge_rows<G, EPL, 16>(m, l, acc);
    merge_rows<G, EPL, 32>(m, l, acc);
    if (row == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<float4*>(&s_acc[w][hh][c * EPL + e]) =
              make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
        if (c == 0) {
          s_ml[w][hh][0] = m[hh];
          s_ml[w][hh][1] = l[hh];
        }
      }
    }
    __syncthreads();
    float* pa = a.partials + (size_t(pair) * kDecMaxUnits + u) * G * D;
    float* pm = part_ml(a, G) + (size_t(pair) * kDecMaxUnits + u) * G * 2;
    for (int o = tid; o < G * D; o += 64 * kDecWaves) {
      const int hh = o / D, dd = o - hh * D;
      float M = -kInf;
#pragma unroll
      for (int q = 0; q < kDecWaves; ++q) M = fmaxf(M, s_ml[q][hh][0]);
      float A = 0.f, L = 0.f;
      if (M != -kInf) {
#pragma unroll
        for (int q = 0; q < kDecWaves; ++q) {
          const float f = __builtin_amdgcn_exp2f(s_ml[q][hh][0] - M);
          A = fmaf(s_acc[q][hh][dd], f, A);
          L = fmaf(s_ml[q][hh][1], f, L);
        }
      }
      pa[o] = A;
      if (dd == 0) *reinterpret_cast<float2*>(pm + hh * 2) = make_float2(M, L);
    }
    __syncthreads();   // s_acc is rewritten by the next unit
  }
}

// Merge the ns unit partials of (pair, head hh) for output dim dd, in unit order; writes O and the LSE.
template <int D, int G>
__device__ void dec_combine_one(const DecodeArgs& a, int b, int g, int hh, int dd, int ns) {
  const int h = g * G + hh;
  const size_t pair = size_t(b) * a.hkv + g;
  const float* pa = a.partials + (pair * kDecMaxUnits * G + hh) * D + dd;   // unit s at + s*G*D
  const float* pm = part_ml(a, G) + (pair * kDecMaxUnits * G + hh) * 2;     // unit s at + s*G*2
  float M = -kInf, A = 0.f, Lsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kDecCombineChunk) {
    float ms[kDecCombineChunk], ls[kDecCombineChunk], as[kDecCombineChunk];
#pragma unroll
    for (int k = 0; k < kDecCombineChunk; ++k) {
      const int sp = s0 + k;
      const bool on = sp < ns;
      const size_t so = on ? size_t(sp) : 0;
      const float2 ml = *reinterpret_cast<const float2*>(pm + so * G * 2);
      ms[k] = on ? ml.x : -kInf;
      ls[k] = on ? ml.y : 0.f;
      as[k] = on ? pa[so * G * D] : 0.f;
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < kDecCombineChunk; ++k) Mc = fmaxf(Mc, ms[k]);
    if (Mc == -kInf) continue;
    const float f = __builtin_amdgcn_exp2f(M - Mc);   // 0 while nothing has been merged
    A *= f;
    Lsum *= f;
#pragma unroll
    for (int k = 0; k < kDecCombineChunk; ++k) {
      const float fk = __builtin_amdgcn_exp2f(ms[k] - Mc);   // 0 for empty units
      A = fmaf(as[k], fk, A);
      Lsum = fmaf(ls[k], fk, Lsum);
    }
    M = Mc;
  }
  const float val = Lsum > 0.f ? A / Lsum : 0.f;
  a.o[(size_t(b) * a.hq + h) * D + dd] = uint16_t(pack_bf16x2(val, 0.f) & 0xFFFFu);
  if (a.lse && dd == 0) a.lse[size_t(b) * a.hq + h] = (Lsum > 0.f) ? (M + __log2f(Lsum)) * kLn2 : -kInf;
}

template <int D, int G>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  dec_combine_one<D, G>(a, b, h / G, h % G, threadIdx.x, dec_units(a.cnt[b]));
}

int decode_num_splits(int, int, int) { return kDecMaxUnits; }

size_t decode_partials_bytes(int batch, int hq, int d, int nsplit) {
  return size_t(batch) * hq * nsplit * (d + 2) * sizeof(float);
}

template <int D, int G>
static hipError_t launch_dg(const DecodeArgs& a, hipStream_t s, float scale_log2) {
  const long long most = (long long)a.batch * a.hkv * kDecMaxUnits;   // units can never exceed this
  const unsigned grid = unsigned(most < SPOT_DECODE_MAX_WGS ? most : SPOT_DECODE_MAX_WGS);
  decode_split_kernel<D, G><<<grid, 64 * kDecWaves, 0, s>>>(a, scale_log2);
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
