// Residual linear attention for gfx950 (SPLA section 2.2, with the
// parameter-free exponential feature map of section 2.3).
//
// What is computed: for a query row, the linear attention with phi(x) =
// exp(x) elementwise and no normaliser over the visible keys that the row's
// kept blocks do not hold, o = sum_t (phi(q) . phi(k_t)) v_t.  Linear
// attention is a sum of per-key outer products, so it goes through states:
// the state of a set of keys is S = sum_t phi(k_t) v_t^T (d x d, fp32), and a
// row's output is phi(q)^T S over the set it needs.
//
// rla_states_kernel   the state of every range of `span` consecutive key
//                     positions (the key blocks in prefill, natural or
//                     through the permutation; chunks of the cache in decode)
// rla_reduce_kernel   the ordered sum of a (batch, KV head)'s chunk states:
//                     the state of the whole cache
// rla_prefill_kernel  per (batch, KV head, query block i): R = the sum of the
//                     states of the earlier blocks the row list does not keep
//                     (blocks of earlier segments through the permutation),
//                     then phi(q)^T R for the G*B rows of the block.  Block i
//                     itself is always kept (recency), so no partial block
//                     enters, and the set is the same for every row of i.
// rla_decode_split_kernel + rla_decode_combine_kernel
//                     per (batch, KV head): phi(q)^T S_cache minus the linear
//                     attention over the kept keys read from the cache (the
//                     page's difference of the all-blocks and kept-blocks
//                     estimates: only the kept blocks are read), the kept
//                     keys split over several workgroups.
// Every sum runs in a fixed order in fp32, so results are deterministic.
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kRlaStage = 32;   // keys staged in LDS per round
#ifndef SPOT_RLA_MFMA
#define SPOT_RLA_MFMA 1   // prefill residual output phi(Q) R on fp32 MFMA (0: fp32 VALU)
#endif

// eight consecutive elements as floats (16 bytes of bf16 or 32 of fp32)
__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
  o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z); o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// ---------------------------------------------------------------- range states
// One workgroup per (range, pair); thread t owns the TR x TR tile of S at
// rows (t / 16) * TR, columns (t % 16) * TR.  Keys are staged kRlaStage at a
// time as fp32 phi(k) and v rows (padded by 4 floats) and accumulated in
// position order.
template <typename T, int D>
__global__ __launch_bounds__(256) void rla_states_kernel(RlaStateArgs a) {
  constexpr int TR = D / 16;
  constexpr int LD = D + 4;
  constexpr int PIECES = kRlaStage * D / 8;   // 8-element pieces per staged tensor
  static_assert(PIECES % 256 == 0 || 256 % PIECES == 0, "pieces spread evenly");
  __shared__ __attribute__((aligned(16))) float fk[kRlaStage * LD];
  __shared__ __attribute__((aligned(16))) float fv[kRlaStage * LD];
  const int tid = threadIdx.x;
  const int range = blockIdx.x, pair = blockIdx.y;
  const int r0 = (tid / 16) * TR, c0 = (tid % 16) * TR;
  const T* K = static_cast<const T*>(a.k) + size_t(pair) * a.L * D;
  const T* V = static_cast<const T*>(a.v) + size_t(pair) * a.L * D;
  const int32_t* pm = a.perm ? a.perm + size_t(pair) * a.L : nullptr;
  const int t_begin = range * a.span, t_end = min(t_begin + a.span, a.L);
  float acc[TR][TR];
#pragma unroll
  for (int x = 0; x < TR; ++x)
#pragma unroll
    for (int y = 0; y < TR; ++y) acc[x][y] = 0.f;
  for (int t0 = t_begin; t0 < t_end; t0 += kRlaStage) {
    for (int pc = tid; pc < PIECES; pc += 256) {
      const int row = pc / (D / 8), col = (pc % (D / 8)) * 8;
      const int t = t0 + row;
      float kx[8], vx[8];
      if (t < t_end) {
        const int phys = pm ? min(max(pm[t], 0), a.L - 1) : t;   // an invalid permutation gives wrong sums, never a stray read
        load8(K + size_t(phys) * D + col, kx);
        load8(V + size_t(phys) * D + col, vx);
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = expf(kx[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = vx[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        *reinterpret_cast<float4*>(fk + row * LD + col + e) = make_float4(kx[e], kx[e + 1], kx[e + 2], kx[e + 3]);
        *reinterpret_cast<float4*>(fv + row * LD + col + e) = make_float4(vx[e], vx[e + 1], vx[e + 2], vx[e + 3]);
      }
    }
    __syncthreads();
    const int n = min(kRlaStage, t_end - t0);
    for (int r = 0; r < n; ++r) {
      float av[TR], bv[TR];
#pragma unroll
      for (int x = 0; x < TR; x += 4) {
        const float4 p = *reinterpret_cast<const float4*>(fk + r * LD + r0 + x);
        const float4 q = *reinterpret_cast<const float4*>(fv + r * LD + c0 + x);
        av[x] = p.x; av[x + 1] = p.y; av[x + 2] = p.z; av[x + 3] = p.w;
        bv[x] = q.x; bv[x + 1] = q.y; bv[x + 2] = q.z; bv[x + 3] = q.w;
      }
#pragma unroll
      for (int x = 0; x < TR; ++x)
#pragma unroll
        for (int y = 0; y < TR; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
    }
    __syncthreads();
  }
  float* out = a.states + (size_t(pair) * a.nranges + range) * D * D;
#pragma unroll
  for (int x = 0; x < TR; ++x)
#pragma unroll
    for (int y = 0; y < TR; y += 4)
      *reinterpret_cast<float4*>(out + (r0 + x) * D + c0 + y) =
          make_float4(acc[x][y], acc[x][y + 1], acc[x][y + 2], acc[x][y + 3]);
}

// ---------------------------------------------------------------- ordered sum of chunk states
__global__ __launch_bounds__(256) void rla_reduce_kernel(const float* __restrict__ chunks, float* __restrict__ out,
                                                         int nranges, int dd) {
  const int pair = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= dd) return;
  const float* p = chunks + size_t(pair) * nranges * dd + e;
  float s = 0.f;
  for (int j = 0; j < nranges; ++j) s += p[size_t(j) * dd];
  out[size_t(pair) * dd + e] = s;
}

// ---------------------------------------------------------------- prefill
// LDS: one region that first holds the kept list and the list of blocks to
// sum, then R (d x d); plus kRlaQRows staged phi(q) rows.
constexpr int kRlaQRows = 16;
template <int D>
constexpr int rla_region_floats() {
  return D * D > 2 * kRlaMaxBlocks ? D * D : 2 * kRlaMaxBlocks;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rla_prefill_kernel(RlaPrefillArgs a) {
  constexpr int PER = D * D / 1024;   // float4 of R per thread
  constexpr int NS = 256 / D;         // row streams (threads per output column)
  __shared__ __attribute__((aligned(16))) float region[rla_region_floats<D>()];
  __shared__ __attribute__((aligned(16))) float fq[kRlaQRows * D];
  __shared__ int s_wave[4];
  int* s_list = reinterpret_cast<int*>(region);
  int* s_rest = s_list + kRlaMaxBlocks;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int pair = blockIdx.x / a.nb, i = blockIdx.x % a.nb;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int G = a.hq / a.hkv, B = a.block, L = a.L;
  const size_t row_id = size_t(pair) * a.nb + i;
  const int n = min(max(a.cnt[row_id], 0), a.nb);
  for (int k = tid; k < n; k += 256) s_list[k] = a.idx[row_id * a.nb + k];
  __syncthreads();

  // the earlier blocks not in the (ascending) kept list, compacted in order
  int nrest = 0;
  for (int base = 0; base < i; base += 256) {
    const int j = base + tid;
    bool rest = false;
    if (j < i) {
      int lo = 0, hi = n;   // first list entry >= j
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_list[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      rest = !(lo < n && s_list[lo] == j);
    }
    const unsigned long long m = __ballot(rest);
    if (lane == 0) s_wave[wv] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wv ? s_wave[w] : 0;
      total += s_wave[w];
    }
    if (rest) s_rest[nrest + before + __popcll(m & ((1ull << lane) - 1ull))] = j;
    nrest += total;
    __syncthreads();
  }

  // R = sum of their states (history blocks through the permutation), two blocks' loads in flight
  // blocks j < hist_end lie in segments before block i's (none without the permuted states)
  const int hist_end = (a.states_perm != nullptr && a.segment > 0) ? ((i * B) / a.segment) * (a.segment / B) : 0;
  const float* nat = a.states + size_t(pair) * a.nb * D * D;
  const float* prm = (a.states_perm != nullptr ? a.states_perm : a.states) + size_t(pair) * a.nb * D * D;
  auto state_of = [&](int j) { return (j < hist_end ? prm : nat) + size_t(j) * D * D; };
  f32x4_t acc[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int r = 0;
  for (; r + 1 < nrest; r += 2) {
    const float* s0 = state_of(s_rest[r]);
    const float* s1 = state_of(s_rest[r + 1]);
    f32x4_t x0[PER], x1[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      x0[m] = *reinterpret_cast<const f32x4_t*>(s0 + (tid + m * 256) * 4);
      x1[m] = *reinterpret_cast<const f32x4_t*>(s1 + (tid + m * 256) * 4);
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) acc[m] = (acc[m] + x0[m]) + x1[m];
  }
  if (r < nrest) {
    const float* s0 = state_of(s_rest[r]);
#pragma unroll
    for (int m = 0; m < PER; ++m) acc[m] += *reinterpret_cast<const f32x4_t*>(s0 + (tid + m * 256) * 4);
  }
  __syncthreads();   // the lists are read; the region becomes R
  float* Rs = region;
#pragma unroll
  for (int m = 0; m < PER; ++m) *reinterpret_cast<f32x4_t*>(Rs + (tid + m * 256) * 4) = acc[m];
  __syncthreads();

#if SPOT_RLA_MFMA
  // o = phi(Q) R on v_mfma_f32_32x32x2_f32, k two at a time: a wave takes tiles of 32 packed rows and all
  // D columns; lane l holds phi(q) of row l % 32 at the k of parity l / 32 (A operand), reads
  // R[2j + l / 32][32 ct + l % 32] from LDS (B operand) and keeps D / 32 accumulator tiles, whose
  // element e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4, column 32 ct + l % 32.
  {
    const int rl = lane & 31, kh = lane >> 5;
    const int GB = G * B;
    const T* Q = static_cast<const T*>(a.q);
    for (int tr = wv; tr * 32 < GB; tr += 4) {
      float fa[D / 2];
      {
        const int pr = tr * 32 + rl;
        const int h = g * G + pr / B, rr = i * B + pr % B;
        const bool valid = pr < GB && rr < L;
        const T* qrow = Q + ((size_t(b) * a.hq + (valid ? h : 0)) * L + (valid ? rr : 0)) * D;
#pragma unroll
        for (int pc = 0; pc < D / 8; ++pc) {
          float x[8];
          load8(qrow + pc * 8, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) fa[pc * 4 + e] = valid ? expf(x[2 * e + kh]) : 0.f;
        }
      }
      constexpr int CT = 2;   // column tiles per pass (accumulator registers: 16 per tile)
#pragma unroll
      for (int c0 = 0; c0 < D / 32; c0 += CT) {
        f32x16_t acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16_t{};
#pragma unroll 4
        for (int j = 0; j < D / 2; ++j)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[j], Rs[(2 * j + kh) * D + (c0 + ct) * 32 + rl],
                                                           acc[ct], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int pr = tr * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
          const int h = g * G + pr / B, rr = i * B + pr % B;
          if (pr < GB && rr < L) {
            float* orow = a.o + ((size_t(b) * a.hq + h) * L + rr) * D;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) orow[(c0 + ct) * 32 + rl] = acc[ct][e];
          }
        }
      }
    }
  }
#else
  // o[p, c] = sum_k phi(q_p)[k] * R[k][c]: thread owns column c, rows p = s, s + NS, ...
  const int c = tid % D, s = tid / D;
  float rc[D];
#pragma unroll
  for (int k = 0; k < D; ++k) rc[k] = Rs[k * D + c];
  const int GB = G * B;
  const T* Q = static_cast<const T*>(a.q);
  for (int p0 = 0; p0 < GB; p0 += kRlaQRows) {
    for (int pc = tid; pc < kRlaQRows * D / 8; pc += 256) {
      const int row = pc / (D / 8), col = (pc % (D / 8)) * 8;
      const int pr = p0 + row;
      const int h = g * G + pr / B, rr = i * B + pr % B;
      float x[8];
      if (pr < GB && rr < L) {
        load8(Q + ((size_t(b) * a.hq + h) * L + rr) * D + col, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = expf(x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      *reinterpret_cast<float4*>(fq + row * D + col) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(fq + row * D + col + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
    __syncthreads();
    for (int pp = s; pp < kRlaQRows; pp += NS) {
      const int pr = p0 + pp;
      const int h = g * G + pr / B, rr = i * B + pr % B;
      float o = 0.f;
#pragma unroll
      for (int k = 0; k < D; k += 4) {
        const float4 f = *reinterpret_cast<const float4*>(fq + pp * D + k);
        o = fmaf(f.x, rc[k], o);
        o = fmaf(f.y, rc[k + 1], o);
        o = fmaf(f.z, rc[k + 2], o);
        o = fmaf(f.w, rc[k + 3], o);
      }
      if (pr < GB && rr < L) a.o[((size_t(b) * a.hq + h) * L + rr) * D + c] = o;
    }
    __syncthreads();
  }
#endif
}

// ---------------------------------------------------------------- decode
// rla_decode_split_kernel: workgroup (split, pair) takes its share of the
// rows of S_cache for phi(q)^T S_cache and the kept key slots in chunks of
// kRlaStage (chunk c = split, split + nsplit, ...; the next chunk's rows are
// loaded while the current one is used), and writes its share of the state
// term minus its partial linear attention over those keys (G x D floats).
// rla_decode_combine_kernel: per pair, the sum of the partials in split order.
template <int D, int G>
__global__ __launch_bounds__(256) void rla_decode_split_kernel(RlaDecodeArgs a) {
  constexpr int LD = D + 4;
  constexpr int OUTS = (G * D + 255) / 256;   // outputs (head, column) per thread
  constexpr int PIECES = kRlaStage * D / 8;   // 16-byte pieces of a staged chunk, per tensor
  constexpr int PPT = (PIECES + 255) / 256;
  static_assert(G * kRlaStage <= 256, "one key-head dot product per thread");
  __shared__ __attribute__((aligned(16))) float fq[G * D];
  __shared__ __attribute__((aligned(16))) float fk[kRlaStage * LD];
  __shared__ __attribute__((aligned(16))) float fv[kRlaStage * LD];
  __shared__ float w[G * kRlaStage];
  const int tid = threadIdx.x;
  const int split = blockIdx.x, pair = blockIdx.y;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int B = a.block, T = a.T;
  for (int e = tid; e < G * D; e += 256)
    fq[e] = expf(bf16_to_f32(a.q[(size_t(b) * a.hq + g * G + e / D) * D + e % D]));
  __syncthreads();

  // this split's share of phi(q)^T S_cache: rows k0 .. k1 of the state
  const int c_col = tid % D;
  float part_o[OUTS];
#pragma unroll
  for (int u = 0; u < OUTS; ++u) part_o[u] = 0.f;
  {
    const int rows_per = (D + a.nsplit - 1) / a.nsplit;
    const int k0 = min(D, split * rows_per), k1 = min(D, k0 + rows_per);
    const float* S = a.state + size_t(pair) * D * D;
    for (int k = k0; k < k1; ++k) {
      const float sk = S[k * D + c_col];
#pragma unroll
      for (int u = 0; u < OUTS; ++u) {
        const int o = tid + u * 256;
        if (o < G * D) part_o[u] = fmaf(fq[(o / D) * D + k], sk, part_o[u]);
      }
    }
  }

  const int nkept = min(max(a.cnt[b], 0), a.nk);
  const int32_t* list = a.idx + size_t(b) * a.nk;
  const uint16_t* K = a.k + size_t(pair) * T * D;
  const uint16_t* V = a.v + size_t(pair) * T * D;
  const int nslots = nkept * B;
  const int nchunks = (nslots + kRlaStage - 1) / kRlaStage;
  uint4 kr[PPT], vr[PPT];
  bool ok[PPT];
  auto fetch = [&](int c) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int pc = tid + p * 256;
      const int row = pc / (D / 8), col = (pc % (D / 8)) * 8;
      const int sl = c * kRlaStage + row;
      const long long pos = (pc < PIECES && sl < nslots) ? (long long)list[sl / B] * B + sl % B : -1;
      ok[p] = pos >= 0 && pos < T;   // list entries outside the cache add nothing
      kr[p] = ok[p] ? *reinterpret_cast<const uint4*>(K + size_t(pos) * D + col) : make_uint4(0u, 0u, 0u, 0u);
      vr[p] = ok[p] ? *reinterpret_cast<const uint4*>(V + size_t(pos) * D + col) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  float otil[OUTS];
#pragma unroll
  for (int u = 0; u < OUTS; ++u) otil[u] = 0.f;
  if (split < nchunks) fetch(split);
  for (int c = split; c < nchunks; c += a.nsplit) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int pc = tid + p * 256;
      if (pc < PIECES) {
        const int row = pc / (D / 8), col = (pc % (D / 8)) * 8;
        const uint32_t kw[4] = {kr[p].x, kr[p].y, kr[p].z, kr[p].w};
        const uint32_t vw[4] = {vr[p].x, vr[p].y, vr[p].z, vr[p].w};
        float kx[8], vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[2 * e] = ok[p] ? expf(bf16_lo(kw[e])) : 0.f;
          kx[2 * e + 1] = ok[p] ? expf(bf16_hi(kw[e])) : 0.f;
          vx[2 * e] = bf16_lo(vw[e]);
          vx[2 * e + 1] = bf16_hi(vw[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          *reinterpret_cast<float4*>(fk + row * LD + col + e) = make_float4(kx[e], kx[e + 1], kx[e + 2], kx[e + 3]);
          *reinterpret_cast<float4*>(fv + row * LD + col + e) = make_float4(vx[e], vx[e + 1], vx[e + 2], vx[e + 3]);
        }
      }
    }
    __syncthreads();
    if (c + a.nsplit < nchunks) fetch(c + a.nsplit);   // in flight while this chunk is used
    if (tid < G * kRlaStage) {
      const int h = tid / kRlaStage, t = tid % kRlaStage;
      float d = 0.f;
#pragma unroll 8
      for (int k = 0; k < D; k += 4) {
        const float4 x = *reinterpret_cast<const float4*>(fk + t * LD + k);
        d = fmaf(fq[h * D + k], x.x, d);
        d = fmaf(fq[h * D + k + 1], x.y, d);
        d = fmaf(fq[h * D + k + 2], x.z, d);
        d = fmaf(fq[h * D + k + 3], x.w, d);
      }
      w[h * kRlaStage + t] = d;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < OUTS; ++u) {
      const int o = tid + u * 256;
      if (o < G * D) {
        const int h = o / D;
        float acc = otil[u];
        for (int t = 0; t < kRlaStage; ++t) acc = fmaf(w[h * kRlaStage + t], fv[t * LD + c_col], acc);
        otil[u] = acc;
      }
    }
    __syncthreads();
  }
  float* part = a.partials + (size_t(pair) * a.nsplit + split) * G * D;
#pragma unroll
  for (int u = 0; u < OUTS; ++u) {
    const int o = tid + u * 256;
    if (o < G * D) part[o] = part_o[u] - otil[u];
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void rla_decode_combine_kernel(RlaDecodeArgs a) {
  const int pair = blockIdx.x;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const float* part = a.partials + size_t(pair) * a.nsplit * G * D;
  for (int o = threadIdx.x; o < G * D; o += 256) {
    float r = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) r += part[size_t(sp) * G * D + o];
    a.o[(size_t(b) * a.hq + g * G + o / D) * D + o % D] = r;
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_rla_states(const RlaStateArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.nranges), unsigned(a.pairs));
  if (a.bf16) {
    if (a.d == 128) rla_states_kernel<uint16_t, 128><<<grid, 256, 0, s>>>(a);
    else rla_states_kernel<uint16_t, 64><<<grid, 256, 0, s>>>(a);
  } else {
    if (a.d == 128) rla_states_kernel<float, 128><<<grid, 256, 0, s>>>(a);
    else rla_states_kernel<float, 64><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_rla_reduce(const float* chunks, float* out, int nranges, int d, int pairs, hipStream_t s) {
  const int dd = d * d;
  rla_reduce_kernel<<<dim3(unsigned((dd + 255) / 256), unsigned(pairs)), 256, 0, s>>>(chunks, out, nranges, dd);
  return hipGetLastError();
}

hipError_t launch_rla_prefill(const RlaPrefillArgs& a, hipStream_t s) {
  const unsigned grid = unsigned(a.batch * a.hkv * a.nb);
  if (a.bf16) {
    if (a.d == 128) rla_prefill_kernel<uint16_t, 128><<<grid, 256, 0, s>>>(a);
    else rla_prefill_kernel<uint16_t, 64><<<grid, 256, 0, s>>>(a);
  } else {
    if (a.d == 128) rla_prefill_kernel<float, 128><<<grid, 256, 0, s>>>(a);
    else rla_prefill_kernel<float, 64><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int D, int G>
static void launch_rla_decode_dg(const RlaDecodeArgs& a, hipStream_t s) {
  const unsigned pairs = unsigned(a.batch * a.hkv);
  rla_decode_split_kernel<D, G><<<dim3(unsigned(a.nsplit), pairs), 256, 0, s>>>(a);
  rla_decode_combine_kernel<D, G><<<pairs, 256, 0, s>>>(a);
}

template <int D>
static void launch_rla_decode_d(const RlaDecodeArgs& a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: launch_rla_decode_dg<D, 1>(a, s); break;
    case 2: launch_rla_decode_dg<D, 2>(a, s); break;
    case 4: launch_rla_decode_dg<D, 4>(a, s); break;
    default: launch_rla_decode_dg<D, 8>(a, s); break;
  }
}

int rla_decode_num_splits(int batch, int hkv) {
  const int pairs = batch * hkv;
  int n = 1024 / (pairs > 0 ? pairs : 1);   // measured: 8 splits at the decode workload beat 32
  return n < 1 ? 1 : (n > 64 ? 64 : n);
}

hipError_t launch_rla_decode(const RlaDecodeArgs& a, hipStream_t s) {
  if (a.d == 128) launch_rla_decode_d<128>(a, s);
  else launch_rla_decode_d<64>(a, s);
  return hipGetLastError();
}

}  // namespace spot
