// Block-sparse causal prefill attention for gfx950.
//
// What is computed: for each query row, softmax attention over the keys of
// the kept key blocks only (PBS-Attn "Probleemstelling": blocks are skipped by
// a precomputed mask inside FlashAttention tiling), with the online-softmax
// state (m, l, acc) carried across key tiles (S2O section 3, passes 1-2).
// Blocks of earlier segments are gathered row by row through the permutation
// index array, leaving K/V in place in HBM (S2O section 1, index-driven
// loading; PBS-Attn section 2, intra-segment permutation); blocks of the
// query's own segment are read in natural order under the causal mask.
//
// prefill_mfma_kernel (bf16, d = 64 or 128)
//   One workgroup = NW waves = NW*32 packed query rows of one (batch, KV
//   head g, query block i); packed row p is head g*G + p/B, row i*B + p%B,
//   so the G query heads of a group share every K/V tile (GQA packing).
//   Key tiles of 64 slots walk the concatenated kept blocks; each slot is
//   gathered (natural or permuted row) from HBM into registers one tile ahead
//   and written to LDS: K row-major, V transposed (Vt[d][key]).
//   S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16, so every
//   lane owns one query column: row max/sum stay in-lane plus one exchange
//   between the two lane halves.  P is rounded to bf16 for the PV product.
//   The running max is only moved when a tile raises it by more than 2^8
//   (the softmax is invariant to the shift, so the result is unchanged).
//   Work units are ordered longest-first (query block descending) and, when
//   the number of (batch, KV head) pairs is a multiple of 8, each KV head is
//   pinned to one XCD so its K/V stay in that XCD's L2.
//
// prefill_rows_kernel (fp32 or bf16, latency path): one wave per query row.
#include "../launch.h"
#include "common.h"

namespace spot {

constexpr int kKT = 64;          // key slots per tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr uint32_t kOnes = 0x3F803F80u;    // bf16 pair (1, 1)

struct SlotMap {
  const int32_t* list;   // kept block ids of this (b, g, i)
  const int32_t* permg;  // perm row of (b, g) or nullptr
  int nkept, lgB, L;
  int seg_start;         // first position of the query block's segment; 0 without a permutation

  // Logical position of kept slot s (requires nkept >= 1), whether its block
  // lies in an earlier segment (read through the permutation, always
  // visible; otherwise natural row, visible iff <= the query row), and
  // whether s is inside the kept list at all.  Slots with pos >= L are empty.
  __device__ __forceinline__ void at(int s, int& pos, bool& hist, bool& inlist) const {
    const int bi = s >> lgB;
    inlist = bi < nkept;
    const int j = list[inlist ? bi : 0];
    const int base = j << lgB;
    pos = base + (s & ((1 << lgB) - 1));
    hist = base < seg_start;
  }
  __device__ __forceinline__ int phys_of(int pos, bool hist) const { return hist ? permg[pos] : pos; }
};

__device__ __forceinline__ void unit_of(int w, int pairs, int nb, int chunks, int& pair, int& i, int& chunk) {
  if ((pairs & 7) == 0) {
    const int x = w & 7, s = w >> 3;
    const int per_i = (pairs >> 3) * chunks;
    i = nb - 1 - s / per_i;
    const int rem = s % per_i;
    pair = (rem / chunks) * 8 + x;
    chunk = rem % chunks;
  } else {
    const int per_i = pairs * chunks;
    i = nb - 1 - w / per_i;
    const int rem = w % per_i;
    pair = rem / chunks;
    chunk = rem % chunks;
  }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_mfma_kernel(PrefillArgs a, int chunks, float scale_log2) {
  constexpr int NT = NW * 64;
  constexpr int KLD = D + 8;        // K tile row stride (elements)
  constexpr int VLD = kKT + 4;      // Vt row stride (elements)
  constexpr int CK = (kKT * D / 8 + NT - 1) / NT;   // 16-byte K chunks per thread
  constexpr int NVB = (kKT / 4) * (D / 4);           // 4x4 V blocks per tile
  constexpr int CV = (NVB + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKT * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VLD];
  __shared__ int kpos[2][kKT];

  const int pairs = a.batch * a.hkv;
  int pair, i, chunk;
  unit_of(blockIdx.x, pairs, a.nb, chunks, pair, i, chunk);
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int G = a.hq / a.hkv, B = a.block, L = a.L;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ql = lane & 31, hf = lane >> 5;
  const int GB = G * B;
  const int pr = chunk * (NW * 32) + wv * 32 + ql;
  const int prc = min(pr, GB - 1);
  const int h = g * G + prc / B;
  const int r_raw = i * B + prc % B;
  const bool qvalid = pr < GB && r_raw < L;
  const int r = min(r_raw, L - 1);

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + size_t(pair) * L * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + size_t(pair) * L * D;

  // Q fragments (B operand of S^T = K Q^T): lane (query ql, half hf)
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qrow = Q + ((size_t(b) * a.hq + h) * L + r) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16 + hf * 8));
  }

  SlotMap sm;
  const size_t row_id = (size_t(pair) * a.nb + i);
  sm.list = a.idx + row_id * a.nb;
  sm.nkept = a.cnt[row_id];
  sm.permg = a.perm ? a.perm + size_t(pair) * L : nullptr;
  sm.lgB = 31 - __builtin_clz(B);
  sm.L = L;
  sm.seg_start = (a.perm && a.segment > 0) ? ((i * B) / a.segment) * a.segment : 0;
  const int total = sm.nkept * B;
  const int ntiles = (total + kKT - 1) / kKT;
  const int last_block_start = (sm.nkept - 1) * B;

  uint4 kreg[CK];
  uint2 vreg[CV][4];
  int kp_lim = 0;

  auto load_tile = [&](int t) {
    const int s0 = t * kKT;
#pragma unroll
    for (int c = 0; c < CK; ++c) {
      const int cid = tid + c * NT;
      const int row = cid / (D / 8), col8 = cid % (D / 8);
      int pos;
      bool hist, inl;
      sm.at(s0 + row, pos, hist, inl);
      const bool ok = cid < kKT * D / 8 && inl && pos < L;
      kreg[c] = make_uint4(0u, 0u, 0u, 0u);
      if (ok) kreg[c] = *reinterpret_cast<const uint4*>(Kg + size_t(sm.phys_of(pos, hist)) * D + col8 * 8);
    }
#pragma unroll
    for (int c = 0; c < CV; ++c) {
      const int vb = tid + c * NT;
      const int dg = vb % (D / 4), kq = vb / (D / 4);
      int pos;
      bool hist, inl;
      sm.at(s0 + 4 * kq, pos, hist, inl);   // 4 consecutive slots of one block (B >= 4)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const bool ok = vb < NVB && inl && pos + rr < L;
        vreg[c][rr] = make_uint2(0u, 0u);
        if (ok) vreg[c][rr] = *reinterpret_cast<const uint2*>(Vg + size_t(sm.phys_of(pos + rr, hist)) * D + dg * 4);
      }
    }
    if (tid < kKT) {
      int pos;
      bool hist, inl;
      sm.at(s0 + tid, pos, hist, inl);
      kp_lim = (inl && pos < L) ? (hist ? -1 : pos) : 0x7fffffff;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CK; ++c) {
      const int cid = tid + c * NT;
      if (cid < kKT * D / 8) {
        const int row = cid / (D / 8), col8 = cid % (D / 8);
        *reinterpret_cast<uint4*>(&Ks[buf][row * KLD + col8 * 8]) = kreg[c];
      }
    }
#pragma unroll
    for (int c = 0; c < CV; ++c) {
      const int vb = tid + c * NT;
      if (vb < NVB) {
        const int dg = vb % (D / 4), kq = vb / (D / 4);
        // 4 keys x 4 dims -> 4 rows of Vt, each 4 consecutive keys
        const uint2* v4 = vreg[c];
        uint2 o0, o1, o2, o3;
        o0.x = __builtin_amdgcn_perm(v4[1].x, v4[0].x, 0x05040100u);
        o0.y = __builtin_amdgcn_perm(v4[3].x, v4[2].x, 0x05040100u);
        o1.x = __builtin_amdgcn_perm(v4[1].x, v4[0].x, 0x07060302u);
        o1.y = __builtin_amdgcn_perm(v4[3].x, v4[2].x, 0x07060302u);
        o2.x = __builtin_amdgcn_perm(v4[1].y, v4[0].y, 0x05040100u);
        o2.y = __builtin_amdgcn_perm(v4[3].y, v4[2].y, 0x05040100u);
        o3.x = __builtin_amdgcn_perm(v4[1].y, v4[0].y, 0x07060302u);
        o3.y = __builtin_amdgcn_perm(v4[3].y, v4[2].y, 0x07060302u);
        uint16_t* base = &Vt[buf][(4 * dg) * VLD + 4 * kq];
        *reinterpret_cast<uint2*>(base) = o0;
        *reinterpret_cast<uint2*>(base + VLD) = o1;
        *reinterpret_cast<uint2*>(base + 2 * VLD) = o2;
        *reinterpret_cast<uint2*>(base + 3 * VLD) = o3;
      }
    }
    if (tid < kKT) kpos[buf][tid] = kp_lim;
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -kInf, l_run = 0.f;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T tile (64 keys x 32 queries per wave)
    f32x16_t sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[rt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(&Ks[buf][(rt * 32 + ql) * KLD + ks * 16 + hf * 8]);
        sacc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[rt], 0, 0, 0);
      }
    }

    if (t * kKT + kKT > last_block_start) {  // tile touches the last kept block: apply the mask
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int slot = rt * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
          if (kpos[buf][slot] > r) sacc[rt][e] = -kInf;
        }
    }

    // online softmax (per lane = per query; halves share the max)
    float mx = sacc[0][0];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[rt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mcand = mx * scale_log2;
    const bool need = mcand > m_run + kRescaleThreshold;
    if (__ballot(need)) {
      const float m_new = need ? mcand : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
      m_run = m_new;
    }
    const float msub = (m_run == -kInf) ? 0.f : m_run;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[rt][e] = __builtin_amdgcn_exp2f(fmaf(sacc[rt][e], scale_log2, -msub));
    float rs = 0.f;   // row sum of the bf16-rounded P that enters the PV product

    // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rt = kk >> 1, hb = (kk & 1) * 8;
      uint4 pp;
      pp.x = pack_bf16x2(sacc[rt][hb + 0], sacc[rt][hb + 1]);
      pp.y = pack_bf16x2(sacc[rt][hb + 2], sacc[rt][hb + 3]);
      pp.z = pack_bf16x2(sacc[rt][hb + 4], sacc[rt][hb + 5]);
      pp.w = pack_bf16x2(sacc[rt][hb + 6], sacc[rt][hb + 7]);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pp);
      rs = dot2_bf16(pp.x, kOnes, dot2_bf16(pp.y, kOnes, dot2_bf16(pp.z, kOnes, dot2_bf16(pp.w, kOnes, rs))));
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint16_t* vrow = &Vt[buf][(dt * 32 + ql) * VLD + kk * 16 + 4 * hf];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[dt], 0, 0, 0);
      }
    }

    l_run += rs;

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + ((size_t(b) * a.hq + h) * L + r) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint2 w;
        w.x = pack_bf16x2(oacc[dt][jj * 4 + 0] * inv, oacc[dt][jj * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[dt][jj * 4 + 2] * inv, oacc[dt][jj * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * jj + 4 * hf) = w;
      }
    if (a.lse && hf == 0) a.lse[(size_t(b) * a.hq + h) * L + r] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------- row kernel
// One wave per query row; lanes take 64 key slots at a time for the logits,
// then own head dimensions for the PV accumulation.
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_rows_kernel(PrefillArgs a, float scale_log2) {
  constexpr int DU = D / 64;
  __shared__ float qs[4][D];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long rid = (long long)blockIdx.x * 4 + wv;
  const int L = a.L, B = a.block, G = a.hq / a.hkv;
  const long long nrows = (long long)a.batch * a.hq * L;
  const bool active = rid < nrows;
  const long long ridc = active ? rid : 0;
  const int r = int(ridc % L);
  const int h = int((ridc / L) % a.hq);
  const int b = int(ridc / ((long long)L * a.hq));
  const int g = h / G, i = r / B;
  const int pair = b * a.hkv + g;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k) + size_t(pair) * L * D;
  const T* V = static_cast<const T*>(a.v) + size_t(pair) * L * D;
  const T* qrow = Q + ((size_t(b) * a.hq + h) * L + r) * D;
  for (int c = lane; c < D; c += 64) qs[wv][c] = Elem<T>::ld(qrow + c);
  __syncthreads();
  if (!active) return;

  SlotMap sm;
  const size_t row_id = size_t(pair) * a.nb + i;
  sm.list = a.idx + row_id * a.nb;
  sm.nkept = a.cnt[row_id];
  sm.permg = a.perm ? a.perm + size_t(pair) * L : nullptr;
  sm.lgB = 31 - __builtin_clz(B);
  sm.L = L;
  sm.seg_start = (a.perm && a.segment > 0) ? ((i * B) / a.segment) * a.segment : 0;
  const int total = sm.nkept * B;

  float m = -kInf, l = 0.f, acc[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) acc[u] = 0.f;
  for (int s0 = 0; s0 < total; s0 += 64) {
    int pos;
    bool hist, inl;
    sm.at(s0 + lane, pos, hist, inl);
    const bool valid = inl && pos < L;
    const bool vis = valid && (hist || pos <= r);
    const int phys = vis ? sm.phys_of(pos, hist) : 0;
    float x = -kInf;
    if (vis) {
      const T* krow = K + size_t(phys) * D;
      float dotv = 0.f;
      for (int c = 0; c < D; ++c) dotv = fmaf(qs[wv][c], Elem<T>::ld(krow + c), dotv);
      x = dotv * scale_log2;
    }
    const float mx = wave_max(x);
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == m) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
    const float p = vis ? __builtin_amdgcn_exp2f(x - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[u] *= alpha;
    m = m_new;
    const int src = vis ? phys : -1;
    for (int j = 0; j < 64; ++j) {
      const int pj_row = __shfl(src, j);
      const float pj = __shfl(p, j);
      if (pj_row >= 0) {
        const T* vrow = V + size_t(pj_row) * D;
#pragma unroll
        for (int u = 0; u < DU; ++u) acc[u] = fmaf(pj, Elem<T>::ld(vrow + lane + 64 * u), acc[u]);
      }
    }
  }
  const float inv = 1.f / l;
  T* orow = static_cast<T*>(a.o) + ((size_t(b) * a.hq + h) * L + r) * D;
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    const float val = acc[u] * inv;
    if constexpr (sizeof(T) == 4) {
      orow[lane + 64 * u] = val;
    } else {
      orow[lane + 64 * u] = uint16_t(pack_bf16x2(val, 0.f) & 0xFFFFu);
    }
  }
  if (a.lse && lane == 0) a.lse[(size_t(b) * a.hq + h) * L + r] = (m + __log2f(l)) * kLn2;
}

template <int D>
static hipError_t launch_mfma(const PrefillArgs& a, hipStream_t s, float scale_log2) {
  constexpr int NW = 8;
  const int G = a.hq / a.hkv;
  const int chunks = (G * a.block + NW * 32 - 1) / (NW * 32);
  const long long units = (long long)a.batch * a.hkv * a.nb * chunks;
  prefill_mfma_kernel<D, NW><<<dim3(unsigned(units)), NW * 64, 0, s>>>(a, chunks, scale_log2);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const float scale_log2 = a.sm_scale * kLog2e;
  if (a.bf16) {
    if (a.d == 128) return launch_mfma<128>(a, s, scale_log2);
    if (a.d == 64) return launch_mfma<64>(a, s, scale_log2);
    return hipErrorInvalidValue;
  }
  const long long rows = (long long)a.batch * a.hq * a.L;
  const unsigned blocks = unsigned((rows + 3) / 4);
  if (a.d == 128) prefill_rows_kernel<float, 128><<<blocks, 256, 0, s>>>(a, scale_log2);
  else if (a.d == 64) prefill_rows_kernel<float, 64><<<blocks, 256, 0, s>>>(a, scale_log2);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace spot
