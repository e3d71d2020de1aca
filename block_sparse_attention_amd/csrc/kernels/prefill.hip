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
//   Key tiles of 64 slots walk the concatenated kept blocks; each slot's row
//   (natural or permuted) is loaded from HBM straight into LDS with 16-byte
//   buffer-to-LDS loads, one step ahead of use (K for tile t+2 and V for
//   tile t+1 while tile t is processed), rows unpadded with their 16-byte
//   chunks XOR-swizzled so the fragment reads stay bank-conflict-free; the
//   V^T operand of the PV product is read with the transposing LDS load.
//   S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16, so every
//   lane owns one query column: row max/sum stay in-lane plus one exchange
//   between the two lane halves (the gfx950 lane-half swap, no LDS round
//   trip).  P is rounded to bf16 for the PV product.
//   The running max is only moved when a tile raises it by more than 2^8
//   (the softmax is invariant to the shift, so the result is unchanged).
//   Work units are ordered longest-first (query block descending) and, when
//   the number of (batch, KV head) pairs is a multiple of 8, each KV head is
//   pinned to one XCD so its K/V stay in that XCD's L2.
//
// prefill_rows_kernel (fp32, latency path): one wave per query row.
#include <type_traits>

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

// lane l and lane l^32 exchange through the gfx950 lane-half swap (a VALU op, no LDS round trip);
// the two results of the swap hold the own and the partner value in either order
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef SPOT_PREFILL_WAVES
#define SPOT_PREFILL_WAVES 8        // waves per workgroup (32 packed query rows each)
#endif
#ifndef SPOT_PREFILL_QG
#define SPOT_PREFILL_QG 1           // groups of 32 query rows per wave (2: each LDS fragment feeds 2 MFMAs)
#endif
#ifndef SPOT_PREFILL_SCHED
#define SPOT_PREFILL_SCHED 3        // 0: compiler default; 1: iglp strategy 0; 3: raised wave priority over the MFMA block
#endif
#if SPOT_PREFILL_SCHED != 0 && SPOT_PREFILL_SCHED != 1 && SPOT_PREFILL_SCHED != 3
#error "SPOT_PREFILL_SCHED: 0, 1 or 3 (iglp strategy 1 runs the compiler out of memory on this kernel)"
#endif
#ifndef SPOT_PREFILL_LIST_CAP
#define SPOT_PREFILL_LIST_CAP 2048  // kept-list entries staged in LDS (0: read from HBM)
#endif
constexpr int kListCap = SPOT_PREFILL_LIST_CAP;

// ES: early-stopped variant (S2O section 2 and 3).  The workgroup first walks
// its own segment's blocks (causal), then the history blocks in the given
// visiting order; after each history block every row compares the block's
// softmax mass with the mass accumulated so far (that block included) and
// stops taking further blocks once it is below tau.  A stopped row adds
// nothing more; the workgroup leaves the loop when all its rows have stopped.
// LLDS: every kept list of the launch fits the LDS copy (the number of blocks
// per sequence is at most its capacity), so list entries are LDS reads; else
// they are read from HBM.
template <int D, int NW, int QG, bool PERM, bool ES, bool LLDS>
__global__ __launch_bounds__(NW * 64, QG == 1 ? 2 : 1) void prefill_mfma_kernel(PrefillArgs a, int chunks,
                                                                               float scale_log2) {
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * 32 * QG;                // packed query rows per workgroup
  // K and V tiles: unpadded rows filled by buffer-to-LDS loads (lane l of a
  // load stores its 16 bytes at the load's base + 16 l), so the 16-byte chunk
  // c of tile row r sits in slot c ^ swz(r) of that row: the 16 rows of a
  // K fragment read and the 4 rows x 4 chunks of a transposing V read each
  // land on distinct bank groups.
  constexpr int RB = D * 2;                         // bytes per row
  constexpr int CPR = D / 8;                        // 16-byte chunks per row
  constexpr int CH = kKT * CPR / NT;                // chunks per thread per tile
  static_assert(CH * NT == kKT * CPR, "every thread loads whole chunks of every tile");
  // the two buffers of each are separate arrays, so the compiler can tell
  // the buffer being read from the one the loads are filling
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[kKT * D], Ks1[kKT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[kKT * D], Vs1[kKT * D];
  auto Ks = [&](auto b) -> uint16_t* {
    if constexpr (decltype(b)::value == 0) return Ks0;
    else return Ks1;
  };
  auto Vs = [&](auto b) -> uint16_t* {
    if constexpr (decltype(b)::value == 0) return Vs0;
    else return Vs1;
  };
  __shared__ int kpos[3][kKT];
  // early stopping always stages its (reordered) list; the top-p kernel when every list of the launch fits
  constexpr int LCAP = ES ? (kListCap > kEsMaxBlocks ? kListCap : kEsMaxBlocks) : kListCap;
  __shared__ int s_list[LCAP > 0 ? LCAP : 1];
  // early stop: per-wave "a row is still taking blocks", by tile parity (one byte per wave, read as one word)
  __shared__ __attribute__((aligned(8))) uint8_t s_act[2][NW];
  static_assert(!ES || LCAP >= kEsMaxBlocks, "early stopping stages its visiting list in LDS");
  static_assert(!ES || LLDS, "early stopping reads its list from LDS");
  static_assert(!LLDS || LCAP > 0, "no LDS copy of the list");

  const int pairs = a.batch * a.hkv;
  int pair, i, chunk;
  unit_of(blockIdx.x, pairs, a.nb, chunks, pair, i, chunk);
  const int b = pair / a.hkv;
  const int G = a.hq / a.hkv, B = a.block, L = a.L;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ql = lane & 31, hf = lane >> 5;
  const int GB = G * B;

  // each wave owns QG groups of 32 packed query rows; lane (query ql, half hf)
  int hq_[QG], r_[QG];
  bool qvalid[QG];
  bf16x8_t qf[QG][D / 16];   // Q fragments (B operand of S^T = K Q^T)
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const int pr = chunk * ROWS + (wv * QG + gq) * 32 + ql;
    const int prc = min(pr, GB - 1);
    hq_[gq] = (pair % a.hkv) * G + prc / B;
    const int r_raw = i * B + prc % B;
    qvalid[gq] = pr < GB && r_raw < L;
    r_[gq] = min(r_raw, L - 1);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((size_t(b) * a.hq + hq_[gq]) * L + r_[gq]) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[gq][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16 + hf * 8));
  }

  const size_t row_id = size_t(pair) * a.nb + i;
  const int32_t* glist = a.idx + row_id * a.nb;
  const int lgB = 31 - __builtin_clz(B);
  const int seg_start = ((PERM || ES) && a.segment > 0) ? ((i * B) / a.segment) * a.segment : 0;
  int nkept, own_tiles = 0;
  if constexpr (ES) {
    // own segment's blocks ascending, then the history blocks in visiting
    // order (with history maps: the runs of the map in order, all of them)
    const int sblk = seg_start >> lgB;
    const int n_own = i - sblk + 1;
    nkept = n_own + (a.es_hmap ? sblk : min(max(a.cnt[row_id], 0), sblk));   // at most the blocks before the segment
    for (int k = tid; k < nkept; k += NT)
      s_list[k] = k < n_own ? sblk + k : (a.es_hmap ? k - n_own : glist[k - n_own]);
    own_tiles = (n_own * B) / kKT;
  } else {
    nkept = a.cnt[row_id];
    if constexpr (LLDS)
      for (int k = tid; k < nkept; k += NT) s_list[k] = glist[k];
  }
  // typed reads (LDS or global), never a generic pointer: a flat read could
  // alias the LDS the tile loads are filling and would wait for them
  auto list_at = [&](int k) -> int {
    if constexpr (LLDS) return s_list[k];
    else return glist[k];
  };
  const int32_t* permg =
      PERM ? a.perm + (ES && a.es_hmap ? size_t(pair) * a.nseg + seg_start / max(a.segment, 1) : size_t(pair)) * L
           : nullptr;
  const int ntiles = (nkept * B + kKT - 1) / kKT;
  // tiles before the last kept block need no mask (history and earlier own-segment blocks are visible)
  const int nfull = min(ntiles, ((nkept - 1) * B) / kKT);

  // K/V slabs of this (batch, KV head) as buffer resources: out-of-range reads return zero
  const uint32_t nrec = uint32_t(L) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.k) + size_t(pair) * L * D), 0, int(nrec), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.v) + size_t(pair) * L * D), 0, int(nrec), 0x00020000);

  // where this thread's chunks of tile t come from: byte offset in the slab
  // (out of range for an empty slot) and the row's mask limit (-1: always
  // visible, position: visible iff <= query row, INT_MAX: no key)
  // With the permutation, the permuted row of a history slot is loaded when the tile is mapped and
  // chosen only when the tile is gathered, a step later: a select right after the load becomes a
  // branch around it whose wait (vmcnt 0) would also wait for the tile loads in flight.
  struct RowMap {
    uint32_t off[CH];        // the slot's natural row and chunk (out of range for an empty slot)
    int lim[CH];
    int pp[PERM ? CH : 1];   // the permuted row of the slot's position
  };
  auto swz = [](int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  };
  // the lane fills slot cid % CPR of tile row cid / CPR: it loads the chunk that slot holds
  uint32_t colb[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int cid = tid + c * NT;
    colb[c] = uint32_t(((cid % CPR) ^ swz(cid / CPR)) << 4);
  }
  auto map_tile = [&](int t, RowMap& m) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cid = tid + c * NT;
      const int s = t * kKT + cid / CPR;
      const int bi = s >> lgB;
      const bool inl = bi < nkept && cid < kKT * CPR;
      const int base = list_at(inl ? bi : 0) << lgB;
      const int pos = base + (s & (B - 1));
      const bool valid = inl && unsigned(pos) < unsigned(L);
      const bool hist = base < seg_start;
      m.off[c] = valid ? uint32_t(pos) * RB + colb[c] : 0x80000000u;
      m.lim[c] = valid ? (hist ? -1 : pos) : 0x7fffffff;
      if constexpr (PERM) m.pp[c] = permg[valid ? pos : 0];
    }
  };
  // HBM -> LDS without registers: the wave's 64 lanes of chunk round c fill
  // the 1 KiB that starts at chunk wv * 64 + c * NT of the tile; a history
  // slot (mask limit -1) reads the permuted row
  auto gather = [&](const __amdgpu_buffer_rsrc_t& rs, const RowMap& m, uint16_t* tile) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t off = m.off[c];
      if constexpr (PERM) off = m.lim[c] == -1 ? uint32_t(m.pp[c]) * RB + colb[c] : off;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + (wv * 64 + c * NT) * 8), 16, off, 0, 0, 0);
    }
  };
  // s_waitcnt vmcnt(0) (immediate fields: vmcnt 3:0, expcnt 6:4, lgkmcnt 11:8;
  // the last two at their maxima): this wave's tile loads are in LDS
  auto loads_landed = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };
  auto put_kpos = [&](int* kp, const RowMap& m) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int cid = tid + c * NT;
      if (cid % CPR == 0) kp[cid / CPR] = m.lim[c];
    }
  };

  // byte offsets of this lane's K fragment (row ql, chunk 2 ks + hf) and V
  // transposing reads (row vrow (+8), columns dt * 32 + vcol ..+3) in a tile
  uint32_t koff[D / 16], voff[D / 32][2];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = ql * RB + (((2 * ks + hf) ^ swz(ql)) << 4);
  const int jl = lane & 15, g16 = lane >> 4;
  const int vrow = 4 * (g16 >> 1) + (jl >> 2);          // key row within a 16-key step
  const int vcol = 16 * (g16 & 1) + 4 * (jl & 3);       // column within a 32-wide d tile
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      voff[dt][h] = (vrow + 8 * h) * RB + (((dt * 4 + (vcol >> 3)) ^ swz(vrow + 8 * h)) << 4) + (vcol & 7) * 2;
  auto kfrag = [&](const uint16_t* kt, int rt, int ks) {
    return *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(kt) + rt * 32 * RB + koff[ks]);
  };

  // S^T tiles = K_tile Q^T (64 keys x 32 queries per group); each K fragment
  // read from LDS feeds the QG groups
  auto qk = [&](const uint16_t* kt, f32x16_t (&s)[QG][2]) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bf16x8_t k0 = kfrag(kt, rt, 0);
#pragma unroll
      for (int gq = 0; gq < QG; ++gq)
        s[gq][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[gq][0], f32x16_t{}, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 1; ks < D / 16; ++ks)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x8_t kf = kfrag(kt, rt, ks);
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
          s[gq][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[gq][ks], s[gq][rt], 0, 0, 0);
      }
  };

  // this lane's max over a score tile (the lane-half exchange comes later)
  auto lane_max = [&](const f32x16_t (&st)[2]) {
    float mx = __builtin_fmaxf(st[0][0], st[1][0]);
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = __builtin_fmaxf(__builtin_fmaxf(mx, st[0][e]), st[1][e]);
    return mx;
  };

  f32x16_t oacc[QG][D / 32];
  float m_run[QG], l_run[QG];   // l_run: this lane half's share of the row sum
  float dsum[QG];               // ES: this lane half's share of the mass of the history block in progress
  int nused[QG];                // ES: history blocks taken
  bool active[QG];              // ES: the row still takes blocks
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[gq][dt] = f32x16_t{};
    m_run[gq] = -kInf;
    l_run[gq] = 0.f;
    dsum[gq] = 0.f;
    nused[gq] = 0;
    active[gq] = true;
  }
  const int tpb = B / kKT;   // ES: tiles per block (block >= 64)

  __syncthreads();   // kept list staged

  RowMap mV, mK, mN;
  map_tile(0, mN);
  gather(rk, mN, Ks0);
  gather(rv, mN, Vs0);
  map_tile(1, mV);
  put_kpos(kpos[0], mN);
  gather(rk, mV, Ks1);
  map_tile(2, mK);
  put_kpos(kpos[1], mV);
  loads_landed();
  __syncthreads();
  f32x16_t sa[QG][2], sb[QG][2];
  float ma[QG], mb[QG];   // lane maxima of the unmasked score tiles
  qk(Ks0, sa);
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) ma[gq] = lane_max(sa[gq]);
  __syncthreads();   // iteration 0 loads into Ks0

  // One tile t: softmax of s_cur (scores of tile t) and PV(t); QK(t+1) -> s_nxt.
  // K runs one tile ahead of V: reads K(t+1) and V(t) from LDS, fetches
  // K(t+2) and V(t+1) from HBM (issued first, so they have the whole step to
  // arrive), and maps tile t+3.  m_cur holds this lane's max over tile t,
  // taken in the previous step beside its MFMAs; only the lane-half exchange
  // and the rescale test are left between the barrier and the MFMA block.
  auto step = [&](auto parity, int t, f32x16_t (&s_cur)[QG][2], f32x16_t (&s_nxt)[QG][2], float (&m_cur)[QG],
                  float (&m_nxt)[QG]) -> bool {
    constexpr int P = decltype(parity)::value;   // t & 1
    using BP = std::integral_constant<int, P>;
    using BQ = std::integral_constant<int, P ^ 1>;
    gather(rk, mK, Ks(BP{}));   // K(t+2) into the buffer QK(t) read in the previous step
    gather(rv, mV, Vs(BQ{}));   // V(t+1) into the buffer PV(t-1) read
    // (A) mask, max, rare rescale of the running state
    float msub[QG];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      float mx = m_cur[gq];   // taken beside the MFMAs of the previous step
      if (ES ? (t < own_tiles && t >= own_tiles - tpb) : (t >= nfull)) {   // masked tile: max again
        const int* kp = kpos[t % 3];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kp[rt * 32 + 8 * (e >> 2) + 4 * hf + (e & 3)] > r_[gq]) s_cur[gq][rt][e] = -kInf;
        mx = lane_max(s_cur[gq]);
      }
      // A row's max exceeds the threshold only if the max of one of its lane halves does, so the
      // lane-half exchange is needed only when the wave votes for a rescale (rare after the first tile).
      if (__ballot(active[gq] && mx * scale_log2 > m_run[gq] + kRescaleThreshold)) {
        const float mcand = xhalf_max(mx) * scale_log2;
        const bool need = active[gq] && mcand > m_run[gq] + kRescaleThreshold;
        const float m_new = need ? mcand : m_run[gq];
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run[gq] - m_new) : 1.0f;
        l_run[gq] *= alpha;
        if constexpr (ES) dsum[gq] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[gq][dt][e] *= alpha;
        m_run[gq] = m_new;
      }
      msub[gq] = (m_run[gq] == -kInf) ? 0.f : m_run[gq];
      if constexpr (ES) msub[gq] = active[gq] ? msub[gq] : kInf;   // a stopped row's exponentials are 0
    }

    // (B) straight-line: next map, QK(t+1) on MFMA beside exp(t), PV(t), max of tile t+1
    __builtin_amdgcn_sched_barrier(0);
#if SPOT_PREFILL_SCHED == 1
    __builtin_amdgcn_iglp_opt(0);
#elif SPOT_PREFILL_SCHED == 3
    __builtin_amdgcn_s_setprio(1);
#endif
    map_tile(t + 3, mN);
    qk(Ks(BQ{}), s_nxt);   // stale but in bounds on the last tile
    const char* vt = reinterpret_cast<const char*>(Vs(BP{}));
    float rs[QG];   // row sums of the bf16-rounded P that enters the PV product
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) rs[gq] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rt = kk >> 1, hb = (kk & 1) * 8;
      bf16x8_t pf[QG];
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pv[e] = __builtin_amdgcn_exp2f(fmaf(s_cur[gq][rt][hb + e], scale_log2, -msub[gq]));
        uint4 pp;
        pp.x = pack_bf16x2(pv[0], pv[1]);
        pp.y = pack_bf16x2(pv[2], pv[3]);
        pp.z = pack_bf16x2(pv[4], pv[5]);
        pp.w = pack_bf16x2(pv[6], pv[7]);
        rs[gq] = dot2_bf16(pp.x, kOnes, dot2_bf16(pp.y, kOnes, dot2_bf16(pp.z, kOnes, dot2_bf16(pp.w, kOnes, rs[gq]))));
        pf[gq] = __builtin_bit_cast(bf16x8_t, pp);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vt + kk * 16 * RB + voff[dt][0]));  // keys kk*16 + 4*hf + 0..3
        const uint2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vt + kk * 16 * RB + voff[dt][1]));  // keys kk*16 + 8 + 4*hf + 0..3
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int gq = 0; gq < QG; ++gq)
          oacc[gq][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[gq], oacc[gq][dt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      m_nxt[gq] = lane_max(s_nxt[gq]);
      asm volatile("" : "+v"(m_nxt[gq]));   // keeps the reduction in this block, beside the MFMAs
    }
#if SPOT_PREFILL_SCHED == 3
    __builtin_amdgcn_s_setprio(0);
#endif
    bool block_end = false;
    if constexpr (ES) {
      block_end = t >= own_tiles && ((t - own_tiles + 1) % tpb) == 0;
      bool any = false;
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) {
        l_run[gq] += rs[gq];
        if (t >= own_tiles) dsum[gq] += rs[gq];
        if (block_end) {
          // the row stops when block mass < tau * row sum: the sign of the sum over both lane halves of
          // (mass - tau * sum), one lane-half exchange per block
          const float below = xhalf_sum(dsum[gq] - a.tau * l_run[gq]);
          if (active[gq]) {
            ++nused[gq];
            if (below < 0.f) active[gq] = false;
          }
          dsum[gq] = 0.f;
        }
        any = any || active[gq];
      }
      if (block_end) {
        const bool wave_any = __ballot(any) != 0;   // whole wave: block_end is uniform
        if (lane == 0) s_act[t & 1][wv] = uint8_t(wave_any);
      }
    } else {
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) l_run[gq] += rs[gq];
    }

    // (C) tile t+2's mask limits; K(t+2) and V(t+1) in LDS before the barrier
    // only a tile that is masked reads its limits, and in the top-p kernel those are the tiles touching
    // the last kept block; the early-stopped kernel writes them every tile (the same test there once
    // spilled its registers, and with the current loop it measures no faster)
    if (ES || t + 2 >= nfull) put_kpos(kpos[(t + 2) % 3], mK);
    loads_landed();
    __syncthreads();
    mV = mK;
    mK = mN;
    if constexpr (ES) {
      if (block_end) {
        if constexpr (NW == 8) {
          return *reinterpret_cast<const uint64_t*>(s_act[t & 1]) != 0;
        } else {
          int any = 0;
#pragma unroll
          for (int w = 0; w < NW; ++w) any |= s_act[t & 1][w];
          return any != 0;
        }
      }
    }
    return true;
  };

  // unrolled by two so the score tiles alternate between register sets.  The
  // early-stopped loop is left only after the second step of a pair: with
  // 64-key blocks every history tile ends a block, and with blocks of 128 or
  // more keys the block ends fall on odd tiles, so the second step's vote
  // covers the first's; a step taken after every row has stopped adds nothing
  // (its exponentials are 0 and no count moves).  Testing after the first
  // step as well made the compiler serialize the LDS fragment reads of the
  // second (6% slower).
  int t = 0;
  bool go = true;
  for (; go && t + 1 < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t, sa, sb, ma, mb);   // a block end here is one at t + 1 too
    go = step(std::integral_constant<int, 1>{}, t + 1, sb, sa, mb, ma);
  }
  if (go && t < ntiles) step(std::integral_constant<int, 0>{}, t, sa, sb, ma, mb);

#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    const float l_tot = xhalf_sum(l_run[gq]);
    if (qvalid[gq]) {
      if (ES && a.nused && hf == 0) a.nused[(size_t(b) * a.hq + hq_[gq]) * L + r_[gq]] = nused[gq];
      const float inv = 1.0f / l_tot;
      uint16_t* orow = static_cast<uint16_t*>(a.o) + ((size_t(b) * a.hq + hq_[gq]) * L + r_[gq]) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint2 w;
          w.x = pack_bf16x2(oacc[gq][dt][jj * 4 + 0] * inv, oacc[gq][dt][jj * 4 + 1] * inv);
          w.y = pack_bf16x2(oacc[gq][dt][jj * 4 + 2] * inv, oacc[gq][dt][jj * 4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * jj + 4 * hf) = w;
        }
      if (a.lse && hf == 0)
        a.lse[(size_t(b) * a.hq + hq_[gq]) * L + r_[gq]] = (m_run[gq] + __log2f(l_tot)) * kLn2;
    }
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
  constexpr int NW = SPOT_PREFILL_WAVES;
  constexpr int QG = SPOT_PREFILL_QG;
  const int G = a.hq / a.hkv;
  const int chunks = (G * a.block + NW * 32 * QG - 1) / (NW * 32 * QG);
  const long long units = (long long)a.batch * a.hkv * a.nb * chunks;
  const dim3 grid{unsigned(units)};
  if (a.es) {
    if (a.perm)
      prefill_mfma_kernel<D, NW, QG, true, true, true><<<grid, NW * 64, 0, s>>>(a, chunks, scale_log2);
    else
      prefill_mfma_kernel<D, NW, QG, false, true, true><<<grid, NW * 64, 0, s>>>(a, chunks, scale_log2);
    return hipGetLastError();
  }
  if constexpr (kListCap > 0) {
    if (a.nb <= kListCap) {   // a kept list holds at most nb blocks: every list fits the LDS copy
      if (a.perm)
        prefill_mfma_kernel<D, NW, QG, true, false, true><<<grid, NW * 64, 0, s>>>(a, chunks, scale_log2);
      else
        prefill_mfma_kernel<D, NW, QG, false, false, true><<<grid, NW * 64, 0, s>>>(a, chunks, scale_log2);
      return hipGetLastError();
    }
  }
  if (a.perm)
    prefill_mfma_kernel<D, NW, QG, true, false, false><<<grid, NW * 64, 0, s>>>(a, chunks, scale_log2);
  else
    prefill_mfma_kernel<D, NW, QG, false, false, false><<<grid, NW * 64, 0, s>>>(a, chunks, scale_log2);
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
