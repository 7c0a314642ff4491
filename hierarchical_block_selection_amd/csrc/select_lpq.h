// Lane-per-query decision kernels of the two-stage selection (K <= 16).
//
// Every Top-K decision of the descent (PISA reading page §4.2 eq. (5), §03
// keep-all rule, §5.3 forced nodes) is taken by one lane for one query: the
// lane holds its query's candidate list (the children of the nodes it kept
// one level up, at most 2K <= 32 of them, ascending) and ranks the rankable
// ones with a sorting network over packed 32-bit keys in registers.
//
// Rank keys.  A candidate in slot j (slots follow node order) is keyed by the
// order-preserving integer image of its score with the low 5 bits replaced by
// 31 - j.  A larger key ranks first; scores that agree to within 2^-18
// relative are therefore ordered by node index, which is the tie rule of the
// selection (equal scores -> lower index first).  Scores are fp32 sums of
// fp32 log-sum-exps, already uncertain at that level.
//
// Forced slots.  In causal mode the forced nodes of a level (current path,
// and with forcing the first and previous leaf's ancestors) are always
// candidates, because their parents were forced one level up.  The valid
// candidates are the prefix of the ascending list with nodes <= lim, so the
// current-path node lim is the last valid slot, the previous leaf's ancestor
// is lim or lim - 1 (then the slot before), and node 0 is slot 0.
//
// Stage 1 (levels L..3).  One wavefront owns 64 (query, head) columns.  For a
// level whose children fit in kDenseRows rows, the wave computes the logits
// of every child row needed by any of its columns on the matrix cores
// (32 rows x 64 columns per step; bf16 hi/lo planes of the fp32 summaries,
// so each product is exact and accumulation is fp32), and while the logits
// are still in the MFMA register layout it forms the log-sum-exp of every
// sibling pair (eq. (7)), sums the group's heads (eq. (11)) and scatters the
// scores of the pairs that are candidates of the column's query into that
// query's slot array.  Candidacy and slot come from a bitmask of the query's
// kept parents: slot = 2 * (#kept parents before) + child.  Larger levels
// gather the candidates' children from the fp32 pyramid, one query at a time.
//
// Final (levels 2 and 1).  One lane per query reads its K kept level-3 nodes
// and the stage-2 scores of their children, decides level 2 and then the
// leaves, and writes the ascending leaf list.
#pragma once

#include <type_traits>

#include "pisa_common.h"

namespace pisa {
namespace lpq {

constexpr int kSlots = 32;       // 2K candidates, K <= 16
constexpr int kMaxK = 16;
constexpr int kWaves = 4;        // independent wavefronts per workgroup
constexpr int kDenseRows = 2048; // child rows scored densely
constexpr int kMaskWords = kDenseRows / 4 / 32;  // parent bitmask words per query
// Per-query LDS arrays are stored slot-major ([slot][query]) so that lanes of
// different queries always touch different banks.

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Order-preserving image of a float (larger float -> larger unsigned).
__device__ __forceinline__ uint32_t ordered_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t rank_key(float s, int slot) {
  return (ordered_bits(s) & ~31u) | uint32_t(31 - slot);
}

// Batcher's odd-even merge sort network on 32 elements (191 comparators),
// generated at compile time.
struct OddEvenNet32 {
  int a[191];
  int b[191];
  int n;
  constexpr OddEvenNet32() : a(), b(), n(0) {
    for (int p = 1; p < 32; p += p)
      for (int k = p; k > 0; k /= 2)
        for (int j = k % p; j + k < 32; j += k + k)
          for (int i = 0; i < k && i + j + k < 32; ++i)
            if ((i + j) / (p + p) == (i + j + k) / (p + p)) {
              a[n] = i + j;
              b[n] = i + j + k;
              ++n;
            }
  }
};
static_assert(OddEvenNet32().n == 191, "odd-even merge network size");

// Sort 32 keys in descending order, in registers.
__device__ __forceinline__ void sort32_desc(uint32_t (&k)[32]) {
  constexpr OddEvenNet32 net{};
#pragma unroll
  for (int x = 0; x < 191; ++x) {
    const uint32_t u = k[net.a[x]], v = k[net.b[x]];
    k[net.a[x]] = max(u, v);
    k[net.b[x]] = min(u, v);
  }
}

__device__ __forceinline__ uint32_t prefix_mask(int n) {
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// Forced slots of a ranked level (n_valid > K >= 1 valid candidates).
__device__ __forceinline__ uint32_t forced_slots(int n_valid, bool causal, bool force,
                                                 bool prev_distinct) {
  uint32_t m = 0;
  if (causal) {
    m = 1u << (n_valid - 1);
    if (force) m |= 1u | (prev_distinct ? (1u << (n_valid - 2)) : 0u);
  }
  return m;
}

// Kept slots of a ranked level: the forced ones plus the best K - #F of the
// other valid ones by score s[j].
__device__ __forceinline__ uint32_t top_slots(int n_valid, int topk, uint32_t fm,
                                              const float (&s)[kSlots]) {
  const uint32_t rm = prefix_mask(n_valid) & ~fm;
  const int keep_n = topk - __popc(fm);
  uint32_t key[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) key[j] = ((rm >> j) & 1u) ? rank_key(s[j], j) : 0u;
  sort32_desc(key);
  uint32_t km = fm;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) km |= (i < keep_n) ? (1u << (31 - (key[i] & 31u))) : 0u;
  return km;
}

// A query's column of a slot-major LDS array.
template <typename E>
struct Column {
  E* p;
  int stride;
  __device__ __forceinline__ E& operator[](int i) const { return p[i * stride]; }
};

// Kept slots -> ascending node list through LDS (kMaxK + 1 entries; entry
// kMaxK takes the stores of slots that are not kept).
template <typename NodeOf>
__device__ __forceinline__ void compact_kept(uint32_t km, Column<int> row, NodeOf node_of) {
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const bool k = (km >> j) & 1u;
    const int pos = __popc(km & ((1u << j) - 1u));
    row[k ? min(pos, kMaxK) : kMaxK] = node_of(j);
  }
}

// Split fp32 pyramid values into bf16 hi/lo planes: x = hi + lo + r with
// |r| <= 2^-16 |x|, so that a bf16 MFMA over both planes reproduces an fp32
// dot product to that accuracy.
__global__ void split_planes_kernel(const float* __restrict__ pyr, bf16_t* __restrict__ hi,
                                    bf16_t* __restrict__ lo, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const float x = pyr[i];
    const uint16_t h = f32_to_bf16(x);
    hi[i] = h;
    lo[i] = f32_to_bf16(x - bf16_to_f32(h));
  }
}

// ---------------------------------------------------------------------------
// Stage 1
// ---------------------------------------------------------------------------

template <int D, int G>
__global__ __launch_bounds__(kWaves * kWave, 2) void stage1_kernel(
    const bf16_t* __restrict__ q, const float* __restrict__ pyr, const bf16_t* __restrict__ phi,
    const bf16_t* __restrict__ plo, int* __restrict__ s1_nodes, int heads_q, int heads_kv,
    int n_tok, int block, int topk, int causal, int force, float scale_log2, LevelTable lv,
    int split_level) {
  constexpr int T = kWave / G;  // queries per wave
  constexpr int KSTEPS = D / 16;
  __shared__ float score_s[kWaves][kSlots + 1][T];
  __shared__ uint32_t mask_s[kWaves][kMaskWords][T];
  __shared__ int list_s[kWaves][kMaxK + 1][T];

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  // A causal query's dense work grows with t: workgroups are dispatched in
  // linear order, so the latest positions of every head go first.
  const unsigned lin = blockIdx.x + blockIdx.y * gridDim.x;
  const int bh = (int)(lin % gridDim.y);
  const int bx = (int)(gridDim.x - 1 - lin / gridDim.y);
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int t0 = (bx * kWaves + wave) * T;
  if (t0 >= n_tok) return;
  const bool cz = causal != 0, fzon = force != 0;
  const size_t head_rows = (size_t)bh * lv.rows;

  // MFMA layout: this lane feeds columns col and 32 + col, k half kh.
  // Columns past the sequence end repeat its last query (never used).
  const int col = lane & 31, kh = lane >> 5;
  bf16x8_t bq[2][KSTEPS];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = 32 * cb + col;
    const int tq = min(t0 + c / G, n_tok - 1);
    const bf16_t* qrow =
        q + (((size_t)b * heads_q + (size_t)kvh * G + c % G) * n_tok + tq) * D + 8 * kh;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      bq[cb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * s));
  }

  // Decision lane: query t0 + lane (lanes >= T idle in decisions).
  const int t = t0 + lane;
  const bool dlane = lane < T && t < n_tok;
  const int cur = dlane ? t / block : 0;
  const int t_last = min(t0 + T, n_tok) - 1;
  const int cur_last = t_last / block;
  int kp[kMaxK];  // kept nodes one level up, ascending
  int nk = 1;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) kp[i] = 0;
  const int ql = lane < T ? lane : 0;
  const Column<float> srow{&score_s[wave][0][ql], T};
  const Column<int> lrow{&list_s[wave][0][ql], T};
  const Column<uint32_t> mrow{&mask_s[wave][0][ql], T};

  for (int l = lv.n; l >= split_level; --l) {
    const int sh = l - 1;
    const int size_l = lv.size[l - 1];
    const int lim = cz ? (cur >> sh) : size_l - 1;
    // Candidates: children of the kept nodes, ascending; the valid ones
    // (existing, not in the future: node <= x_max) form a prefix.
    const int x_max = min(size_l - 1, lim);
    int n_valid = 0;
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
      const int c = 2 * kp[i];
      n_valid += (i < nk) ? int(c <= x_max) + int(c + 1 <= x_max) : 0;
    }
    if (!dlane) n_valid = 0;
    const bool need = n_valid > topk;

    if (__ballot(need) != 0) {
      const int m_child = lv.size[l - 2];
      const size_t child0 = head_rows + lv.off[l - 2];
      if (m_child <= kDenseRows) {
        // Parent masks were written after the previous level's decision.
        const int lim_last = cz ? (cur_last >> sh) : size_l - 1;
        const int rows_needed = min(m_child, 2 * lim_last + 2);
        int base[2] = {0, 0};
        const Column<uint32_t> mcol[2] = {{&mask_s[wave][0][(32 * 0 + col) / G], T},
                                          {&mask_s[wave][0][(32 * 1 + col) / G], T}};
        const Column<float> scol[2] = {{&score_s[wave][0][(32 * 0 + col) / G], T},
                                       {&score_s[wave][0][(32 * 1 + col) / G], T}};
        const bool writer = (col % G) == 0;
        // The next chunk at or after row r whose parents some query of the
        // wave keeps (rows_needed when there is none).
        auto next_chunk = [&](int r) __attribute__((always_inline)) {
          for (; r < rows_needed; r += 32) {
            const int p = r >> 2;
            uint32_t any = 0;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) any |= (mcol[cb][p >> 5] >> (p & 31)) & 0xffu;
            if (__ballot(any != 0u) != 0) break;
          }
          return r;
        };
        // Summary rows r0 + col of a chunk (rows past the level end repeat its
        // last row; their logits are never used: see the ragged-chunk masking).
        uint4 hv[KSTEPS], lv4[KSTEPS];
        auto fetch = [&](int r0) __attribute__((always_inline)) {
          const int r = min(r0 + col, m_child - 1);
          const bf16_t* hrow = phi + (child0 + r) * D + 8 * kh;
          const bf16_t* lrow2 = plo + (child0 + r) * D + 8 * kh;
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
            hv[s] = *reinterpret_cast<const uint4*>(hrow + 16 * s);
            lv4[s] = *reinterpret_cast<const uint4*>(lrow2 + 16 * s);
          }
        };
        // One chunk: S = summaries x queries on MFMA (hv, lv4 hold its rows),
        // then the candidates' LSEs picked up into the slot arrays.
        auto chunk = [&](int r0, auto&& between) __attribute__((always_inline)) {
          // Rows of this chunk: r0 + 8g + 4kh + i%4 (acc element 4g + i%4);
          // level-l candidates n = r0/2 + 4g + 2kh + m own rows 2n, 2n+1;
          // their parents p = r0/4 + 2g + kh (bits p0..p0+7 of the masks).
          const int p0 = r0 >> 2;  // multiple of 8
          uint32_t byte[2];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) byte[cb] = (mcol[cb][p0 >> 5] >> (p0 & 31)) & 0xffu;
          f32x16_t acc[2] = {};
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lv4[s]), bq[cb][s],
                                                                acc[cb], 0, 0, 0);
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(hv[s]), bq[cb][s],
                                                                acc[cb], 0, 0, 0);
            }
          }
          between();
          auto pickup = [&](auto full_tag) {
            constexpr bool kFull = decltype(full_tag)::value;  // every row of the chunk exists
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int pb = 2 * g + kh;
                const bool has = writer & ((byte[cb] >> pb) & 1u);
                const int pslot = base[cb] + __popc(byte[cb] & ((1u << pb) - 1u));
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                  const int n = (r0 >> 1) + 4 * g + 2 * kh + m;
                  const float z0 = acc[cb][4 * g + 2 * m];
                  float z1 = acc[cb][4 * g + 2 * m + 1];
                  bool w = has;
                  if (!kFull) {
                    z1 = 2 * n + 1 < m_child ? z1 : neg_inf();
                    w &= 2 * n < m_child;
                  }
                  const float mx = fmaxf(z0, z1), mn = fminf(z0, z1);
                  float v =
                      fmaf(mx, scale_log2, fast_log2(1.f + fast_exp2((mn - mx) * scale_log2)));
                  if (G >= 2) v += __shfl_xor(v, 1, kWave);
                  if (G >= 4) v += __shfl_xor(v, 2, kWave);
                  if (G >= 8) v += __shfl_xor(v, 4, kWave);
                  if (G >= 16) v += __shfl_xor(v, 8, kWave);
                  scol[cb][w ? 2 * pslot + m : kSlots] = v;
                }
              }
              base[cb] += __popc(byte[cb]);
            }
          };
          if (r0 + 32 <= m_child)
            pickup(std::true_type{});
          else
            pickup(std::false_type{});
        };
        if constexpr (G == 1) {
          // the next chunk's rows are in flight while this one is picked up
          int r0 = next_chunk(0);
          if (r0 < rows_needed) fetch(r0);
          while (r0 < rows_needed) {
            const int rn = next_chunk(r0 + 32);
            chunk(r0, [&] { if (rn < rows_needed) fetch(rn); });
            r0 = rn;
          }
        } else {  // larger groups need the registers: fetch, then compute
          for (int r0 = next_chunk(0); r0 < rows_needed; r0 = next_chunk(r0 + 32)) {
            fetch(r0);
            chunk(r0, [] {});
          }
        }
      } else {
        // Gather: one query at a time; lane L scores child row L of the
        // query's candidate list (candidate L >> 1, child L & 1).
        for (int qi = 0; qi < T; ++qi) {
          if (!__builtin_amdgcn_readlane(need ? 1 : 0, qi)) continue;
          const int j = lane >> 1;
          const int nkq = __builtin_amdgcn_readlane(nk, qi);
          const int nvq = __builtin_amdgcn_readlane(n_valid, qi);
          const int par = list_s[wave][j >> 1][qi];
          const int cnode = 2 * par + (j & 1);
          const int row = 2 * cnode + (lane & 1);
          const bool live = ((j >> 1) < nkq) & (j < nvq) & (row < m_child);
          const float* xr = pyr + (child0 + (live ? row : 0)) * D;
          float tot = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const bf16_t* qr =
                q + (((size_t)b * heads_q + (size_t)kvh * G + h) * n_tok + (t0 + qi)) * D;
            float a = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < D; c8 += 8) {
              float qv[8];
              load16(qr + c8, qv);
              const float4 x0 = *reinterpret_cast<const float4*>(xr + c8);
              const float4 x1 = *reinterpret_cast<const float4*>(xr + c8 + 4);
              a += qv[0] * x0.x + qv[1] * x0.y + qv[2] * x0.z + qv[3] * x0.w + qv[4] * x1.x +
                   qv[5] * x1.y + qv[6] * x1.z + qv[7] * x1.w;
            }
            const float z = live ? a * scale_log2 : neg_inf();
            const float zo = __shfl_xor(z, 1, kWave);
            const float mx = fmaxf(z, zo), mn = fminf(z, zo);
            tot += mx + fast_log2(1.f + fast_exp2(mn - mx));
          }
          if ((lane & 1) == 0) score_s[wave][live ? j : kSlots][qi] = tot;
        }
      }
      wave_lds_sync();
    }

    // Decision for this lane's query.
    uint32_t km = prefix_mask(n_valid);
    if (need) {
      float sc[kSlots];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) sc[j] = srow[j];
      const bool prev_distinct = cur >= 1 && ((cur - 1) >> sh) != lim;
      km = top_slots(n_valid, topk, forced_slots(n_valid, cz, fzon, prev_distinct), sc);
    }
    compact_kept(km, lrow, [&](int j) { return 2 * kp[j >> 1] + (j & 1); });
    wave_lds_sync();
    nk = __popc(km);
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) kp[i] = lrow[i];
    if (l == split_level) break;
    // Parent bitmask for the next level's dense pass (kept nodes of level l).
    const int nl = l - 1;
    if (lv.size[nl - 1] > topk && lv.size[nl - 2] <= kDenseRows) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) mrow[w] = 0u;
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < kMaxK; ++i)
        if (dlane & (i < nk)) atomicOr(&mrow[kp[i] >> 5], 1u << (kp[i] & 31));
    }
    wave_lds_sync();
  }
  if (dlane) {
    int* out = s1_nodes + ((size_t)bh * n_tok + t) * topk;
    if ((topk & 3) == 0) {
#pragma unroll
      for (int i = 0; i < kMaxK; i += 4)
        if (i < topk)
          *reinterpret_cast<int4*>(out + i) =
              make_int4(i < nk ? kp[i] : -1, i + 1 < nk ? kp[i + 1] : -1,
                        i + 2 < nk ? kp[i + 2] : -1, i + 3 < nk ? kp[i + 3] : -1);
    } else {
#pragma unroll
      for (int i = 0; i < kMaxK; ++i)
        if (i < topk) out[i] = i < nk ? kp[i] : -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Final decisions at levels 2 and 1
// ---------------------------------------------------------------------------

// scores[(u*K + slot)*STRIDE + j]: j = 0..3 exact LSE of leaf 4n + j, j = 4, 5
// level-2 score of child 2n + (j - 4), for the slot's level-3 node n (nats).
template <int STRIDE>
__global__ __launch_bounds__(kWaves * kWave) void final_kernel(
    const int* __restrict__ s1_nodes, const float* __restrict__ scores, int32_t* __restrict__ idx,
    float* __restrict__ score_out, int n_tok, int block, int topk, int causal, int force, int m1,
    int m2, int vec_out) {
  __shared__ int list_s[kWaves][kMaxK + 1][kWave];
  __shared__ float out_s[kWaves][kMaxK + 1][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int t = (blockIdx.x * kWaves + wave) * kWave + lane;
  const bool live = t < n_tok;
  const int bh = blockIdx.y;
  const size_t u = (size_t)bh * n_tok + (live ? t : n_tok - 1);
  const bool cz = causal != 0, fzon = force != 0;
  const int cur = live ? t / block : 0;
  const Column<int> lrow{&list_s[wave][0][lane], kWave};
  const Column<float> frow{&out_s[wave][0][lane], kWave};
  const float* sc = scores + u * topk * STRIDE;

  int n3[kMaxK];
  const int* s1 = s1_nodes + u * topk;
  if ((topk & 3) == 0) {  // 16-byte rows
#pragma unroll
    for (int i = 0; i < kMaxK; i += 4) {
      const int4 v = i < topk ? *reinterpret_cast<const int4*>(s1 + i) : make_int4(-1, -1, -1, -1);
      n3[i] = v.x; n3[i + 1] = v.y; n3[i + 2] = v.z; n3[i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) n3[i] = i < topk ? s1[i] : -1;
  }
  int nk3 = 0;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) nk3 += n3[i] >= 0 ? 1 : 0;
  // Every slot's four leaf LSEs and two level-2 scores, loaded in one pass
  // (slot indices are clamped so that unused entries never read past this
  // query's K slots).  Reading the leaf LSEs only after the level-2 decision
  // fetched the query's score lines from memory a second time.
  float4 lv[kMaxK];
  float2 l2[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    const float* p = sc + min(i, topk - 1) * STRIDE;
    lv[i] = *reinterpret_cast<const float4*>(p);
    l2[i] = *reinterpret_cast<const float2*>(p + 4);
  }

  // Level 2: candidate j = child (j & 1) of level-3 node n3[j >> 1].
  int lim = cz ? (cur >> 1) : m2 - 1;
  int x_max = min(m2 - 1, lim);
  int nv = 0;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    const int c = 2 * n3[i];
    nv += (i < nk3) ? int(c <= x_max) + int(c + 1 <= x_max) : 0;
  }
  if (!live) nv = 0;
  uint32_t km2 = prefix_mask(nv);
  if (nv > topk) {
    float s2[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) s2[j] = (j & 1) ? l2[j >> 1].y : l2[j >> 1].x;
    const bool prev_distinct = cur >= 1 && ((cur - 1) >> 1) != lim;
    km2 = top_slots(nv, topk, forced_slots(nv, cz, fzon, prev_distinct), s2);
  }
  // Kept level-2 candidates, ascending, as (node << 5) | j.
  compact_kept(km2, lrow, [&](int j) { return ((2 * n3[j >> 1] + (j & 1)) << 5) | j; });
  wave_lds_sync();
  const int nk2 = __popc(km2);
  int k2[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) k2[i] = lrow[i];
  wave_lds_sync();
  // Level 1: candidate j = leaf (j & 1) of the kept level-2 node k2[j >> 1]
  // (node k2 >> 5).  The leaf pairs of the kept level-2 candidates are
  // compacted through LDS in the same order as k2: the first leaf's LSE as
  // bits through the int column, the second's through the float column.
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const bool k = (km2 >> j) & 1u;
    const int pos = k ? min(__popc(km2 & ((1u << j) - 1u)), kMaxK) : kMaxK;
    const float4 v = lv[j >> 1];
    lrow[pos] = __float_as_int((j & 1) ? v.z : v.x);
    frow[pos] = (j & 1) ? v.w : v.y;
  }
  wave_lds_sync();
  float2 l1[kMaxK];  // entries past nk2 are stale and never ranked
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) l1[i] = make_float2(__int_as_float(lrow[i]), frow[i]);
  wave_lds_sync();
  lim = cz ? cur : m1 - 1;
  x_max = min(m1 - 1, lim);
  nv = 0;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    const int c = 2 * (k2[i] >> 5);
    nv += (i < nk2) ? int(c <= x_max) + int(c + 1 <= x_max) : 0;
  }
  if (!live) nv = 0;
  const bool ranked = nv > topk;
  uint32_t km1 = prefix_mask(nv), fm1 = 0;
  float s1v[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) s1v[j] = (j & 1) ? l1[j >> 1].y : l1[j >> 1].x;
  if (ranked) {
    fm1 = forced_slots(nv, cz, fzon, cur >= 1);
    km1 = top_slots(nv, topk, fm1, s1v);
  }
  const bool want_score = score_out != nullptr;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const bool k = (km1 >> j) & 1u;
    const int pos = k ? min(__popc(km1 & ((1u << j) - 1u)), kMaxK) : kMaxK;
    lrow[pos] = 2 * (k2[j >> 1] >> 5) + (j & 1);
    if (want_score) frow[pos] = (ranked & !((fm1 >> j) & 1u)) ? s1v[j] : pos_inf();
  }
  wave_lds_sync();
  if (!live) return;
  const int nk1 = __popc(km1);
  int32_t* orow = idx + u * topk;
  float* srow = want_score ? score_out + u * topk : nullptr;
  int o[kMaxK];
  float f[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    const bool kept = i < nk1;
    o[i] = kept ? lrow[i] : -1;
    f[i] = kept ? frow[i] : neg_inf();
  }
  if (vec_out) {  // K % 4 == 0 and 16-byte aligned outputs
#pragma unroll
    for (int i = 0; i < kMaxK; i += 4) {
      if (i < topk) {
        *reinterpret_cast<int4*>(orow + i) = make_int4(o[i], o[i + 1], o[i + 2], o[i + 3]);
        if (want_score)
          *reinterpret_cast<float4*>(srow + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
      if (i < topk) {
        orow[i] = o[i];
        if (want_score) srow[i] = f[i];
      }
    }
  }
}

}  // namespace lpq
}  // namespace pisa
