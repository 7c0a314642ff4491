// Lane-per-query decision kernels of the two-stage selection (K <= 16).
//
// Every Top-K decision of the descent (PISA reading page §4.2 eq. (5), §03
// keep-all rule, §5.3 forced nodes) is taken by one lane for one query: the
// lane holds its query's candidate list (the children of the nodes it kept
// one level up, at most 2K <= 32 of them, ascending) and ranks the rankable
// ones with a sorting network over packed 32-bit keys in registers.
//
// Rank keys.  A candidate in slot j (slots follow node order) is keyed by its
// score's distance below the best rankable score of the decision, in fixed
// point (rank_key_rel: quantum 2^-12 of the score unit), with 31 - j in the
// low 5 bits.  A larger key ranks first: scores more than 2^-11 units apart
// are ordered by score at any magnitude, equal scores by node index, which is
// the tie rule of the selection (equal scores -> lower index first).
//
// Forced slots.  In causal mode the forced nodes of a level (current path,
// and with forcing the first and previous leaf's ancestors) are always
// candidates, because their parents were forced one level up.  The valid
// candidates are the prefix of the ascending list with nodes <= lim, so the
// current-path node lim is the last valid slot, the previous leaf's ancestor
// is lim or lim - 1 (then the slot before), and node 0 is slot 0.
//
// Stage 1 (levels L..3).  One wavefront owns 64 (query, head) columns.  A
// level's child rows are taken in windows of kDenseRows rows.  In a window
// the workgroup's waves walk together over the 32-row chunks of child rows
// needed by any of their columns: each chunk is loaded once, coalesced, into
// LDS (the next one is in flight in registers meanwhile), and every wave
// computes its logits on the matrix cores (32 rows x 64 columns per step;
// bf16 hi/lo planes of the fp32 summaries times the logit scale in log2
// units, so each product is exact and accumulation is fp32).  While the logits are still in the MFMA register
// layout it forms the log-sum-exp of every sibling pair (eq. (7)), sums the
// group's heads (eq. (11)) and scatters the
// scores of the pairs that are candidates of the column's query into that
// query's slot array.  Candidacy and slot come from a bitmask of the query's
// kept parents in the window: slot = 2 * (#kept parents before) + child, the
// count running on across windows.  With 16 heads per group (4 queries per
// wave) each wave instead packs the union of its queries' kept parents, 8 to
// a 32-row tile, so that its work per level is bounded by 4 K parents (its
// windows are kTileRows long).
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
constexpr int kDenseRows = 2048; // child rows per window of stage 1
constexpr int kMaskWords = kDenseRows / 4 / 32;  // parent bitmask words per query
// Child rows per window with union tiles (few queries per wave: one bitmap per
// wave, a word per lane).
constexpr int kTileRows = 4 * kDenseRows;
constexpr int kTileWords = kTileRows / 4 / 32;
// Per-query LDS arrays are stored slot-major ([slot][query]) so that lanes of
// different queries always touch different banks.

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int piece_t;  // 16 bytes

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

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

// Lane permutations inside a row of 16 lanes as DPP operand modifiers (no
// LDS crossbar): swap neighbours, swap pairs, mirror each half row (i <-> 7 - i),
// mirror the row (i <-> 15 - i).  Applied in this order with a commutative
// operation they combine all lanes of an aligned group of 2, 4, 8 or 16; the
// lanes may associate differently, so for floating-point sums only one lane's
// total should be used.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                             0xf, 0xf, false));
}
constexpr int kDppSwap1 = 0xb1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4e;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
template <int G>
__device__ __forceinline__ float group_add(float v) {
  if (G >= 2) v += dpp_f32<kDppSwap1>(v);
  if (G >= 4) v += dpp_f32<kDppSwap2>(v);
  if (G >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if (G >= 16) v += dpp_f32<kDppMirror>(v);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if (G >= 2) v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  if (G >= 4) v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  if (G >= 8) v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  if (G >= 16) v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}
template <int G>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  if (G >= 2) v |= dpp_u32<kDppSwap1>(v);
  if (G >= 4) v |= dpp_u32<kDppSwap2>(v);
  if (G >= 8) v |= dpp_u32<kDppHalfMirror>(v);
  if (G >= 16) v |= dpp_u32<kDppMirror>(v);
  return v;
}

// Kept slots of a ranked level: the forced ones plus the best K - #F of the
// other valid ones by score s[j].
__device__ __forceinline__ uint32_t top_slots(int n_valid, int topk, uint32_t fm,
                                              const float (&s)[kSlots]) {
  const uint32_t rm = prefix_mask(n_valid) & ~fm;
  const int keep_n = topk - __popc(fm);
  // best rankable score by a tree of maxima (independent steps, not a chain)
  float mv[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) mv[j] = ((rm >> j) & 1u) ? s[j] : neg_inf();
#pragma unroll
  for (int w = kSlots / 2; w >= 1; w /= 2)
#pragma unroll
    for (int j = 0; j < w; ++j) mv[j] = fmaxf(mv[j], mv[j + w]);
  const float smax = mv[0];
  uint32_t key[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) key[j] = ((rm >> j) & 1u) ? rank_key_rel(s[j], smax, j) : 0u;
  sort32_desc(key);
  uint32_t km = fm;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) km |= (i < keep_n) ? (1u << (31 - (key[i] & 31u))) : 0u;
  return km;
}

// Kept slots of a ranked level, decided by the G lanes of one query's group
// (G >= 2: lane sub holds slots sub * S .. sub * S + S - 1, S = 32 / G, scores
// s[i]).  The rank keys are those of top_slots; a bitonic sort of the 32 keys
// runs across the group (compare-exchanges between lanes through xor
// shuffles, inside a lane in registers), leaving rank e at lane e / S,
// element e % S; the kept slots' bits are OR-ed over the group.  The keys are
// distinct, so the kept set equals top_slots'.  Every lane of the group
// returns the same mask.
template <int G>
__device__ __forceinline__ uint32_t top_slots_group(int n_valid, int topk, uint32_t fm,
                                                    const float (&s)[kSlots / G], int sub) {
  constexpr int S = kSlots / G;
  const uint32_t rm = prefix_mask(n_valid) & ~fm;
  const int keep_n = topk - __popc(fm);
  float smax = neg_inf();
#pragma unroll
  for (int i = 0; i < S; ++i) smax = ((rm >> (sub * S + i)) & 1u) ? fmaxf(smax, s[i]) : smax;
  smax = group_max<G>(smax);
  uint32_t key[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int j = sub * S + i;
    key[i] = ((rm >> j) & 1u) ? rank_key_rel(s[i], smax, j) : 0u;
  }
  // Descending bitonic sort over element e = sub * S + i.
#pragma unroll
  for (int k = 2; k <= kSlots; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj < S) {
#pragma unroll
        for (int i = 0; i < S; ++i) {
          if (i & jj) continue;
          const int e = sub * S + i;
          const bool desc = (e & k) == 0;
          const uint32_t a = key[i], b = key[i | jj];
          key[i] = desc ? max(a, b) : min(a, b);
          key[i | jj] = desc ? min(a, b) : max(a, b);
        }
      } else {
#pragma unroll
        for (int i = 0; i < S; ++i) {
          const int e = sub * S + i;
          const uint32_t other = (uint32_t)__shfl_xor((int)key[i], jj / S, kWave);
          const bool keep_max = ((e & jj) == 0) == ((e & k) == 0);
          key[i] = keep_max ? max(key[i], other) : min(key[i], other);
        }
      }
    }
  }
  uint32_t km = fm;
#pragma unroll
  for (int i = 0; i < S; ++i)
    km |= (sub * S + i < keep_n) ? (1u << (31 - (key[i] & 31u))) : 0u;
  km = group_or<G>(km);
  return km;
}

// A query's column of a slot-major LDS array.
template <typename E>
struct Column {
  E* p;
  int stride;
  __device__ __forceinline__ E& operator[](int i) const { return p[i * stride]; }
  __device__ __forceinline__ void set(int i, E v) const { p[i * stride] = v; }
};

// An int column stored as bit patterns in a float array, so that one LDS
// array holds a query's slot scores and, once the decision has read them into
// registers, its kept-node list.
struct IntInFloatColumn {
  float* p;
  int stride;
  __device__ __forceinline__ int get(int i) const { return __float_as_int(p[i * stride]); }
  __device__ __forceinline__ void set(int i, int v) const { p[i * stride] = __int_as_float(v); }
};

// Kept slots -> ascending node list through LDS (kMaxK + 1 entries; entry
// kMaxK takes the stores of slots that are not kept).
template <typename Col, typename NodeOf>
__device__ __forceinline__ void compact_kept(uint32_t km, Col row, NodeOf node_of) {
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const bool k = (km >> j) & 1u;
    const int pos = __popc(km & ((1u << j) - 1u));
    row.set(k ? min(pos, kMaxK) : kMaxK, node_of(j));
  }
}

// Split fp32 pyramid values, times mul (the logit scale in log2 units, so
// that stage 1's products come out as log2-unit logits), into bf16 hi/lo
// planes: mul x = hi + lo + r with |r| <= 2^-16 |mul x|, so that a bf16 MFMA
// over both planes reproduces an fp32 dot product to that accuracy.  Stage 1
// reads child rows of levels 2 and up only, so each head's level 1 (its first
// skip_rows rows of row_len values) is left out; 8 values per thread and step.
__global__ void split_planes_kernel(const float* __restrict__ pyr, bf16_t* __restrict__ hi,
                                    bf16_t* __restrict__ lo, int heads, size_t head_len,
                                    size_t skip, float mul) {
  const size_t per_head = (head_len - skip) / 8;  // 8-value groups split per head
  const size_t n = per_head * heads;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t e = (i / per_head) * head_len + skip + 8 * (i % per_head);
    const float4 x0 = *reinterpret_cast<const float4*>(pyr + e);
    const float4 x1 = *reinterpret_cast<const float4*>(pyr + e + 4);
    const float x[8] = {x0.x * mul, x0.y * mul, x0.z * mul, x0.w * mul,
                        x1.x * mul, x1.y * mul, x1.z * mul, x1.w * mul};
    uint32_t h2[4], l2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t ha = f32_to_bf16(x[2 * j]), hb = f32_to_bf16(x[2 * j + 1]);
      const uint16_t la = f32_to_bf16(x[2 * j] - bf16_to_f32(ha));
      const uint16_t lb = f32_to_bf16(x[2 * j + 1] - bf16_to_f32(hb));
      h2[j] = uint32_t(ha) | (uint32_t(hb) << 16);
      l2[j] = uint32_t(la) | (uint32_t(lb) << 16);
    }
    *reinterpret_cast<uint4*>(hi + e) = make_uint4(h2[0], h2[1], h2[2], h2[3]);
    *reinterpret_cast<uint4*>(lo + e) = make_uint4(l2[0], l2[1], l2[2], l2[3]);
  }
}

// ---------------------------------------------------------------------------
// Stage 1
// ---------------------------------------------------------------------------

// Two workgroups per CU; three when a query spans several lanes at d = 64,
// where the kernel then fits 168 VGPRs (at d = 128 the spills cost more than
// the third workgroup gains).
template <int D, int G>
__global__ __launch_bounds__(kWaves * kWave, (G >= 2 && D == 64) ? 3 : 2) void stage1_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ phi, const bf16_t* __restrict__ plo,
    int* __restrict__ s1_nodes, int heads_q, int heads_kv,
    int n_tok, int block, int topk, int causal, int force, LevelTable lv, int split_level,
    int tile_rows) {
  constexpr int T = kWave / G;  // queries per wave
  constexpr int KSTEPS = D / 16;
  // With 8 or more queries per wave the waves of a workgroup need nearly the
  // same chunks, and sharing their loads pays; with 4 (G = 16) each wave
  // needs under half of the workgroup's chunks, and independent waves are
  // faster.
  constexpr bool kShared = T >= 8;
  // Summary chunk shared by the workgroup's waves: 32 rows of the hi plane,
  // then the same 32 rows of the lo plane, each row padded by 16 bytes.
  constexpr int CROW = D + 8;
  constexpr int CPIECES = 2 * 32 * D / 8;  // 16-byte pieces of a chunk
  constexpr int CLOADS = CPIECES / (kWaves * kWave);
  static_assert(CPIECES % (kWaves * kWave) == 0, "chunk pieces per thread");
  // score_s holds a query's slot scores and, after its decision has read
  // them, its kept-node list (int bit patterns in rows 0..kMaxK).  Rows
  // kSlots and kSlots + 1 take the stores of positions that are no candidate.
  __shared__ float score_s[kWaves][kSlots + 2][T];
  __shared__ uint32_t mask_s[kWaves][kShared ? kMaskWords : 1][T];
  __shared__ __align__(16) bf16_t chunk_s[kShared ? 2 * 32 * CROW : 8];
  __shared__ uint32_t chunks_s[2][kWaves][2];
  // The union of a wave's kept parents, as a bitmap and as an ascending list
  // (few queries per wave only).
  __shared__ uint32_t umask_s[kWaves][kShared ? 1 : kTileWords];
  __shared__ int ulist_s[kWaves][kShared ? 1 : kWave];
  // Kept-node lists when a query spans several lanes.
  __shared__ int kp_s[kWaves][kMaxK][G == 1 ? 1 : T];

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  // A causal query's dense work grows with t: workgroups are dispatched in
  // linear order, so the latest positions of every head go first.
  const unsigned lin = blockIdx.x + blockIdx.y * gridDim.x;
  const int bh = (int)(lin % gridDim.y);
  const int bx = (int)(gridDim.x - 1 - lin / gridDim.y);
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  // Waves past the sequence end take part in the workgroup's chunk loads and
  // barriers with no live query.
  const int t0 = (bx * kWaves + wave) * T;
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
  const int ql = lane < T ? lane : 0;
  // The query's kept nodes one level up, ascending: in registers when every
  // lane holds a query (G = 1), else in the query's LDS column (lanes >= T
  // read query 0's and write nothing).
  int kp_r[G == 1 ? kMaxK : 1];
  auto kp = [&](int i) __attribute__((always_inline)) -> int {
    if constexpr (G == 1)
      return kp_r[i];
    else
      return kp_s[wave][i][ql];
  };
  auto kp_put = [&](int i, int v) __attribute__((always_inline)) {
    if constexpr (G == 1)
      kp_r[i] = v;
    else if (lane < T)
      kp_s[wave][i][ql] = v;
  };
  int nk = 1;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) kp_put(i, 0);
  wave_lds_sync();
  const Column<float> srow{&score_s[wave][0][ql], T};
  const IntInFloatColumn lrow{&score_s[wave][0][ql], T};
  const Column<uint32_t> mrow{&mask_s[wave][0][ql], T};

  int phase = 0;  // windows so far (parity selects the chunk-bits buffer)
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
      const int c = 2 * kp(i);
      n_valid += (i < nk) ? int(c <= x_max) + int(c + 1 <= x_max) : 0;
    }
    if (!dlane) n_valid = 0;
    const bool need = n_valid > topk;
    const int m_child = lv.size[l - 2];
    const size_t child0 = head_rows + lv.off[l - 2];

    // The candidates' children are scored in windows of kDenseRows child
    // rows (kTileRows with union tiles) w0 .. (parents pw = w0 / 4 onwards),
    // in ascending order, so that a query's slot base runs on from one window
    // to the next and its slots come out as from one pass over the level.
    int base[2] = {0, 0};
    auto window = [&](const int w0) __attribute__((always_inline)) {
      const int pw = w0 >> 2;
      if constexpr (kShared) {
        // The window's parent bitmask: the query's kept nodes one level up.
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) mrow[w] = 0u;
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) {
          const int p = kp(i) - pw;
          if (dlane & (i < nk) & (p >= 0) & (p < 32 * kMaskWords))
            atomicOr(&mrow[p >> 5], 1u << (p & 31));
        }
        wave_lds_sync();
        // Chunk c holds child rows w0 + 32c .. w0 + 32c + 31, whose parents
        // pw + 8c .. pw + 8c + 7 are byte c of the parent masks.  The workgroup
        // scores every chunk that holds a kept parent of one of its ranking
        // queries, all waves together.
        uint32_t cw[2] = {0u, 0u};
        if (need) {
#pragma unroll
          for (int w = 0; w < kMaskWords; ++w) {
            const uint32_t word = mrow[w];
            // bit 8j + 7 set iff byte j is nonzero, then the four flags packed
            // into bits 0..3
            const uint32_t f = (((word & 0x7f7f7f7fu) + 0x7f7f7f7fu) | word) & 0x80808080u;
            const uint32_t y = f >> 7;
            const uint32_t nib = (y | (y >> 7) | (y >> 14) | (y >> 21)) & 0xfu;
            cw[w >> 3] |= nib << (4 * (w & 7));
          }
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          cw[0] |= __shfl_xor(cw[0], o, kWave);
          cw[1] |= __shfl_xor(cw[1], o, kWave);
        }
        if (lane == 0) {
          chunks_s[phase & 1][wave][0] = cw[0];
          chunks_s[phase & 1][wave][1] = cw[1];
        }
        lds_barrier();
        uint32_t todo[2] = {0u, 0u};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          todo[0] |= chunks_s[phase & 1][w][0];
          todo[1] |= chunks_s[phase & 1][w][1];
        }
        todo[0] = __builtin_amdgcn_readfirstlane(todo[0]);
        todo[1] = __builtin_amdgcn_readfirstlane(todo[1]);

        if ((todo[0] | todo[1]) != 0u) {
          // Pop the lowest pending chunk (the masks are nonzero).
          auto pop = [&]() __attribute__((always_inline)) {
            int c;
            if (todo[0] != 0u) {
              c = __builtin_ctz(todo[0]);
              todo[0] &= todo[0] - 1u;
            } else {
              c = 32 + __builtin_ctz(todo[1]);
              todo[1] &= todo[1] - 1u;
            }
            return c;
          };
          // This thread's pieces of a chunk: piece p = tid + 256 i is plane
          // p / (32 D / 8), row (p / (D / 8)) % 32, 16-byte column p % (D / 8).
          // Rows past the level end repeat its last row (see the ragged-chunk
          // masking of the pickup).
          piece_t stage[CLOADS];
          auto fetch = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < CLOADS; ++i) {
              const int p = threadIdx.x + i * kWaves * kWave;
              const int plane = p / (32 * D / 8), row = (p / (D / 8)) % 32, c8 = p % (D / 8);
              const bf16_t* src = plane ? plo : phi;
              stage[i] = *reinterpret_cast<const piece_t*>(
                  src + (child0 + min(r0 + row, m_child - 1)) * D + 8 * c8);
            }
          };
          auto put = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < CLOADS; ++i) {
              const int p = threadIdx.x + i * kWaves * kWave;
              const int plane = p / (32 * D / 8), row = (p / (D / 8)) % 32, c8 = p % (D / 8);
              *reinterpret_cast<piece_t*>(chunk_s + (plane * 32 + row) * CROW + 8 * c8) = stage[i];
            }
          };
          const Column<uint32_t> mcol[2] = {{&mask_s[wave][0][(32 * 0 + col) / G], T},
                                            {&mask_s[wave][0][(32 * 1 + col) / G], T}};
          const Column<float> scol[2] = {{&score_s[wave][0][(32 * 0 + col) / G], T},
                                         {&score_s[wave][0][(32 * 1 + col) / G], T}};
          const bool writer = (col % G) == 0;
          // One chunk: S = summaries x queries on MFMA from the LDS chunk, then
          // the candidates' LSEs picked up into the slot arrays.  byte[cb]: the
          // column's kept parents among the chunk's 8.
          auto chunk = [&](int r0, const uint32_t (&byte)[2]) __attribute__((always_inline)) {
            // Rows of this chunk: r0 + 8g + 4kh + i%4 (acc element 4g + i%4);
            // level-l candidates n = r0/2 + 4g + 2kh + m own rows 2n, 2n+1;
            // their parents p = r0/4 + 2g + kh (bits p0..p0+7 of the masks).
            const bf16_t* arow = chunk_s + col * CROW + 8 * kh;
            f32x16_t acc[2] = {};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
              const uint4 hv = *reinterpret_cast<const uint4*>(arow + 16 * s);
              const uint4 lo = *reinterpret_cast<const uint4*>(arow + 32 * CROW + 16 * s);
#pragma unroll
              for (int cb = 0; cb < 2; ++cb) {
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lo), bq[cb][s],
                                                                  acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(hv), bq[cb][s],
                                                                  acc[cb], 0, 0, 0);
              }
            }
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
                    // the planes carry scale * log2(e) already: logits in
                    // log2 units; -|z0 - z1| folds into the exp's input
                    // modifiers
                    const float mx = fmaxf(z0, z1);
                    float v = mx + fast_log2(1.f + fast_exp2(-fabsf(z0 - z1)));
                    v = group_add<G>(v);  // the writer lane's total is stored
                    if constexpr (kFull)  // both children exist: one row select per pair
                      scol[cb][(has ? 2 * pslot : kSlots) + m] = v;
                    else
                      scol[cb][w ? 2 * pslot + m : kSlots] = v;
                  }
                }
              }
            };
            if (r0 + 32 <= m_child)
              pickup(std::true_type{});
            else
              pickup(std::false_type{});
          };
          // The next chunk's pieces are in flight while this one is scored.
          int c = pop();
          fetch(w0 + 32 * c);
          for (;;) {
            const bool more = (todo[0] | todo[1]) != 0u;
            const int cn = more ? pop() : c;
            wait_vmcnt<0>();
            lds_barrier();  // every wave has read the previous chunk
            put();
            if (more) fetch(w0 + 32 * cn);
            lds_barrier();  // this chunk is in LDS
            // A wave none of whose columns keeps a parent here (large groups:
            // few queries per wave) takes part in the loads only.  Parents in
            // chunks skipped by the workgroup are no kept parents of a ranking
            // query, so the slot bases of those queries stay exact.
            const int p0 = 8 * c;
            uint32_t byte[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) byte[cb] = (mcol[cb][p0 >> 5] >> (p0 & 31)) & 0xffu;
            if (__ballot((byte[0] | byte[1]) != 0u) != 0) chunk(w0 + 32 * c, byte);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) base[cb] += __popc(byte[cb]);
            if (!more) break;
            c = cn;
          }
        }
      } else {
        // Few queries per wave (T = 64 / G <= 4): the wave scores only the
        // union of its ranking queries' kept parents, 8 parents to a 32-row
        // MFMA tile (a parent's 4 grandchild rows are its two candidates'
        // children), so a level costs it at most T K / 8 tiles whatever the
        // level's size.  The parents are tiled in ascending order, so a
        // query's slot base advances over its own kept parents in the same
        // order as over the level's rows.
        static_assert(T * kMaxK <= kWave && kTileWords == kWave, "union of kept parents");
        const uint32_t needers = (uint32_t)__ballot(need);  // query qi is lane qi
        if (needers != 0u) {
          // Bitmap of the union of the ranking queries' kept parents in the
          // window: lane x then holds parents pw + 32x .. pw + 32x + 31.
          umask_s[wave][lane] = 0u;
          wave_lds_sync();
#pragma unroll
          for (int i = 0; i < kMaxK; ++i) {
            const int p = kp(i) - pw;
            if (need & (i < nk) & (p >= 0) & (p < (tile_rows >> 2)))
              atomicOr(&umask_s[wave][p >> 5], 1u << (p & 31));
          }
          wave_lds_sync();
          const uint32_t ub = umask_s[wave][lane];
          // Union rank of lane x's first parent (exclusive prefix of the
          // popcounts); the ascending union list.
          const int cnt = __popc(ub);
          int incl = cnt;
#pragma unroll
          for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o, kWave);
            incl += lane >= o ? y : 0;
          }
          const int rbase = incl - cnt;
          const int n_union = __builtin_amdgcn_readlane(incl, kWave - 1);
          for (uint32_t bits = ub, o = rbase; bits != 0u; bits &= bits - 1u, ++o)
            ulist_s[wave][o] = pw + 32 * lane + __builtin_ctz(bits);
          // A ranking query's kept parents as bits of their union ranks (its
          // decision lane; at most 64 ranks).
          uint32_t ur_lo = 0u, ur_hi = 0u;
#pragma unroll
          for (int i = 0; i < kMaxK; ++i) {
            const int p = kp(i) - pw;  // in the window: 0 .. tile_rows / 4 - 1
            const bool in = (p >= 0) & (p < (tile_rows >> 2));
            const int x = (p >> 5) & (kWave - 1);
            const int rb = __shfl(rbase, x, kWave);
            const uint32_t bb = (uint32_t)__shfl((int)ub, x, kWave);
            const int r = rb + __popc(bb & ((1u << (p & 31)) - 1u));
            const uint32_t bit = (need && i < nk && in) ? 1u << (r & 31) : 0u;
            ur_lo |= r < 32 ? bit : 0u;
            ur_hi |= r < 32 ? 0u : bit;
          }
          wave_lds_sync();  // the union list is complete
          // Column c = 32 cb + col belongs to query c / G.
          uint32_t ur[2][2];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const int qc = (32 * cb + col) / G;
            ur[cb][0] = (uint32_t)__shfl((int)ur_lo, qc, kWave);
            ur[cb][1] = (uint32_t)__shfl((int)ur_hi, qc, kWave);
          }
          const Column<float> scol[2] = {{&score_s[wave][0][(32 * 0 + col) / G], T},
                                         {&score_s[wave][0][(32 * 1 + col) / G], T}};
          const bool writer = (col % G) == 0;
          const int n_tiles = (n_union + 7) >> 3;
          for (int tt = 0; tt < n_tiles; ++tt) {
            // Tile row col: union parent 8 tt + col / 4 (past the union's end
            // its last parent, which no column keeps here), child row
            // 4 p + col % 4 (rows past the level end repeat its last row;
            // their logits are masked below).
            const int pr = ulist_s[wave][min(8 * tt + (col >> 2), n_union - 1)];
            const int r = min(4 * pr + (col & 3), m_child - 1);
            const bf16_t* hrow = phi + (child0 + r) * D + 8 * kh;
            const bf16_t* lrow2 = plo + (child0 + r) * D + 8 * kh;
            uint4 hv[KSTEPS], lv4[KSTEPS];
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
              hv[s] = *reinterpret_cast<const uint4*>(hrow + 16 * s);
              lv4[s] = *reinterpret_cast<const uint4*>(lrow2 + 16 * s);
            }
            // The tile's last parent is its largest.
            const int pmax = ulist_s[wave][min(8 * tt + 7, n_union - 1)];
            uint32_t byte[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              byte[cb] = (((tt >> 2) ? ur[cb][1] : ur[cb][0]) >> (8 * (tt & 3))) & 0xffu;
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
            // Lane rows 8g + 4kh + i%4 (acc element 4g + i%4) belong to tile
            // parent pb = 2g + kh, fetched by lane 4 pb; candidate m = 0, 1
            // of that parent owns its rows 2m, 2m + 1.
            auto pickup = [&](auto full_tag) {
              constexpr bool kFull = decltype(full_tag)::value;  // every row of the tile exists
#pragma unroll
              for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  const int pb = 2 * g + kh;
                  const bool has = writer & ((byte[cb] >> pb) & 1u);
                  const int pslot = base[cb] + __popc(byte[cb] & ((1u << pb) - 1u));
                  const int pp = kFull ? 0 : __shfl(pr, 4 * pb, kWave);
#pragma unroll
                  for (int m = 0; m < 2; ++m) {
                    const int n = 2 * pp + m;
                    const float z0 = acc[cb][4 * g + 2 * m];
                    float z1 = acc[cb][4 * g + 2 * m + 1];
                    bool w = has;
                    if (!kFull) {
                      z1 = 2 * n + 1 < m_child ? z1 : neg_inf();
                      w &= 2 * n < m_child;
                    }
                    // the planes carry scale * log2(e) already: logits in
                    // log2 units; -|z0 - z1| folds into the exp's input
                    // modifiers
                    const float mx = fmaxf(z0, z1);
                    float v = mx + fast_log2(1.f + fast_exp2(-fabsf(z0 - z1)));
                    v = group_add<G>(v);  // the writer lane's total is stored
                    if constexpr (kFull)  // both children exist: one row select per pair
                      scol[cb][(has ? 2 * pslot : kSlots) + m] = v;
                    else
                      scol[cb][w ? 2 * pslot + m : kSlots] = v;
                  }
                }
                base[cb] += __popc(byte[cb]);
              }
            };
            if (4 * pmax + 4 <= m_child)
              pickup(std::true_type{});
            else
              pickup(std::false_type{});
          }
        }
      }
      wave_lds_sync();
      ++phase;
    };
    // A level within one window (every level up to 256K tokens at C = 64)
    // runs a copy of the window code compiled for w0 = 0.
    if (size_l > topk) {
      // tile_rows: a multiple of 64 up to kTileRows (the union bitmap's span)
      const int win = kShared ? kDenseRows : tile_rows;
      if (m_child <= win) {
        window(0);
      } else {
        for (int w0 = 0; w0 < m_child; w0 += win) window(w0);
      }
    }

    // Decision for this lane's query.
    uint32_t km = prefix_mask(n_valid);
    if constexpr (G == 1) {
      if (need) {
        float sc[kSlots];
#pragma unroll
        for (int j = 0; j < kSlots; ++j) sc[j] = srow[j];
        const bool prev_distinct = cur >= 1 && ((cur - 1) >> sh) != lim;
        km = top_slots(n_valid, topk, forced_slots(n_valid, cz, fzon, prev_distinct), sc);
      }
    } else {
      // T = 64 / G queries per wave: query qd is decided by lanes qd G ..
      // qd G + G - 1 together instead of by lane qd alone.
      const bool prev_distinct = cur >= 1 && ((cur - 1) >> sh) != lim;
      const uint32_t fm = need ? forced_slots(n_valid, cz, fzon, prev_distinct) : 0u;
      const int qd = lane / G, sub = lane % G;
      const int nv_g = __shfl(n_valid, qd, kWave);
      const uint32_t fm_g = (uint32_t)__shfl((int)fm, qd, kWave);
      uint32_t km_g = 0u;
      if (__ballot(nv_g > topk) != 0) {
        float s_loc[kSlots / G];
#pragma unroll
        for (int i = 0; i < kSlots / G; ++i) s_loc[i] = score_s[wave][sub * (kSlots / G) + i][qd];
        km_g = top_slots_group<G>(nv_g, topk, fm_g, s_loc, sub);
      }
      const uint32_t kq = (uint32_t)__shfl((int)km_g, lane < T ? lane * G : 0, kWave);
      if (need) km = kq;
    }
    wave_lds_sync();
    compact_kept(km, lrow, [&](int j) { return 2 * kp(j >> 1) + (j & 1); });
    wave_lds_sync();
    nk = __popc(km);
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) kp_put(i, lrow.get(i));
    if (l == split_level) break;
    wave_lds_sync();
  }
  if (dlane) {
    int* out = s1_nodes + ((size_t)bh * n_tok + t) * topk;
    if ((topk & 3) == 0) {
#pragma unroll
      for (int i = 0; i < kMaxK; i += 4)
        if (i < topk)
          *reinterpret_cast<int4*>(out + i) =
              make_int4(i < nk ? kp(i) : -1, i + 1 < nk ? kp(i + 1) : -1,
                        i + 2 < nk ? kp(i + 2) : -1, i + 3 < nk ? kp(i + 3) : -1);
    } else {
#pragma unroll
      for (int i = 0; i < kMaxK; ++i)
        if (i < topk) out[i] = i < nk ? kp(i) : -1;
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
