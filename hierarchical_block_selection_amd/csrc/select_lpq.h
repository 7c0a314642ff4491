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

#include "pisa_common.h"

namespace pisa {
namespace lpq {

constexpr int kSlots = 32;       // 2K candidates, K <= 16
constexpr int kMaxK = 16;
constexpr int kWaves = 4;        // independent wavefronts per workgroup
constexpr int kDenseRows = 2048; // child rows scored densely
constexpr int kMaskWords = kDenseRows / 4 / 32;  // parent bitmask words per query
constexpr int kScoreRow = 36;    // floats per query of the slot array (16-byte rows)
constexpr int kListRow = 20;     // ints per query of the kept-list staging (16 + trash)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Order-preserving image of a float (larger float -> larger unsigned).
__device__ __forceinline__ uint32_t ordered_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
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

// Forced-node test of §5.3 at a level with shift sh (current-path node always;
// first and previous leaf's ancestors when forcing is on).
struct Forced {
  int lim, prev;  // prev < 0: no previous leaf
  bool causal, force;
  __device__ __forceinline__ bool operator()(int node) const {
    return causal & ((node == lim) | (force & ((node == 0) | (node == prev))));
  }
};

// One decision over candidate slots 0..n_valid-1 (ascending nodes c(j)).
// score_of(j) is read only when ranking is needed.  Returns the mask of kept
// slots.
template <typename NodeOf, typename ScoreOf>
__device__ __forceinline__ uint32_t decide(int n_valid, int topk, const Forced& fz,
                                           NodeOf node_of, ScoreOf score_of) {
  const uint32_t vm = n_valid >= 32 ? 0xffffffffu : ((1u << n_valid) - 1u);
  if (n_valid <= topk) return vm;
  uint32_t fm = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) fm |= (fz(node_of(j)) ? (1u << j) : 0u);
  fm &= vm;
  const int keep_n = topk - __popc(fm);
  const uint32_t rm = vm & ~fm;
  uint32_t key[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) key[j] = ((rm >> j) & 1u) ? rank_key(score_of(j), j) : 0u;
  sort32_desc(key);
  uint32_t km = fm;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i)
    km |= (i < keep_n) ? (1u << (31 - (key[i] & 31u))) : 0u;
  return km;
}

// Kept slots -> ascending node list through LDS (row of kListRow ints; slot
// kMaxK of the row takes the stores of slots that are not kept).
template <typename NodeOf>
__device__ __forceinline__ void compact_kept(uint32_t km, int* row, NodeOf node_of) {
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
  __shared__ __attribute__((aligned(16))) float score_s[kWaves][T][kScoreRow];
  __shared__ __attribute__((aligned(16))) uint32_t mask_s[kWaves][T][kMaskWords];
  __shared__ __attribute__((aligned(16))) int list_s[kWaves][T][kListRow];

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int bh = blockIdx.y;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int t0 = (blockIdx.x * kWaves + wave) * T;
  if (t0 >= n_tok) return;
  const bool cz = causal != 0, fzon = force != 0;
  const size_t head_rows = (size_t)bh * lv.rows;

  // MFMA layout: this lane feeds columns col and 32 + col, k half kh.
  const int col = lane & 31, kh = lane >> 5;
  bf16x8_t bq[2][KSTEPS];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = 32 * cb + col;
    const int t = t0 + c / G;
    const bool ok = t < n_tok;
    const bf16_t* qrow =
        q + (((size_t)b * heads_q + (size_t)kvh * G + c % G) * n_tok + (ok ? t : 0)) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      bq[cb][s] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * kh)
                               : make_uint4(0, 0, 0, 0));
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
  float* srow = &score_s[wave][lane < T ? lane : 0][0];
  int* lrow = &list_s[wave][lane < T ? lane : 0][0];
  uint32_t* mrow = &mask_s[wave][lane < T ? lane : 0][0];

  for (int l = lv.n; l >= split_level; --l) {
    const int sh = l - 1;
    const int size_l = lv.size[l - 1];
    const int lim = cz ? (cur >> sh) : size_l - 1;
    // Candidates: children of the kept nodes, ascending; the valid ones
    // (existing, not in the future) form a prefix of the list.
    int n_valid = 0;
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int c = 2 * kp[j >> 1] + (j & 1);
      n_valid += (((j >> 1) < nk) & (c < size_l) & (c <= lim)) ? 1 : 0;
    }
    if (!dlane) n_valid = 0;
    const bool need = n_valid > topk;
    const bool any_need = __ballot(need) != 0;

    if (any_need) {
      const int m_child = lv.size[l - 2];
      const size_t child0 = head_rows + lv.off[l - 2];
      if (m_child <= kDenseRows) {
        // Parent masks were written after the previous level's decision.
        const int lim_last = cz ? (cur_last >> sh) : size_l - 1;
        const int rows_needed = min(m_child, 2 * lim_last + 2);
        int base[2] = {0, 0};
        const uint32_t* mcol[2] = {&mask_s[wave][(32 * 0 + col) / G][0],
                                   &mask_s[wave][(32 * 1 + col) / G][0]};
        float* scol[2] = {&score_s[wave][(32 * 0 + col) / G][0],
                          &score_s[wave][(32 * 1 + col) / G][0]};
        const bool writer = (col % G) == 0;
        for (int r0 = 0; r0 < rows_needed; r0 += 32) {
          const int r = r0 + col;
          const bool ok = r < m_child;
          const bf16_t* hrow = phi + (child0 + (ok ? r : 0)) * D + 8 * kh;
          const bf16_t* lrow2 = plo + (child0 + (ok ? r : 0)) * D + 8 * kh;
          f32x16_t acc[2] = {};
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
            const uint4 hv = ok ? *reinterpret_cast<const uint4*>(hrow + 16 * s) : make_uint4(0, 0, 0, 0);
            const uint4 lv4 = ok ? *reinterpret_cast<const uint4*>(lrow2 + 16 * s) : make_uint4(0, 0, 0, 0);
            const bf16x8_t ah = as_bf16x8(hv), al = as_bf16x8(lv4);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bq[cb][s], acc[cb], 0, 0, 0);
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bq[cb][s], acc[cb], 0, 0, 0);
            }
          }
          // Rows of this chunk: r0 + 8g + 4kh + i%4 (acc element 4g + i%4);
          // level-l candidates n = r0/2 + 4g + 2kh + m own rows 2n, 2n+1;
          // their parents p = r0/4 + 2g + kh.
          const int p0 = r0 >> 2;  // multiple of 8
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const uint32_t byte = (mcol[cb][p0 >> 5] >> (p0 & 31)) & 0xffu;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int pb = 2 * g + kh;
              const bool has = (byte >> pb) & 1u;
              const int pslot = base[cb] + __popc(byte & ((1u << pb) - 1u));
#pragma unroll
              for (int m = 0; m < 2; ++m) {
                const int n = (r0 >> 1) + 4 * g + 2 * kh + m;
                const float z0 = acc[cb][4 * g + 2 * m] * scale_log2;
                const float z1 = acc[cb][4 * g + 2 * m + 1] * scale_log2;
                const bool has1 = 2 * n + 1 < m_child;
                const float mx = has1 ? fmaxf(z0, z1) : z0;
                const float mn = has1 ? fminf(z0, z1) : neg_inf();
                float v = mx + fast_log2(1.f + fast_exp2(mn - mx));
                if (G >= 2) v += __shfl_xor(v, 1, kWave);
                if (G >= 4) v += __shfl_xor(v, 2, kWave);
                const int slot = 2 * pslot + m;
                const bool w = writer & has & (2 * n < m_child) & (slot < kSlots);
                scol[cb][w ? slot : kSlots] = v;
              }
            }
            base[cb] += __popc(byte);
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
          const int par = list_s[wave][qi][j >> 1];
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
          if ((lane & 1) == 0) score_s[wave][qi][live ? j : kSlots] = tot;
        }
      }
      wave_lds_sync();
    }

    // Decision for this lane's query.
    const Forced fz{lim, (cz && fzon && cur >= 1) ? ((cur - 1) >> sh) : -1, cz, fzon};
    auto node_of = [&](int j) { return 2 * kp[j >> 1] + (j & 1); };
    auto score_of = [&](int j) { return srow[j]; };
    const uint32_t km = dlane ? decide(n_valid, topk, fz, node_of, score_of) : 0u;
    compact_kept(km, lrow, node_of);
    wave_lds_sync();
    nk = __popc(km);
#pragma unroll
    for (int i = 0; i < kMaxK; i += 4) {
      const int4 v = *reinterpret_cast<const int4*>(lrow + i);
      kp[i] = v.x; kp[i + 1] = v.y; kp[i + 2] = v.z; kp[i + 3] = v.w;
    }
    if (l == split_level) break;
    // Parent bitmask for the next level's dense pass (kept nodes of level l).
    const int nl = l - 1;
    if (lv.size[nl - 1] > topk && lv.size[nl - 2] <= kDenseRows) {
#pragma unroll
      for (int w = 0; w < kMaskWords; w += 4)
        *reinterpret_cast<uint4*>(mrow + w) = make_uint4(0, 0, 0, 0);
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < kMaxK; ++i)
        if (dlane & (i < nk)) atomicOr(mrow + (kp[i] >> 5), 1u << (kp[i] & 31));
    }
    wave_lds_sync();
  }
  if (dlane) {
    int* out = s1_nodes + ((size_t)bh * n_tok + t) * topk;
#pragma unroll
    for (int i = 0; i < kMaxK; ++i)
      if (i < topk) out[i] = i < nk ? kp[i] : -1;
  }
}

// ---------------------------------------------------------------------------
// Final decisions at levels 2 and 1
// ---------------------------------------------------------------------------

// scores[(u*K + slot)*stride + j]: j = 0..3 exact LSE of leaf 4n + j, j = 4, 5
// level-2 score of child 2n + (j - 4), for the slot's level-3 node n (nats).
template <int STRIDE>
__global__ __launch_bounds__(kWaves * kWave) void final_kernel(
    const int* __restrict__ s1_nodes, const float* __restrict__ scores, int32_t* __restrict__ idx,
    float* __restrict__ score_out, int n_tok, int block, int topk, int causal, int force, int m1,
    int m2) {
  __shared__ __attribute__((aligned(16))) int list_s[kWaves][kWave][kListRow];
  __shared__ __attribute__((aligned(16))) float out_s[kWaves][kWave][kListRow];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int t = (blockIdx.x * kWaves + wave) * kWave + lane;
  const bool live = t < n_tok;
  const int bh = blockIdx.y;
  const size_t u = (size_t)bh * n_tok + (live ? t : 0);
  const bool cz = causal != 0, fzon = force != 0;
  const int cur = live ? t / block : 0;
  int* lrow = &list_s[wave][lane][0];
  float* frow = &out_s[wave][lane][0];
  const float* sc = scores + u * topk * STRIDE;

  int n3[kMaxK];
  int nk3 = 0;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    n3[i] = (i < topk && live) ? s1_nodes[u * topk + i] : -1;
    nk3 += n3[i] >= 0 ? 1 : 0;
  }
  // Level 2: candidate j = child (j & 1) of level-3 node n3[j >> 1]; its score
  // sits in the slot j >> 1 of the stage-2 output.
  int lim = cz ? (cur >> 1) : m2 - 1;
  int nv = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int c = 2 * n3[j >> 1] + (j & 1);
    nv += (((j >> 1) < nk3) & (c < m2) & (c <= lim)) ? 1 : 0;
  }
  if (!live) nv = 0;
  Forced fz{lim, (cz && fzon && cur >= 1) ? ((cur - 1) >> 1) : -1, cz, fzon};
  auto node2 = [&](int j) { return 2 * n3[j >> 1] + (j & 1); };
  // (slot indices are clamped so that unused list entries never read past
  // this query's K slots)
  auto score2 = [&](int j) { return sc[min(j >> 1, topk - 1) * STRIDE + 4 + (j & 1)]; };
  const uint32_t km2 = decide(nv, topk, fz, node2, score2);
  // Kept level-2 candidates, ascending, as (node << 5) | j.
  compact_kept(km2, lrow, [&](int j) { return (node2(j) << 5) | j; });
  wave_lds_sync();
  const int nk2 = __popc(km2);
  int k2[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; i += 4) {
    const int4 v = *reinterpret_cast<const int4*>(lrow + i);
    k2[i] = v.x; k2[i + 1] = v.y; k2[i + 2] = v.z; k2[i + 3] = v.w;
  }
  wave_lds_sync();
  // Level 1: candidate j = leaf (j & 1) of the kept level-2 node k2[j >> 1];
  // its exact LSE sits in slot (j2 >> 1), entry 2 * (j2 & 1) + (j & 1).
  lim = cz ? cur : m1 - 1;
  auto node1 = [&](int j) { return 2 * (k2[j >> 1] >> 5) + (j & 1); };
  auto score1 = [&](int j) {
    const int j2 = k2[j >> 1] & 31;
    return sc[min(j2 >> 1, topk - 1) * STRIDE + 2 * (j2 & 1) + (j & 1)];
  };
  nv = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int c = node1(j);
    nv += (((j >> 1) < nk2) & (c < m1) & (c <= lim)) ? 1 : 0;
  }
  if (!live) nv = 0;
  fz = Forced{lim, (cz && fzon && cur >= 1) ? (cur - 1) : -1, cz, fzon};
  const bool ranked = nv > topk;
  const uint32_t km1 = decide(nv, topk, fz, node1, score1);
  const bool want_score = score_out != nullptr;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const bool k = (km1 >> j) & 1u;
    const int pos = k ? min(__popc(km1 & ((1u << j) - 1u)), kMaxK) : kMaxK;
    const int node = node1(j);
    lrow[pos] = node;
    if (want_score) frow[pos] = (ranked & !fz(node)) ? score1(j) : pos_inf();
  }
  wave_lds_sync();
  if (!live) return;
  const int nk1 = __popc(km1);
  int32_t* orow = idx + u * topk;
  float* srow = want_score ? score_out + u * topk : nullptr;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    if (i < topk) {
      const bool kept = i < nk1;
      orow[i] = kept ? lrow[i] : -1;
      if (want_score) srow[i] = kept ? frow[i] : neg_inf();
    }
  }
}

}  // namespace lpq
}  // namespace pisa
