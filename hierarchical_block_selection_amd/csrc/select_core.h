// Per-query coarse-to-fine descent run by one wavefront.
//
// PISA reading page §4.2 eqs. (5), (6): candidates A^(l) are at most gK = 2K
// <= 64 nodes, so lane j of the wave owns candidate j.  At every level the
// wave drops nodes entirely after the current leaf, keeps every candidate if
// at most K remain (§03), otherwise keeps the forced nodes (§5.3) plus the
// best K-#F others by eq. (11)'s sum over the group's heads of eq. (7)'s LSE
// (ties to the lower node index), and expands the kept nodes into their
// children with a ballot/prefix-count compaction through a 64-entry LDS list.
//
// Intermediate levels: each lane scores its own node from the node's two
// child summaries (fp32 pyramid rows) against the group's queries staged in
// LDS.  Leaf level: for each rankable candidate the whole wave computes the
// exact LSE over the leaf's C <= 64 raw keys, one key per lane.
#pragma once

#include "pisa_common.h"

namespace pisa {

struct SelectResult {
  int node;     // this lane's final leaf (valid where keep)
  float score;  // ranking score in nats; +inf when kept without ranking
  bool keep;
};

// Stage the group's query vectors into LDS as floats: q_s[h*D + i].
template <typename T, int D>
__device__ __forceinline__ void stage_queries(const T* __restrict__ q0, size_t head_stride, int group,
                                              float* q_s) {
  constexpr int VEC = Vec16<T>::n;
  constexpr int PER_HEAD = D / VEC;
  for (int x = lane_id(); x < group * PER_HEAD; x += kWave) {
    const int h = x / PER_HEAD, c = (x % PER_HEAD) * VEC;
    float v[VEC];
    load16(q0 + (size_t)h * head_stride + c, v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) q_s[h * D + c + e] = v[e];
  }
  wave_lds_sync();
}

// Eq. (7) at an intermediate level, summed over heads (eq. 11), for the node
// of this lane: children 2*node and 2*node+1 (if it exists) of the level below.
template <int D>
__device__ __forceinline__ float score_node_lse(const float* __restrict__ child_rows, int m_child,
                                                int node, const float* q_s, int group,
                                                float scale_log2, int variant = 0) {
  const int c0 = 2 * node;
  const bool has1 = c0 + 1 < m_child;
  const float* r0 = child_rows + (size_t)c0 * D;
  const float* r1 = r0 + (has1 ? D : 0);
  float a0[kMaxGroup], a1[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) a0[h] = a1[h] = 0.f;
#pragma unroll 4
  for (int d0 = 0; d0 < D; d0 += 4) {
    const float4 x0 = *reinterpret_cast<const float4*>(r0 + d0);
    const float4 x1 = *reinterpret_cast<const float4*>(r1 + d0);
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < group) {
        const float4 qq = *reinterpret_cast<const float4*>(q_s + h * D + d0);
        a0[h] += qq.x * x0.x + qq.y * x0.y + qq.z * x0.z + qq.w * x0.w;
        a1[h] += qq.x * x1.x + qq.y * x1.y + qq.z * x1.z + qq.w * x1.w;
      }
    }
  }
  if (variant != 0) {  // eq. (9) over the (one or two) children, in nats
    const float sc = scale_log2 * kLn2;
    float total = 0.f;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < group) {
        const float z0 = a0[h] * sc, z1 = has1 ? a1[h] * sc : z0;
        const float half = 0.5f * (z0 - z1);
        total += 0.5f * (z0 + z1) + (variant == 2 ? 0.5f * half * half : 0.f);
      }
    }
    return total;
  }
  float total = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < group) {
      const float z0 = a0[h] * scale_log2;
      if (has1) {
        const float z1 = a1[h] * scale_log2;
        const float m = fmaxf(z0, z1);
        total += m + log2f(exp2f(z0 - m) + exp2f(z1 - m));
      } else {
        total += z0;
      }
    }
  }
  return total * kLn2;
}

// Exact leaf LSE of eq. (7) at level 1 over the leaf's raw keys, summed over
// the group's heads; the whole wave cooperates (lane r takes key leaf*C + r).
template <typename T, int D>
__device__ __forceinline__ float score_leaf_lse_wave(const T* __restrict__ kb, int n_tok, int block,
                                                     int leaf, const float* q_s, int group,
                                                     float scale_log2, int variant = 0) {
  constexpr int VEC = Vec16<T>::n;
  const int lane = lane_id();
  const int tok = leaf * block + lane;
  const bool ok = lane < block && tok < n_tok;
  float acc[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.f;
  if (ok) {
    const T* row = kb + (size_t)tok * D;
#pragma unroll 4
    for (int d0 = 0; d0 < D; d0 += VEC) {
      float v[VEC];
      load16(row + d0, v);
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < group) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h] += q_s[h * D + d0 + e] * v[e];
        }
      }
    }
  }
  if (variant != 0) {  // eq. (9) over the leaf's raw keys, in nats
    const float sc = scale_log2 * kLn2;
    const float cnt = float(min(block, n_tok - leaf * block));
    float total = 0.f;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < group) {
        const float z = acc[h] * sc;
        const float mean = wave_sum(ok ? z : 0.f) / cnt;
        total += mean;
        if (variant == 2) {
          const float dz = z - mean;
          total += 0.5f * wave_sum(ok ? dz * dz : 0.f) / cnt;
        }
      }
    }
    return total;
  }
  float total = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < group) {
      const float z = ok ? acc[h] * scale_log2 : neg_inf();
      const float m = wave_max(z);
      const float s = wave_sum(ok ? exp2f(z - m) : 0.f);
      total += m + log2f(s);
    }
  }
  return total * kLn2;
}

// The full descent for query position t.  nbuf: 64 ints of this wave's LDS.
// intermediate_only: stop after level 2 and return the level-1 candidates
// (keep = candidate valid) without scoring them.
template <typename T, int D>
__device__ SelectResult select_descend(const float* q_s, int group, const T* __restrict__ kb,
                                       const float* __restrict__ pb, const LevelTable& lv,
                                       int n_tok, int block, int topk, int t, bool causal,
                                       bool force, float scale_log2, int* nbuf,
                                       bool intermediate_only = false, int variant = 0) {
  const int lane = lane_id();
  const int cur = t / block;
  int node = lane == 0 ? 0 : -1;
  bool keep = false;
  float score = pos_inf();
  for (int l = lv.n; l >= 1; --l) {
    const int sh = l - 1;
    const int lim = cur >> sh;
    bool valid = node >= 0 && (!causal || node <= lim);
    const uint64_t vm = ballot(valid);
    const int ncand = __popcll(vm);
    if (valid) nbuf[lanes_below(vm)] = node;
    wave_lds_sync();
    node = lane < ncand ? nbuf[lane] : -1;
    wave_lds_sync();
    valid = lane < ncand;
    if (l == 1 && intermediate_only) {
      keep = valid;
      score = pos_inf();
      break;
    }
    const bool forced = valid && causal &&
                        (node == lim || (force && (node == 0 || (cur >= 1 && node == ((cur - 1) >> sh)))));
    if (ncand <= topk) {
      keep = valid;
      score = pos_inf();
    } else {
      const int keep_n = topk - __popcll(ballot(forced));
      const bool rankable = valid && !forced;
      const uint64_t rm = ballot(rankable);
      float s = neg_inf();
      if (l >= 2) {
        if (rankable)
          s = score_node_lse<D>(pb + (size_t)lv.off[l - 2] * D, lv.size[l - 2], node, q_s, group,
                                scale_log2, variant);
      } else {
        uint64_t todo = rm;
        while (todo) {
          const int j = __builtin_ctzll(todo);
          todo &= todo - 1;
          const int leaf = readlane_i(node, j);
          const float sj =
              score_leaf_lse_wave<T, D>(kb, n_tok, block, leaf, q_s, group, scale_log2, variant);
          if (lane == j) s = sj;
        }
      }
      int rank = 0;
      uint64_t it = rm;
      while (it) {
        const int j = __builtin_ctzll(it);
        it &= it - 1;
        rank += ranks_before(readlane_f(s, j), readlane_i(node, j), s, node) ? 1 : 0;
      }
      keep = forced || (rankable && rank < keep_n);
      score = forced ? pos_inf() : s;
    }
    if (l > 1) {
      const uint64_t km = ballot(keep);
      const int p = lanes_below(km);
      const int m_child = lv.size[l - 2];
      if (keep && p < topk) {  // p < K unless NaN inputs broke the order
        nbuf[2 * p] = 2 * node;
        nbuf[2 * p + 1] = (2 * node + 1 < m_child) ? 2 * node + 1 : -1;
      }
      wave_lds_sync();
      node = lane < 2 * min(__popcll(km), topk) ? nbuf[lane] : -1;
      wave_lds_sync();
      keep = false;
    }
  }
  return {node, score, keep};
}

// Write the kept leaves ascending (with their scores), then -1 / -inf padding.
__device__ __forceinline__ void write_selection(const SelectResult& r, int topk,
                                                int32_t* __restrict__ idx_row,
                                                float* __restrict__ score_row) {
  const int lane = lane_id();
  const uint64_t km = ballot(r.keep);
  const int nk = __popcll(km);
  int pos = 0;
  uint64_t it = km;
  while (it) {
    const int j = __builtin_ctzll(it);
    it &= it - 1;
    pos += readlane_i(r.node, j) < r.node ? 1 : 0;
  }
  // pos < nk <= topk whenever the scores are totally ordered; the bound keeps
  // the row in place even if NaN inputs broke that order.
  if (r.keep && pos < topk) {
    idx_row[pos] = r.node;
    if (score_row) score_row[pos] = r.score;
  }
  if (lane >= nk && lane < topk) {
    idx_row[lane] = -1;
    if (score_row) score_row[lane] = neg_inf();
  }
}

}  // namespace pisa
