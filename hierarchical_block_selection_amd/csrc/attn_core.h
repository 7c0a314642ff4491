// Block-sparse attention for one query head, run by one wavefront.
//
// PISA reading page §02 eq. (2): softmax(scale q.k_j) weighted sum of v_j over
// the tokens of the selected leaf blocks, with future tokens of the current
// block masked in causal mode (§5.3).  Online softmax over the blocks: lane r
// scores key r of the block, the block's probabilities go through LDS and each
// lane accumulates D/64 output columns.
#pragma once

#include "pisa_common.h"

namespace pisa {

template <typename T, int D>
__device__ __forceinline__ void attend_wave(const float* q_s, const T* __restrict__ kb,
                                            const T* __restrict__ vb, int n_tok, int block,
                                            const int32_t* leaves, int n_leaves, int t, bool causal,
                                            float scale_log2, float* p_s, T* __restrict__ out,
                                            float* __restrict__ lse_out) {
  constexpr int VEC = Vec16<T>::n;
  constexpr int CPL = D / kWave;  // output columns per lane
  const int lane = lane_id();
  const int n_blocks = (n_tok + block - 1) / block;
  float m = neg_inf(), l = 0.f, o[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = 0.f;
  for (int j = 0; j < n_leaves; ++j) {
    const int leaf = __builtin_amdgcn_readfirstlane(leaves[j]);
    if (leaf < 0 || leaf >= n_blocks) continue;  // padding (or an index outside the sequence)
    const int base = leaf * block;
    const int tok = base + lane;
    const bool ok = lane < block && tok < n_tok && (!causal || tok <= t);
    float s = neg_inf();
    if (ok) {
      const T* row = kb + (size_t)tok * D;
      float acc = 0.f;
#pragma unroll 4
      for (int d0 = 0; d0 < D; d0 += VEC) {
        float v[VEC];
        load16(row + d0, v);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += q_s[d0 + e] * v[e];
      }
      s = acc * scale_log2;
    }
    const float mn = fmaxf(m, wave_max(s));
    if (mn == neg_inf()) continue;
    const float p = ok ? exp2f(s - mn) : 0.f;
    const float alpha = exp2f(m - mn);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] *= alpha;
    m = mn;
    p_s[lane] = p;
    wave_lds_sync();
    const int rows = min(block, n_tok - base);
    const T* vcol = vb + (size_t)base * D + lane * CPL;
    for (int r = 0; r < rows; ++r) {
      const float pr = p_s[r];
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] += pr * to_f32(vcol[(size_t)r * D + c]);
    }
    wave_lds_sync();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) store_from_f32(out + lane * CPL + c, o[c] * inv);
  if (lse_out && lane == 0) *lse_out = l > 0.f ? (m + log2f(l)) * kLn2 : neg_inf();
}

}  // namespace pisa
