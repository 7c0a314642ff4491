// One decode step (PISA reading page §5.1: decode uses a single fused stage
// that reuses the already-loaded queries; §5.3 pyramid cache).  One
// wavefront per (sequence, KV head): the group's queries are staged once, the
// descent of select_core.h runs at t = cache_len - 1 over the pyramid of the
// cache, and attention for every head of the group follows over the selected
// blocks.
#include "attn_core.h"
#include "pisa_common.h"
#include "pisa_launch.h"
#include "select_core.h"

namespace pisa {

template <typename T, int D>
__global__ __launch_bounds__(kWave) void decode_kernel(
    const int32_t* __restrict__ cache_len, const T* __restrict__ q, const T* __restrict__ kc,
    const T* __restrict__ vc, const float* __restrict__ pyr, int32_t* __restrict__ idx,
    float* __restrict__ score, T* __restrict__ out, float* __restrict__ lse, int heads_q,
    int heads_kv, int capacity, int block, int topk, int group, int force, float scale_log2,
    LevelTable lv) {
  extern __shared__ float smem[];
  float* q_s = smem;                                        // group * D
  float* p_s = q_s + group * D;                             // 64
  int* nbuf = reinterpret_cast<int*>(p_s + kWave);          // 64
  int* sel = nbuf + kWave;                                  // topk (<= 32)
  const int bh = blockIdx.x;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int lane = lane_id();
  const int n = __builtin_amdgcn_readfirstlane(cache_len[b]);
  int32_t* idx_row = idx + (size_t)bh * topk;
  float* score_row = score ? score + (size_t)bh * topk : nullptr;
  const size_t head0 = (size_t)b * heads_q + (size_t)kvh * group;
  if (n < 1 || n > capacity) {
    if (lane < topk) {
      idx_row[lane] = -1;
      if (score_row) score_row[lane] = neg_inf();
    }
    for (int x = lane; x < group * D; x += kWave) store_from_f32(out + head0 * D + x, 0.f);
    if (lse && lane < group) lse[head0 + lane] = neg_inf();
    return;
  }
  const int t = n - 1;
  stage_queries<T, D>(q + head0 * D, D, group, q_s);
  const T* kb = kc + (size_t)bh * capacity * D;
  const T* vb = vc + (size_t)bh * capacity * D;
  const float* pb = pyr + (size_t)bh * lv.rows * D;
  const SelectResult r = select_descend<T, D>(q_s, group, kb, pb, lv, capacity, block, topk, t,
                                              true, force != 0, scale_log2, nbuf);
  write_selection(r, topk, idx_row, score_row);
  // Same ascending list into LDS for the attention loop.
  const uint64_t km = ballot(r.keep);
  const int nk = __popcll(km);
  int pos = 0;
  uint64_t it = km;
  while (it) {
    const int j = __builtin_ctzll(it);
    it &= it - 1;
    pos += readlane_i(r.node, j) < r.node ? 1 : 0;
  }
  if (r.keep) sel[pos] = r.node;
  wave_lds_sync();
  for (int h = 0; h < group; ++h) {
    attend_wave<T, D>(q_s + h * D, kb, vb, capacity, block, sel, nk, t, true, scale_log2, p_s,
                      out + (head0 + h) * D, lse ? lse + head0 + h : nullptr);
  }
}

template <typename T, int D>
static hipError_t launch_decode_t(const LaunchShape& s, const int32_t* cache_len, const void* q,
                                  const void* kc, const void* vc, const float* pyr, int32_t* idx,
                                  float* score, void* out, float* lse, hipStream_t st) {
  const size_t lds = ((size_t)s.group * D + 3 * kWave) * sizeof(float);
  prof::Scope ps("decode", st);
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3(s.batch * s.heads_kv), dim3(kWave), lds, st,
                     cache_len, static_cast<const T*>(q), static_cast<const T*>(kc),
                     static_cast<const T*>(vc), pyr, idx, score, static_cast<T*>(out), lse,
                     s.heads_q, s.heads_kv, s.seq_len, s.block, s.topk, s.group, s.force ? 1 : 0,
                     s.scale * kLog2e, s.lv);
  return hipGetLastError();
}

size_t decode_ws_bytes(const LaunchShape&) { return 0; }

hipError_t launch_decode(const LaunchShape& s, const int32_t* cache_len, const void* q,
                         const void* kc, const void* vc, const float* pyr, int32_t* idx,
                         float* score, void* out, float* lse, void* /*ws*/, hipStream_t st) {
  if (s.bf16)
    return s.head_dim == 128
               ? launch_decode_t<bf16_t, 128>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st)
               : launch_decode_t<bf16_t, 64>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
  return s.head_dim == 128
             ? launch_decode_t<float, 128>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st)
             : launch_decode_t<float, 64>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
}

}  // namespace pisa
