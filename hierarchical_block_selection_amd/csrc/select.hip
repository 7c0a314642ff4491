// PISA selection, per-query fused form: one wavefront per (batch, KV head,
// query position) runs the whole descent of select_core.h, leaf level
// included, and writes the ascending leaf list.  This is the "per-query"
// implementation of the PISA reading page (§7.3, Table 4).
#include "pisa_common.h"
#include "pisa_launch.h"
#include "select_core.h"

namespace pisa {

constexpr int kSelWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(kSelWaves * kWave) void select_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ pyr,
    int32_t* __restrict__ idx, float* __restrict__ score, int heads_q, int heads_kv, int n_tok,
    int block, int topk, int group, int causal, int force, int variant, float scale_log2,
    LevelTable lv) {
  extern __shared__ float smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  float* q_s = smem + wave * (group * D + kWave);
  int* nbuf = reinterpret_cast<int*>(q_s + group * D);
  const int t = blockIdx.x * kSelWaves + wave;
  if (t >= n_tok) return;
  const int bh = blockIdx.y;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const T* q0 = q + (((size_t)b * heads_q + (size_t)kvh * group) * n_tok + t) * D;
  stage_queries<T, D>(q0, (size_t)n_tok * D, group, q_s);
  const T* kb = k + (size_t)bh * n_tok * D;
  const float* pb = pyr + (size_t)bh * lv.rows * D;
  const SelectResult r = select_descend<T, D>(q_s, group, kb, pb, lv, n_tok, block, topk, t,
                                              causal != 0, force != 0, scale_log2, nbuf, false,
                                              variant);
  const size_t orow = ((size_t)bh * n_tok + t) * topk;
  write_selection(r, topk, idx + orow, score ? score + orow : nullptr);
}

template <typename T, int D>
static hipError_t launch_fused_t(const LaunchShape& s, const void* q, const void* k,
                                 const float* pyr, int32_t* idx, float* score, hipStream_t st) {
  dim3 grid((s.seq_len + kSelWaves - 1) / kSelWaves, s.batch * s.heads_kv);
  const size_t lds = (size_t)kSelWaves * (s.group * D + kWave) * sizeof(float);
  prof::Scope ps("select_fused", st);
  hipLaunchKernelGGL((select_fused_kernel<T, D>), grid, dim3(kSelWaves * kWave), lds, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), pyr, idx, score,
                     s.heads_q, s.heads_kv, s.seq_len, s.block, s.topk, s.group, s.causal ? 1 : 0,
                     s.force ? 1 : 0, s.variant, s.scale * kLog2e, s.lv);
  return hipGetLastError();
}

hipError_t launch_select_fused(const LaunchShape& s, const void* q, const void* k,
                               const float* pyr, int32_t* idx, float* score, hipStream_t st) {
  if (s.bf16)
    return s.head_dim == 128 ? launch_fused_t<bf16_t, 128>(s, q, k, pyr, idx, score, st)
                             : launch_fused_t<bf16_t, 64>(s, q, k, pyr, idx, score, st);
  return s.head_dim == 128 ? launch_fused_t<float, 128>(s, q, k, pyr, idx, score, st)
                           : launch_fused_t<float, 64>(s, q, k, pyr, idx, score, st);
}

}  // namespace pisa
