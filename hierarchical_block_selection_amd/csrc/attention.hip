// Block-sparse attention over the selected leaf blocks (PISA reading page §02
// eq. (2), causal mask of §5.3), per-query form: one wavefront per
// (batch, query head, position) runs attend_wave over the K blocks of its KV
// group's index row.
#include "attn_core.h"
#include "pisa_common.h"
#include "pisa_launch.h"

namespace pisa {

constexpr int kAttnWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_query_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, T* __restrict__ out, float* __restrict__ lse, int heads_q,
    int heads_kv, int n_tok, int block, int topk, int group, int causal, float scale_log2) {
  __shared__ float q_sm[kAttnWaves][D];
  __shared__ float p_sm[kAttnWaves][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * kAttnWaves + wave;
  if (t >= n_tok) return;
  const int bh = blockIdx.y;  // b * heads_q + h
  const int b = bh / heads_q, h = bh % heads_q;
  const int bkv = b * heads_kv + h / group;
  const T* qrow = q + ((size_t)bh * n_tok + t) * D;
  const int lane = lane_id();
  for (int x = lane; x < D; x += kWave) q_sm[wave][x] = to_f32(qrow[x]);
  wave_lds_sync();
  const int32_t* leaves = idx + ((size_t)bkv * n_tok + t) * topk;
  attend_wave<T, D>(q_sm[wave], k + (size_t)bkv * n_tok * D, v + (size_t)bkv * n_tok * D, n_tok,
                    block, leaves, topk, t, causal != 0, scale_log2, p_sm[wave],
                    out + ((size_t)bh * n_tok + t) * D,
                    lse ? lse + (size_t)bh * n_tok + t : nullptr);
}

template <typename T, int D>
static hipError_t launch_attn_t(const LaunchShape& s, const void* q, const void* k, const void* v,
                                const int32_t* idx, void* out, float* lse, hipStream_t st) {
  dim3 grid((s.seq_len + kAttnWaves - 1) / kAttnWaves, s.batch * s.heads_q);
  hipLaunchKernelGGL((attn_query_kernel<T, D>), grid, dim3(kAttnWaves * kWave), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     idx, static_cast<T*>(out), lse, s.heads_q, s.heads_kv, s.seq_len, s.block,
                     s.topk, s.group, s.causal ? 1 : 0, s.scale * kLog2e);
  return hipGetLastError();
}

size_t attn_ws_bytes(const LaunchShape&) { return 0; }

hipError_t launch_attn(const LaunchShape& s, const void* q, const void* k, const void* v,
                       const int32_t* idx, void* out, float* lse, void* /*ws*/, hipStream_t st) {
  if (s.bf16)
    return s.head_dim == 128 ? launch_attn_t<bf16_t, 128>(s, q, k, v, idx, out, lse, st)
                             : launch_attn_t<bf16_t, 64>(s, q, k, v, idx, out, lse, st);
  return s.head_dim == 128 ? launch_attn_t<float, 128>(s, q, k, v, idx, out, lse, st)
                           : launch_attn_t<float, 64>(s, q, k, v, idx, out, lse, st);
}

}  // namespace pisa
