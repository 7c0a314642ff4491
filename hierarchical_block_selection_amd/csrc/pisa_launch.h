// Host-side launch interface between the C ABI (pisa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pisa_common.h"

namespace pisa {

namespace prof {
// Brackets the launches issued while it lives with HIP events on `st` when
// timing is enabled (pisa_profile_enable); does nothing otherwise.
class Scope {
 public:
  Scope(const char* name, hipStream_t st);
  ~Scope();
  Scope(const Scope&) = delete;
  Scope& operator=(const Scope&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  hipEvent_t start_;
};
}  // namespace prof

// A validated problem in the form the launchers use.
struct LaunchShape {
  int batch, heads_q, heads_kv, seq_len, head_dim, block, topk, group;
  bool bf16, causal, force;
  int variant;  // candidate score: 0 LSE (eq. 7), 1 mean (PISA-1), 2 mean + var/2 (PISA-2)
  float scale;
  LevelTable lv;
};

hipError_t launch_pyramid(const LaunchShape& s, const void* k, float* pyr, hipStream_t st);
hipError_t launch_pyramid_append(const LaunchShape& s, const int32_t* cache_len, const void* kc,
                                 float* pyr, hipStream_t st);

// Per-query fused selection (leaf level included).
hipError_t launch_select_fused(const LaunchShape& s, const void* q, const void* k,
                               const float* pyr, int32_t* idx, float* score, hipStream_t st);

// Two-stage selection: workspace layout and launch.
size_t select_two_stage_ws_bytes(const LaunchShape& s);
bool select_two_stage_supported(const LaunchShape& s);
hipError_t launch_select_two_stage(const LaunchShape& s, const void* q, const void* k,
                                   const float* pyr, int32_t* idx, float* score, void* ws,
                                   hipStream_t st);

// BSA flat selection: scores to workspace, then Top-K.
size_t bsa_ws_bytes(const LaunchShape& s);
hipError_t launch_bsa(const LaunchShape& s, const void* q, const float* pyr, int32_t* idx,
                      float* score, void* ws, hipStream_t st);

// Block-sparse attention.
size_t attn_ws_bytes(const LaunchShape& s);
hipError_t launch_attn(const LaunchShape& s, const void* q, const void* k, const void* v,
                       const int32_t* idx, void* out, float* lse, void* ws, hipStream_t st);

// Backward of the block-sparse attention (block lists held fixed).
bool attn_bwd_supported(const LaunchShape& s);
size_t attn_bwd_ws_bytes(const LaunchShape& s);
hipError_t launch_attn_bwd(const LaunchShape& s, const void* q, const void* k, const void* v,
                           const int32_t* idx, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, void* ws,
                           hipStream_t st);

// Decode step.
size_t decode_ws_bytes(const LaunchShape& s);
hipError_t launch_decode(const LaunchShape& s, const int32_t* cache_len, const void* q,
                         const void* kc, const void* vc, const float* pyr, int32_t* idx,
                         float* score, void* out, float* lse, void* ws, hipStream_t st);

}  // namespace pisa
