// C ABI of libpisa: argument validation, pyramid geometry, workspace sizing and
// kernel dispatch.  Nothing is enqueued unless every argument is valid.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "pisa.h"
#include "pisa_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* what) {
  g_last_error = what;
  return code;
}

int fail_hip(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return PISA_ERR_HIP;
}

bool layout(int64_t n, int64_t c, pisa::LevelTable* lv) {
  int64_t m = (n + c - 1) / c;
  int levels = 0;
  int64_t off = 0;
  while (true) {
    if (levels >= PISA_MAX_LEVELS) return false;
    lv->size[levels] = (int)m;
    lv->off[levels] = (int)off;
    off += m;
    ++levels;
    if (m == 1) break;
    m = (m + 1) / 2;
  }
  if (off > INT32_MAX) return false;
  lv->n = levels;
  lv->rows = (int)off;
  return true;
}

// Shared validation of the problem description.  `op` selects op-specific rules.
int check_problem(const pisa_problem* p, int op, pisa::LaunchShape* s) {
  if (!p) return fail(PISA_ERR_INVALID, "problem is NULL");
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->seq_len < 1 || p->head_dim < 1 ||
      p->block < 1 || p->topk < 1)
    return fail(PISA_ERR_INVALID, "batch, heads, seq_len, head_dim, block and topk must be >= 1");
  if (p->heads_q % p->heads_kv != 0) return fail(PISA_ERR_INVALID, "heads_q % heads_kv != 0");
  if (p->dtype != PISA_F32 && p->dtype != PISA_BF16) return fail(PISA_ERR_INVALID, "bad dtype");
  if (p->flags & ~(uint32_t)(PISA_CAUSAL | PISA_FORCE_FIRST_PREV | PISA_SCORE_MEAN |
                             PISA_SCORE_MEAN_VAR))
    return fail(PISA_ERR_INVALID, "unknown flag bits");
  if ((p->flags & PISA_SCORE_MEAN) && (p->flags & PISA_SCORE_MEAN_VAR))
    return fail(PISA_ERR_INVALID, "PISA_SCORE_MEAN and PISA_SCORE_MEAN_VAR are exclusive");
  if ((p->flags & PISA_FORCE_FIRST_PREV) && !(p->flags & PISA_CAUSAL))
    return fail(PISA_ERR_INVALID, "PISA_FORCE_FIRST_PREV requires PISA_CAUSAL");
  if (!std::isfinite(p->scale)) return fail(PISA_ERR_INVALID, "scale is not finite");
  if (p->branch != 2) return fail(PISA_ERR_UNSUPPORTED, "only branch g = 2 is supported");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PISA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->block != 16 && p->block != 32 && p->block != 64)
    return fail(PISA_ERR_UNSUPPORTED, "block must be 16, 32 or 64");
  if (p->topk > 32) return fail(PISA_ERR_UNSUPPORTED, "topk must be <= 32");
  if ((p->flags & PISA_FORCE_FIRST_PREV) && p->topk < 3)
    return fail(PISA_ERR_UNSUPPORTED, "PISA_FORCE_FIRST_PREV needs topk >= 3");
  const int group = p->heads_q / p->heads_kv;
  if (group > pisa::kMaxGroup) return fail(PISA_ERR_UNSUPPORTED, "heads_q / heads_kv must be <= 16");
  if (op == PISA_OP_DECODE && !(p->flags & PISA_CAUSAL))
    return fail(PISA_ERR_INVALID, "decode requires PISA_CAUSAL");
  const int64_t elems = (int64_t)p->batch * std::max(p->heads_q, p->heads_kv) * p->seq_len *
                        p->head_dim;
  if (elems <= 0 || elems > (int64_t(1) << 40)) return fail(PISA_ERR_INVALID, "tensor too large");
  s->batch = p->batch;
  s->heads_q = p->heads_q;
  s->heads_kv = p->heads_kv;
  s->seq_len = p->seq_len;
  s->head_dim = p->head_dim;
  s->block = p->block;
  s->topk = p->topk;
  s->group = group;
  s->bf16 = p->dtype == PISA_BF16;
  s->causal = (p->flags & PISA_CAUSAL) != 0;
  s->force = (p->flags & PISA_FORCE_FIRST_PREV) != 0;
  s->variant = (p->flags & PISA_SCORE_MEAN) ? 1 : (p->flags & PISA_SCORE_MEAN_VAR) ? 2 : 0;
  s->scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->head_dim);
  if (!layout(p->seq_len, p->block, &s->lv)) return fail(PISA_ERR_INVALID, "pyramid too tall");
  if (op == PISA_OP_ATTN_BWD && !pisa::attn_bwd_supported(*s))
    return fail(PISA_ERR_UNSUPPORTED, "the backward needs bf16, block 64 and a power-of-two group");
  // Past 4096 leaf blocks only the MFMA path's Top-K (bf16, power-of-two
  // group, leaf count a multiple of 4) takes rows in segments.
  if (op == PISA_OP_BSA && s->lv.size[0] > 4096 &&
      !(s->bf16 && (s->group & (s->group - 1)) == 0 && s->lv.size[0] % 4 == 0))
    return fail(PISA_ERR_UNSUPPORTED,
                "BSA past 4096 leaf blocks needs bf16, a power-of-two group and a multiple of 4 "
                "leaf blocks");
  return PISA_OK;
}

size_t ws_bytes_for(const pisa::LaunchShape& s, int op) {
  switch (op) {
    case PISA_OP_SELECT: return pisa::select_two_stage_ws_bytes(s);
    case PISA_OP_BSA: return pisa::bsa_ws_bytes(s);
    case PISA_OP_ATTN: return pisa::attn_ws_bytes(s);
    case PISA_OP_DECODE: return pisa::decode_ws_bytes(s);
    case PISA_OP_ATTN_BWD: return pisa::attn_bwd_ws_bytes(s);
    default: return 0;
  }
}

// The kernels read and write these tensors (and the workspace) with 16-byte
// vector accesses: a pointer off that alignment is refused before any launch.
bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return true;
  return false;
}

int fail_align() { return fail(PISA_ERR_INVALID, "tensor pointer not 16-byte aligned"); }

int check_ws(const pisa::LaunchShape& s, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(s, op);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(PISA_ERR_WORKSPACE, "workspace missing or too small");
  if (need > 0 && misaligned({ws})) return fail(PISA_ERR_INVALID, "workspace not 16-byte aligned");
  return PISA_OK;
}

}  // namespace

extern "C" {

int pisa_pyramid_layout(int32_t seq_len, int32_t block, int32_t branch, int32_t* levels,
                        int64_t* row_offsets, int32_t max_offsets) {
  if (seq_len < 1 || block < 1) return fail(PISA_ERR_INVALID, "seq_len and block must be >= 1");
  if (branch != 2) return fail(PISA_ERR_INVALID, "branch must be 2");
  pisa::LevelTable lv;
  if (!layout(seq_len, block, &lv)) return fail(PISA_ERR_INVALID, "pyramid too tall");
  if (row_offsets) {
    if (max_offsets < lv.n + 1) return fail(PISA_ERR_INVALID, "row_offsets too small");
    for (int l = 0; l < lv.n; ++l) row_offsets[l] = lv.off[l];
    row_offsets[lv.n] = lv.rows;
  }
  if (levels) *levels = lv.n;
  return PISA_OK;
}

int pisa_workspace_bytes(const pisa_problem* problem, int32_t op, size_t* bytes) {
  if (!bytes) return fail(PISA_ERR_INVALID, "bytes is NULL");
  if (op < PISA_OP_PYRAMID || op > PISA_OP_ATTN_BWD) return fail(PISA_ERR_INVALID, "bad op");
  pisa::LaunchShape s;
  const int rc = check_problem(problem, op, &s);
  if (rc != PISA_OK) return rc;
  *bytes = ws_bytes_for(s, op);
  return PISA_OK;
}

int pisa_build_pyramid(const pisa_problem* problem, const void* k, float* pyramid, void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_PYRAMID, &s);
  if (rc != PISA_OK) return rc;
  if (!k || !pyramid) return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({k, pyramid})) return fail_align();
  const hipError_t e = pisa::launch_pyramid(s, k, pyramid, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_build_pyramid");
}

int pisa_select(const pisa_problem* problem, const void* q, const void* k, const float* pyramid,
                int32_t* block_idx, float* block_score, int32_t strategy, void* ws,
                size_t ws_bytes, void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_SELECT, &s);
  if (rc != PISA_OK) return rc;
  if (!q || !k || !pyramid || !block_idx) return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({q, k, pyramid})) return fail_align();
  if (strategy < PISA_SELECT_AUTO || strategy > PISA_SELECT_TWO_STAGE)
    return fail(PISA_ERR_INVALID, "bad strategy");
  bool two_stage = false;
  if (strategy == PISA_SELECT_TWO_STAGE) {
    if (!pisa::select_two_stage_supported(s))
      return fail(PISA_ERR_UNSUPPORTED, "two-stage selection does not support this problem");
    two_stage = true;
  } else if (strategy == PISA_SELECT_AUTO) {
    two_stage = pisa::select_two_stage_supported(s) && ws != nullptr &&
                ws_bytes >= pisa::select_two_stage_ws_bytes(s);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (two_stage) {
    if ((rc = check_ws(s, PISA_OP_SELECT, ws, ws_bytes)) != PISA_OK) return rc;
    e = pisa::launch_select_two_stage(s, q, k, pyramid, block_idx, block_score, ws, st);
  } else {
    e = pisa::launch_select_fused(s, q, k, pyramid, block_idx, block_score, st);
  }
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_select");
}

// ---------------------------------------------------------------------------
// Selection that allocates nothing: the two-stage selector's workspace lives
// in one fixed device array of the library.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(PISA_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

// Each device holds its own copy for the life of the process.  In host code
// the name only identifies the symbol; the device address of a device's copy
// comes from hipGetSymbolAddress with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up once per device).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "pisa_select_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PISA_ERR_UNSUPPORTED, "pisa_select_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "pisa_select_noalloc: hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PISA_OK;
}

}  // namespace

int pisa_select_noalloc(const pisa_problem* problem, const void* q, const void* k,
                        const float* pyramid, int32_t* block_idx, float* block_score,
                        int32_t strategy, void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_SELECT, &s);
  if (rc != PISA_OK) return rc;
  if (!q || !k || !pyramid || !block_idx) return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({q, k, pyramid})) return fail_align();
  if (strategy < PISA_SELECT_AUTO || strategy > PISA_SELECT_TWO_STAGE)
    return fail(PISA_ERR_INVALID, "bad strategy");
  bool two_stage = false;
  if (strategy == PISA_SELECT_TWO_STAGE) {
    if (!pisa::select_two_stage_supported(s))
      return fail(PISA_ERR_UNSUPPORTED, "two-stage selection does not support this problem");
    two_stage = true;
  } else if (strategy == PISA_SELECT_AUTO) {
    two_stage = pisa::select_two_stage_supported(s);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (two_stage) {
    const size_t need = pisa::select_two_stage_ws_bytes(s);
    if (need > kScratchBytes) {
      char msg[200];
      std::snprintf(msg, sizeof msg,
                    "pisa_select_noalloc: the problem needs %zu bytes of scratch, more than the "
                    "fixed %zu (use pisa_select with a workspace)",
                    need, kScratchBytes);
      return fail(PISA_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != PISA_OK) return rc;
    e = pisa::launch_select_two_stage(s, q, k, pyramid, block_idx, block_score, ws, st);
  } else {
    e = pisa::launch_select_fused(s, q, k, pyramid, block_idx, block_score, st);
  }
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_select_noalloc");
}

int pisa_bsa_select(const pisa_problem* problem, const void* q, const float* pyramid,
                    int32_t* block_idx, float* block_score, void* ws, size_t ws_bytes,
                    void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_BSA, &s);
  if (rc != PISA_OK) return rc;
  if (!q || !pyramid || !block_idx) return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({q, pyramid})) return fail_align();
  if ((rc = check_ws(s, PISA_OP_BSA, ws, ws_bytes)) != PISA_OK) return rc;
  const hipError_t e = pisa::launch_bsa(s, q, pyramid, block_idx, block_score, ws,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_bsa_select");
}

int pisa_block_sparse_attn(const pisa_problem* problem, const void* q, const void* k,
                           const void* v, const int32_t* block_idx, void* out, float* row_lse,
                           void* ws, size_t ws_bytes, void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_ATTN, &s);
  if (rc != PISA_OK) return rc;
  if (!q || !k || !v || !block_idx || !out) return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({q, k, v, out})) return fail_align();
  if ((rc = check_ws(s, PISA_OP_ATTN, ws, ws_bytes)) != PISA_OK) return rc;
  const hipError_t e = pisa::launch_attn(s, q, k, v, block_idx, out, row_lse, ws,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_block_sparse_attn");
}

int pisa_block_sparse_attn_backward(const pisa_problem* problem, const void* q, const void* k,
                                    const void* v, const int32_t* block_idx, const void* out,
                                    const float* row_lse, const void* dout, void* dq, void* dk,
                                    void* dv, void* ws, size_t ws_bytes, void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_ATTN_BWD, &s);
  if (rc != PISA_OK) return rc;
  if (!q || !k || !v || !block_idx || !out || !row_lse || !dout || !dq || !dk || !dv)
    return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({q, k, v, out, dout, dq, dk, dv})) return fail_align();
  if ((rc = check_ws(s, PISA_OP_ATTN_BWD, ws, ws_bytes)) != PISA_OK) return rc;
  const hipError_t e = pisa::launch_attn_bwd(s, q, k, v, block_idx, out, row_lse, dout, dq, dk, dv,
                                             ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_block_sparse_attn_backward");
}

int pisa_pyramid_append(const pisa_problem* problem, const int32_t* cache_len,
                        const void* k_cache, float* pyramid, void* stream) {
  pisa::LaunchShape s;
  const int rc = check_problem(problem, PISA_OP_PYRAMID, &s);
  if (rc != PISA_OK) return rc;
  if (!cache_len || !k_cache || !pyramid) return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({k_cache, pyramid})) return fail_align();
  const hipError_t e =
      pisa::launch_pyramid_append(s, cache_len, k_cache, pyramid, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_pyramid_append");
}

int pisa_decode_step(const pisa_problem* problem, const int32_t* cache_len, const void* q,
                     const void* k_cache, const void* v_cache, const float* pyramid,
                     int32_t* block_idx, float* block_score, void* out, float* row_lse,
                     void* ws, size_t ws_bytes, void* stream) {
  pisa::LaunchShape s;
  int rc = check_problem(problem, PISA_OP_DECODE, &s);
  if (rc != PISA_OK) return rc;
  if (!cache_len || !q || !k_cache || !v_cache || !pyramid || !block_idx || !out)
    return fail(PISA_ERR_INVALID, "null tensor pointer");
  if (misaligned({q, k_cache, v_cache, pyramid, out})) return fail_align();
  if ((rc = check_ws(s, PISA_OP_DECODE, ws, ws_bytes)) != PISA_OK) return rc;
  const hipError_t e = pisa::launch_decode(s, cache_len, q, k_cache, v_cache, pyramid, block_idx,
                                           block_score, out, row_lse, ws,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PISA_OK : fail_hip(e, "pisa_decode_step");
}

const char* pisa_status_string(int status) {
  switch (status) {
    case PISA_OK: return "ok";
    case PISA_ERR_INVALID: return "invalid argument";
    case PISA_ERR_UNSUPPORTED: return "unsupported problem";
    case PISA_ERR_WORKSPACE: return "workspace missing or too small";
    case PISA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* pisa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
