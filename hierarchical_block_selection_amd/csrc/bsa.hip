// BSA flat block selection, the comparison baseline of the PISA reading page
// (§02 eq. (1); Table 1 row 5; §7.3 Figure 3): every query scores every
// eligible leaf summary, the scores are written in full, then a Top-K pass
// keeps the forced blocks plus the best K-#F others (ties to the lower index).
//
// Scores: s[t, i] = scale * sum over the group's heads of q_h,t . kbar_i
// (eq. (1) summed over the group's heads).
// bf16 inputs: the leaf summaries are split once into three bf16 planes
// (hi + mid + lo carries the fp32 value), and each workgroup computes a tile of
// 128 queries x 64 leaves as bf16 MFMA 32x32x16 (queries as the A operand, so
// each output row is a coalesced 128-byte store), skipping tiles entirely
// above the causal diagonal.  fp32 inputs use the LDS-tiled FMA kernel.
// Top-K runs one wavefront per query row: the row (<= 4096 scores) is held in
// registers, 64 lane-local maxima bound the K-th best from below, the few
// scores at or above that bound are compacted into LDS and ranked exactly.
#include <algorithm>

#include "pisa_common.h"
#include "pisa_launch.h"

namespace pisa {

constexpr int kBsaTile = 64;
constexpr int kBsaDk = 32;
constexpr int kBsaMaxLeaves = 4096;  // row length held in registers by the Top-K pass

template <typename T, int D>
__global__ __launch_bounds__(256) void bsa_scores_kernel(const T* __restrict__ q,
                                                         const float* __restrict__ pyr,
                                                         float* __restrict__ S, int heads_q,
                                                         int heads_kv, int n_tok, int block,
                                                         int group, int m1, int rows, int causal,
                                                         float scale) {
  __shared__ float qs[kBsaTile][kBsaDk + 1];
  __shared__ float ks[kBsaTile][kBsaDk + 1];
  const int bh = blockIdx.z;
  const int t0 = blockIdx.y * kBsaTile, i0 = blockIdx.x * kBsaTile;
  const int t_last = min(t0 + kBsaTile, n_tok) - 1;
  if (causal && i0 > t_last / block) return;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const float* kbar = pyr + (size_t)bh * rows * D;  // level 1 = first m1 rows
  float acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += kBsaDk) {
    for (int x = tid; x < kBsaTile * kBsaDk; x += 256) {
      const int r = x / kBsaDk, c = x % kBsaDk;
      const int t = t0 + r, i = i0 + r;
      float qv = 0.f;
      if (t < n_tok) {
        for (int h = 0; h < group; ++h)
          qv += to_f32(q[(((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t) * D + d0 + c]);
      }
      qs[r][c] = qv;
      ks[r][c] = i < m1 ? kbar[(size_t)i * D + d0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int dd = 0; dd < kBsaDk; ++dd) {
      float a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = qs[ty * 4 + u][dd];
        bb[u] = ks[tx + 16 * u][dd];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] += a[u] * bb[w];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = t0 + ty * 4 + u;
    if (t >= n_tok) continue;
    const int lim = causal ? t / block : m1 - 1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = i0 + tx + 16 * w;
      if (i <= lim && i < m1) S[((size_t)bh * n_tok + t) * m1 + i] = acc[u][w] * scale;
    }
  }
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int kMfmaQ = 128;  // queries per workgroup tile (32 per wave)
constexpr int kMfmaL = 64;   // leaves per workgroup tile

// Level-1 summaries of every head -> three bf16 planes x = hi + mid + lo.
__global__ void bsa_split_kernel(const float* __restrict__ pyr, bf16_t* __restrict__ planes,
                                 int rows, int m1, int d, size_t n) {
  // n = heads * m1 * d values; plane p of head bh, leaf i: planes[((p*heads + bh)*m1 + i)*d]
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = x / ((size_t)m1 * d), rem = x % ((size_t)m1 * d);
    const float v = pyr[bh * (size_t)rows * d + rem];
    const uint16_t h = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h);
    const uint16_t m = f32_to_bf16(r1);
    planes[x] = h;
    planes[n + x] = m;
    planes[2 * n + x] = f32_to_bf16(r1 - bf16_to_f32(m));
  }
}

template <int D>
__global__ __launch_bounds__(256) void bsa_scores_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ planes, float* __restrict__ S,
    int heads_q, int heads_kv, int n_tok, int block, int group, int m1, int causal, float scale,
    size_t plane_stride) {
  constexpr int KSTEPS = D / 16;
  const int bh = blockIdx.z;
  const int t0 = blockIdx.y * kMfmaQ, i0 = blockIdx.x * kMfmaL;
  const int t_last = min(t0 + kMfmaQ, n_tok) - 1;
  if (causal && i0 > t_last / block) return;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 31, kh = lane >> 5;
  const int tq0 = t0 + 32 * wave;  // this wave's 32 queries
  if (tq0 >= n_tok) return;
  f32x16_t acc[2] = {};
  const int tq = min(tq0 + col, n_tok - 1);  // A row (clamped; extra rows are not stored)
#pragma unroll
  for (int lb = 0; lb < 2; ++lb) {
    const int leaf = min(i0 + 32 * lb + col, m1 - 1);  // B column (clamped)
    const bf16_t* kp = planes + ((size_t)bh * m1 + leaf) * D;
    for (int h = 0; h < group; ++h) {
      const bf16_t* qrow = q + (((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + tq) * D;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * kh));
#pragma unroll
        for (int p = 2; p >= 0; --p) {
          const bf16x8_t bb = as_bf16x8(
              *reinterpret_cast<const uint4*>(kp + p * plane_stride + 16 * s + 8 * kh));
          acc[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[lb], 0, 0, 0);
        }
      }
    }
  }
  // acc[lb][i] = S[query tq0 + (i/4)*8 + kh*4 + i%4][leaf i0 + 32*lb + col]
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tq0 + (i / 4) * 8 + kh * 4 + (i % 4);
    if (t >= n_tok) continue;
    const int lim = causal ? t / block : m1 - 1;
#pragma unroll
    for (int lb = 0; lb < 2; ++lb) {
      const int leaf = i0 + 32 * lb + col;
      if (leaf <= lim && leaf < m1) S[((size_t)bh * n_tok + t) * m1 + leaf] = acc[lb][i] * scale;
    }
  }
}

__device__ __forceinline__ bool is_forced_leaf(int i, int cur, bool causal, bool force) {
  return causal && (i == cur || (force && (i == 0 || i == cur - 1)));
}

template <int VPL>
__global__ __launch_bounds__(256) void bsa_topk_kernel(const float* __restrict__ S,
                                                       int32_t* __restrict__ idx,
                                                       float* __restrict__ score, int n_tok,
                                                       int block, int m1, int topk, int causal,
                                                       int force) {
  __shared__ float cs[4][kWave];
  __shared__ int ci[4][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= n_tok) return;
  const int bh = blockIdx.y;
  const size_t row = (size_t)bh * n_tok + t;
  int32_t* idx_row = idx + row * topk;
  float* score_row = score ? score + row * topk : nullptr;
  const int cur = t / block;
  const int n_el = causal ? cur + 1 : m1;
  const bool cz = causal != 0, fz = force != 0;
  if (n_el <= topk) {  // every eligible block is kept without ranking
    if (lane < topk) {
      idx_row[lane] = lane < n_el ? lane : -1;
      if (score_row) score_row[lane] = lane < n_el ? pos_inf() : neg_inf();
    }
    return;
  }
  int n_forced = 0;
  if (cz) n_forced = (fz ? (cur >= 2 ? 3 : 2) : 1);
  const int keep_n = topk - n_forced;
  // Row in registers; forced and out-of-range entries become -inf.
  const float* srow = S + row * m1;
  float v[VPL];
  float best = neg_inf();
  int best_i = 0x7fffffff;
#pragma unroll
  for (int r = 0; r < VPL; ++r) {
    const int i = r * kWave + lane;
    v[r] = (i < n_el && !is_forced_leaf(i, cur, cz, fz)) ? srow[i] : neg_inf();
    if (i < n_el && !is_forced_leaf(i, cur, cz, fz) && ranks_before(v[r], i, best, best_i)) {
      best = v[r];
      best_i = i;
    }
  }
  // Threshold: the keep_n-th best lane maximum (in the total order score desc,
  // index asc) ranks no better than the keep_n-th best element of the row.
  float thr = neg_inf();
  int thr_i = 0x7fffffff;
  if (keep_n > 0) {
    int rank = 0;
    for (int j = 0; j < kWave; ++j)
      rank += ranks_before(readlane_f(best, j), readlane_i(best_i, j), best, best_i) ? 1 : 0;
    const uint64_t hit = ballot(rank == keep_n - 1 && best_i != 0x7fffffff);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      thr = readlane_f(best, src);
      thr_i = readlane_i(best_i, src);
    }
  }
  // Candidates: entries ranking at or before the threshold.
  int mine = 0;
#pragma unroll
  for (int r = 0; r < VPL; ++r) {
    const int i = r * kWave + lane;
    mine += (i < n_el && v[r] != neg_inf() && !ranks_before(thr, thr_i, v[r], i)) ? 1 : 0;
  }
  if (keep_n <= 0) mine = 0;
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  float cand_s = neg_inf();
  int cand_i = 0x7fffffff;
  bool chosen = false;
  if (total <= kWave) {
    int off = incl - mine;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
      const int i = r * kWave + lane;
      if (i < n_el && v[r] != neg_inf() && !ranks_before(thr, thr_i, v[r], i) && keep_n > 0) {
        cs[wave][off] = v[r];
        ci[wave][off] = i;
        ++off;
      }
    }
    wave_lds_sync();
    if (lane < total) {
      cand_s = cs[wave][lane];
      cand_i = ci[wave][lane];
    }
    wave_lds_sync();
    int rank = 0;
    for (int j = 0; j < total; ++j)
      rank += ranks_before(readlane_f(cand_s, j), readlane_i(cand_i, j), cand_s, cand_i) ? 1 : 0;
    chosen = lane < total && rank < keep_n;
  } else {
    // Rare: many candidates.  Extract the keep_n best one at a time.
    for (int k = 0; k < keep_n; ++k) {
      float bs = neg_inf();
      int bi = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < VPL; ++r) {
        const int i = r * kWave + lane;
        if (v[r] != neg_inf() && ranks_before(v[r], i, bs, bi)) {
          bs = v[r];
          bi = i;
        }
      }
      float ws = bs;
      int wi = bi;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float os = __shfl_xor(ws, o, kWave);
        const int oi = __shfl_xor(wi, o, kWave);
        if (ranks_before(os, oi, ws, wi)) {
          ws = os;
          wi = oi;
        }
      }
#pragma unroll
      for (int r = 0; r < VPL; ++r)
        if (r * kWave + lane == wi) v[r] = neg_inf();
      if (lane == k) {
        cand_s = ws;
        cand_i = wi;
        chosen = true;
      }
    }
  }
  // Final list: chosen candidates compacted first, then the forced leaves
  // (unranked, +inf); each lane then places its entry in ascending order.
  const uint64_t chm = ballot(chosen);
  const int n_ch = __popcll(chm);
  if (chosen) {
    cs[wave][lanes_below(chm)] = cand_s;
    ci[wave][lanes_below(chm)] = cand_i;
  }
  if (cz && lane == 0) {
    int f = n_ch;
    ci[wave][f] = cur;
    cs[wave][f++] = pos_inf();
    if (fz && cur >= 1) {
      ci[wave][f] = 0;
      cs[wave][f++] = pos_inf();
    }
    if (fz && cur >= 2) {
      ci[wave][f] = cur - 1;
      cs[wave][f++] = pos_inf();
    }
  }
  wave_lds_sync();
  const int nk = n_ch + n_forced;
  const bool keep = lane < nk;
  const int node = keep ? ci[wave][lane] : 0x7fffffff;
  const float sc = keep ? cs[wave][lane] : neg_inf();
  int pos = 0;
  for (int j = 0; j < nk; ++j) pos += readlane_i(node, j) < node ? 1 : 0;
  if (keep) {
    idx_row[pos] = node;
    if (score_row) score_row[pos] = sc;
  }
  if (lane >= nk && lane < topk) {
    idx_row[lane] = -1;
    if (score_row) score_row[lane] = neg_inf();
  }
}

static size_t scores_bytes(const LaunchShape& s) {
  return ((size_t)s.batch * s.heads_kv * s.seq_len * s.lv.size[0] * sizeof(float) + 255) &
         ~size_t(255);
}

size_t bsa_ws_bytes(const LaunchShape& s) {
  const size_t planes = s.bf16 ? 3 * (size_t)s.batch * s.heads_kv * s.lv.size[0] * s.head_dim *
                                     sizeof(bf16_t)
                               : 0;
  return scores_bytes(s) + planes;
}

template <typename T, int D>
static hipError_t launch_bsa_scores_t(const LaunchShape& s, const void* q, const float* pyr,
                                      float* S, hipStream_t st) {
  const int m1 = s.lv.size[0];
  dim3 grid((m1 + kBsaTile - 1) / kBsaTile, (s.seq_len + kBsaTile - 1) / kBsaTile,
            s.batch * s.heads_kv);
  prof::Scope ps("bsa_scores", st);
  hipLaunchKernelGGL((bsa_scores_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                     pyr, S, s.heads_q, s.heads_kv, s.seq_len, s.block, s.group, m1, s.lv.rows,
                     s.causal ? 1 : 0, s.scale);
  return hipGetLastError();
}

template <int VPL>
static hipError_t launch_bsa_topk_t(const LaunchShape& s, const float* S, int32_t* idx,
                                    float* score, hipStream_t st) {
  dim3 grid((s.seq_len + 3) / 4, s.batch * s.heads_kv);
  prof::Scope ps("bsa_topk", st);
  hipLaunchKernelGGL((bsa_topk_kernel<VPL>), grid, dim3(256), 0, st, S, idx, score, s.seq_len,
                     s.block, s.lv.size[0], s.topk, s.causal ? 1 : 0, s.force ? 1 : 0);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bsa_mfma_t(const LaunchShape& s, const void* q, const float* pyr,
                                    float* S, bf16_t* planes, hipStream_t st) {
  const int m1 = s.lv.size[0];
  const size_t n = (size_t)s.batch * s.heads_kv * m1 * D;
  {
    prof::Scope ps("bsa_split", st);
    hipLaunchKernelGGL(bsa_split_kernel, dim3((unsigned)std::min<size_t>(65536, (n + 255) / 256)),
                       dim3(256), 0, st, pyr, planes, s.lv.rows, m1, D, n);
  }
  dim3 grid((m1 + kMfmaL - 1) / kMfmaL, (s.seq_len + kMfmaQ - 1) / kMfmaQ, s.batch * s.heads_kv);
  prof::Scope ps("bsa_scores", st);
  hipLaunchKernelGGL((bsa_scores_mfma_kernel<D>), grid, dim3(256), 0, st,
                     static_cast<const bf16_t*>(q), planes, S, s.heads_q, s.heads_kv, s.seq_len,
                     s.block, s.group, m1, s.causal ? 1 : 0, s.scale, n);
  return hipGetLastError();
}

hipError_t launch_bsa(const LaunchShape& s, const void* q, const float* pyr, int32_t* idx,
                      float* score, void* ws, hipStream_t st) {
  float* S = static_cast<float*>(ws);
  hipError_t e;
  if (s.bf16) {
    bf16_t* planes = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + scores_bytes(s));
    e = s.head_dim == 128 ? launch_bsa_mfma_t<128>(s, q, pyr, S, planes, st)
                          : launch_bsa_mfma_t<64>(s, q, pyr, S, planes, st);
  } else
    e = s.head_dim == 128 ? launch_bsa_scores_t<float, 128>(s, q, pyr, S, st)
                          : launch_bsa_scores_t<float, 64>(s, q, pyr, S, st);
  if (e != hipSuccess) return e;
  const int m1 = s.lv.size[0];
  if (m1 <= 1 * kWave) return launch_bsa_topk_t<1>(s, S, idx, score, st);
  if (m1 <= 4 * kWave) return launch_bsa_topk_t<4>(s, S, idx, score, st);
  if (m1 <= 16 * kWave) return launch_bsa_topk_t<16>(s, S, idx, score, st);
  return launch_bsa_topk_t<kBsaMaxLeaves / kWave>(s, S, idx, score, st);
}

}  // namespace pisa
