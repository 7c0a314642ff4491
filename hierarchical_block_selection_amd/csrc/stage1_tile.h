// Stage 1 of the two-stage selection, tile form: one workgroup walks the
// levels L..3 of the descent (PISA reading page §4.2 eq. (5)) for a tile of
// 64 (query, head) columns in lockstep.
//
// Scoring a level-l candidate needs q . kbar for its two children on level
// l-1 (eq. (7)).  When level l-1 holds at most kDenseMax rows, the tile
// computes the logits of every needed child row for all its columns on the
// matrix cores, 128 rows at a time: each summary is pre-split into bf16
// hi + lo planes (x = hi + lo + r with |r| <= 2^-16 |x|; q is bf16, so every
// product is exact and the fp32 accumulation behaves like an fp32 dot), and
// each query lane picks up the logits of its own two children from LDS.
// Reading a level costs 512 B per row for the whole tile, i.e. 8 B per row
// and column, below the 1 KB per candidate a gather moves, and the work per
// query is bounded by the constant 2 * kDenseMax rows, so selection stays
// O(log N) per query.  Larger levels are gathered per query (fp32 rows, 8
// lanes per row, loads batched).
//
// Decisions run per query in a 32-lane half-wave (two queries per wave, K <=
// 16 so 2K <= 32 candidates fit): future nodes dropped, keep-all when at most
// K remain (§03), otherwise the forced nodes (§5.3) plus the best K-#F by a
// 32-lane bitonic sort (score descending, node ascending on ties).
#pragma once

#include "pisa_common.h"

namespace pisa {
namespace tile1 {

constexpr int kCols = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kDenseMax = 1024;
constexpr int kChunk = 128;            // dense rows per LDS pass
constexpr int kSStride = 72;           // floats per logit row: 64 columns + 8 (rows r and r+4
                                       // of one MFMA store land 32 banks apart)
constexpr int kGatherBatch = 2;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t half_mask(uint64_t m, int half) {
  return uint32_t(m >> (32 * half));
}
__device__ __forceinline__ int below_in_half(uint32_t m32, int lane32) {
  return __popc(m32 & ((1u << lane32) - 1u));
}

// Bitonic sort over each 32-lane half: best (score desc, node asc) first.
// N independent lists are sorted together so that their lane exchanges
// overlap (each step issues 2N exchanges before consuming any).
template <int N>
__device__ __forceinline__ void sort32(float (&s)[N], int (&id)[N]) {
  const int l32 = lane_id() & 31;
#pragma unroll
  for (int k = 2; k <= 32; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      float ps[N];
      int pid[N];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        ps[n] = __shfl_xor(s[n], j, kWave);
        pid[n] = __shfl_xor(id[n], j, kWave);
      }
      const bool desc = (l32 & k) == 0 || k == 32;
      const bool lower = (l32 & j) == 0;
      const bool want_better = desc == lower;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const bool pb = ranks_before(ps[n], pid[n], s[n], id[n]);
        const bool sb = ranks_before(s[n], id[n], ps[n], pid[n]);
        const bool take = want_better ? pb : sb;
        s[n] = take ? ps[n] : s[n];
        id[n] = take ? pid[n] : id[n];
      }
    }
  }
}

// Split fp32 pyramid values into bf16 hi/lo planes (x ~ hi + lo).
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

template <int D, int G>
__global__ __launch_bounds__(kThreads) void stage1_tile_kernel(
    const bf16_t* __restrict__ q, const float* __restrict__ pyr, const bf16_t* __restrict__ phi,
    const bf16_t* __restrict__ plo, int* __restrict__ s1_nodes, int heads_q, int heads_kv,
    int n_tok, int block, int topk, int causal, int force, float scale_log2, LevelTable lv,
    int split_level) {
  constexpr int T = kCols / G;          // queries per tile
  constexpr int NPW = T / 2 / kWaves;   // query pairs per wave
  constexpr int KSTEPS = D / 16;
  constexpr int CPL = D / 8;            // gathered columns per lane (8 lanes per row)
  static_assert(NPW >= 1, "tile too small");
  constexpr int QROW = D + 8;  // padded query row (bf16) in LDS
  __shared__ float S[kChunk * kSStride];
  __shared__ int cand_s[T][32];
  __shared__ int tmp_s[kWaves][NPW][64];
  __shared__ float dots_s[kWaves][2][G][64];
  __shared__ __attribute__((aligned(16))) bf16_t qs[kCols * QROW];

  const int bh = blockIdx.y;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int t0 = blockIdx.x * T;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 31, kh = lane >> 5;
  const bool cz = causal != 0, fz = force != 0;

  // The tile's 64 query columns -> LDS (MFMA B operands are read from there).
  for (int x = threadIdx.x; x < kCols * (D / 8); x += kThreads) {
    const int c = x / (D / 8), d8 = (x % (D / 8)) * 8;
    const int qi = c / G, h = c % G, t = t0 + qi;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < n_tok)
      v = *reinterpret_cast<const uint4*>(
          q + (((size_t)b * heads_q + (size_t)kvh * G + h) * n_tok + t) * D + d8);
    *reinterpret_cast<uint4*>(&qs[c * QROW + d8]) = v;
  }
  for (int x = threadIdx.x; x < T * 32; x += kThreads) cand_s[x / 32][x % 32] = (x % 32) ? -1 : 0;
  const int t_last = min(t0 + T, n_tok) - 1;
  const int last_cur = t_last / block;
  const size_t head_rows = (size_t)bh * lv.rows;
  __syncthreads();

  for (int l = lv.n; l >= split_level; --l) {
    const int sh = l - 1;
    const int m_child = lv.size[l - 2];
    const bool may_score = lv.size[l - 1] > topk;
    const bool dense = may_score && m_child <= kDenseMax;
    const size_t child0 = head_rows + lv.off[l - 2];

    // A. Per query: eligible candidates (compacted), forced flags.  All pairs
    // of the wave go through each step together.
    int node_r[NPW];
    bool forced_r[NPW], scoring_r[NPW];
    float z_r[NPW][2][G];
    int ncand_r[NPW];
#pragma unroll
    for (int pi = 0; pi < NPW; ++pi) {
      const int qi = 2 * (wave * NPW + pi) + kh;
      const int t = t0 + qi;
      const int lim = (t < n_tok ? t / block : 0) >> sh;
      const int node = t < n_tok ? cand_s[qi][col] : -1;
      const bool valid = node >= 0 && (!cz || node <= lim);
      const uint32_t vm = half_mask(ballot(valid), kh);
      ncand_r[pi] = __popc(vm);
      if (valid) tmp_s[wave][pi][32 * kh + below_in_half(vm, col)] = node;
    }
    wave_lds_sync();
#pragma unroll
    for (int pi = 0; pi < NPW; ++pi) node_r[pi] = col < ncand_r[pi] ? tmp_s[wave][pi][32 * kh + col] : -1;
    wave_lds_sync();
#pragma unroll
    for (int pi = 0; pi < NPW; ++pi) {
      const int qi = 2 * (wave * NPW + pi) + kh;
      const int t = t0 + qi;
      const int cur = t < n_tok ? t / block : 0;
      const int lim = cur >> sh;
      const int node = node_r[pi];
      forced_r[pi] = node >= 0 && cz &&
                     (node == lim || (fz && (node == 0 || (cur >= 1 && node == ((cur - 1) >> sh)))));
      scoring_r[pi] = ncand_r[pi] > topk;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < G; ++h) z_r[pi][c][h] = neg_inf();
    }

    // B. Child logits of every rankable candidate.
    if (dense) {
      const int lim_last = cz ? (last_cur >> sh) : lv.size[l - 1] - 1;
      const int rows_needed = min(m_child, 2 * lim_last + 2);
      for (int r0 = 0; r0 < rows_needed; r0 += kChunk) {
        const int blk = r0 + 32 * wave;  // one 32-row block per wave
        if (blk < rows_needed) {
          const int r = blk + col;
          f32x16_t acc0 = {}, acc1 = {};
          const bool ok = r < m_child;
          const bf16_t* hrow = phi + (child0 + (ok ? r : 0)) * D;
          const bf16_t* lrow = plo + (child0 + (ok ? r : 0)) * D;
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
            uint4 hv = make_uint4(0, 0, 0, 0), lv4 = make_uint4(0, 0, 0, 0);
            if (ok) {
              hv = *reinterpret_cast<const uint4*>(hrow + 16 * s + 8 * kh);
              lv4 = *reinterpret_cast<const uint4*>(lrow + 16 * s + 8 * kh);
            }
            const bf16x8_t ah = as_bf16x8(hv), al = as_bf16x8(lv4);
            const bf16x8_t b0 =
                as_bf16x8(*reinterpret_cast<const uint4*>(&qs[col * QROW + 16 * s + 8 * kh]));
            const bf16x8_t b1 = as_bf16x8(
                *reinterpret_cast<const uint4*>(&qs[(32 + col) * QROW + 16 * s + 8 * kh]));
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b1, acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b1, acc1, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 32 * wave + (i / 4) * 8 + kh * 4 + (i % 4);
            S[row * kSStride + col] = acc0[i];
            S[row * kSStride + 32 + col] = acc1[i];
          }
        }
        __syncthreads();
#pragma unroll
        for (int pi = 0; pi < NPW; ++pi) {
          const int qi = 2 * (wave * NPW + pi) + kh;
          const int node = node_r[pi];
          const bool want = scoring_r[pi] & (node >= 0) & !forced_r[pi];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int row = 2 * node + c - r0;
            const bool in = want & (row >= 0) & (row < kChunk) & (2 * node + c < m_child);
            const int rr = in ? row : 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float v = S[rr * kSStride + qi * G + h];
              z_r[pi][c][h] = in ? v : z_r[pi][c][h];
            }
          }
        }
        __syncthreads();
      }
    } else if (may_score) {
      const float* child_rows = pyr + child0 * D;
#pragma unroll
      for (int pi = 0; pi < NPW; ++pi) {
        const int qi = 2 * (wave * NPW + pi) + kh;
        const int t = t0 + qi;
        const bool active = t < n_tok;
        const int node = node_r[pi];
        const bool rankable = scoring_r[pi] && node >= 0 && !forced_r[pi];
        if (!__ballot(rankable)) continue;
        float qreg[G][CPL];
        const int part = col & 7, sub = col >> 3;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (active) {
            const bf16_t* qrow = q + (((size_t)b * heads_q + (size_t)kvh * G + h) * n_tok + t) * D +
                                 part * CPL;
#pragma unroll
            for (int c = 0; c < CPL; c += 8) load16(qrow + c, &qreg[h][c]);
          } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c) qreg[h][c] = 0.f;
          }
        }
        const uint32_t rm = half_mask(ballot(rankable), kh);
        const int my_rows = rm ? 2 * (32 - __clz(rm)) : 0;
        const int n_rows = max(my_rows, __shfl_xor(my_rows, 32, kWave));
        for (int r0 = 0; r0 < n_rows; r0 += 4 * kGatherBatch) {
          float4 x[kGatherBatch][CPL / 4];
          bool live[kGatherBatch];
#pragma unroll
          for (int pp = 0; pp < kGatherBatch; ++pp) {
            const int r = r0 + 4 * pp + sub;
            const int cnd = (r >> 1) & 31;
            const int cnode = __shfl(node, 32 * kh + cnd, kWave);
            live[pp] = r < my_rows && ((rm >> cnd) & 1u) && (2 * cnode + (r & 1) < m_child);
            const float* row =
                child_rows + (size_t)(live[pp] ? 2 * cnode + (r & 1) : 0) * D + part * CPL;
#pragma unroll
            for (int c = 0; c < CPL / 4; ++c)
              x[pp][c] = live[pp] ? *reinterpret_cast<const float4*>(row + 4 * c)
                                  : make_float4(0, 0, 0, 0);
          }
#pragma unroll
          for (int pp = 0; pp < kGatherBatch; ++pp) {
            const int r = r0 + 4 * pp + sub;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float a = 0.f;
#pragma unroll
              for (int c = 0; c < CPL / 4; ++c)
                a += qreg[h][4 * c] * x[pp][c].x + qreg[h][4 * c + 1] * x[pp][c].y +
                     qreg[h][4 * c + 2] * x[pp][c].z + qreg[h][4 * c + 3] * x[pp][c].w;
              a += __shfl_xor(a, 1, kWave);
              a += __shfl_xor(a, 2, kWave);
              a += __shfl_xor(a, 4, kWave);
              if (part == 0 && r < 64) dots_s[wave][kh][h][r] = a;
            }
          }
        }
        wave_lds_sync();
        if (rankable) {
#pragma unroll
          for (int c = 0; c < 2; ++c)
            if (2 * node + c < m_child)
#pragma unroll
              for (int h = 0; h < G; ++h) z_r[pi][c][h] = dots_s[wave][kh][h][2 * col + c];
        }
        wave_lds_sync();
      }
    }

    // C. Scores, ranking, next candidates (or the kept level-split nodes).
    float ks[NPW];
    int kid[NPW];
    bool any_scoring = false;
#pragma unroll
    for (int pi = 0; pi < NPW; ++pi) {
      const int node = node_r[pi];
      const bool rankable = scoring_r[pi] & (node >= 0) & !forced_r[pi];
      any_scoring |= scoring_r[pi];
      // LSE of the two children (a missing second child has logit -inf).
      const bool has1 = 2 * node + 1 < m_child;
      float tot = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float z0 = z_r[pi][0][h] * scale_log2;
        const float z1 = has1 ? z_r[pi][1][h] * scale_log2 : neg_inf();
        const float mm = fmaxf(z0, z1);
        tot += mm + fast_log2(fast_exp2(z0 - mm) + fast_exp2(z1 - mm));
      }
      ks[pi] = rankable ? tot * kLn2 : neg_inf();
      kid[pi] = rankable ? node : 0x7fffffff;
    }
    if (__ballot(any_scoring)) sort32<NPW>(ks, kid);
#pragma unroll
    for (int pi = 0; pi < NPW; ++pi) {
      const int node = node_r[pi];
      const bool forced = forced_r[pi];
      const uint32_t fmask = half_mask(ballot(forced), kh);
      const int n_forced = __popc(fmask);
      const int keep_n = topk - n_forced;
      if (scoring_r[pi]) {
        if (forced) tmp_s[wave][pi][32 * kh + below_in_half(fmask, col)] = node;
        if (col < keep_n) tmp_s[wave][pi][32 * kh + n_forced + col] = kid[pi];
      } else if (node >= 0) {
        tmp_s[wave][pi][32 * kh + col] = node;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int pi = 0; pi < NPW; ++pi) {
      const int qi = 2 * (wave * NPW + pi) + kh;
      const int t = t0 + qi;
      const int n_kept = scoring_r[pi] ? topk : ncand_r[pi];
      const int kept = col < n_kept ? tmp_s[wave][pi][32 * kh + col] : -1;
      if (t < n_tok) {
        if (l > split_level) {
          if (col < 16) {
            cand_s[qi][2 * col] = kept >= 0 ? 2 * kept : -1;
            cand_s[qi][2 * col + 1] = (kept >= 0 && 2 * kept + 1 < m_child) ? 2 * kept + 1 : -1;
          }
        } else if (col < topk) {
          s1_nodes[((size_t)bh * n_tok + t) * topk + col] = kept;
        }
      }
    }
    wave_lds_sync();
    __syncthreads();
  }
}

}  // namespace tile1
}  // namespace pisa
