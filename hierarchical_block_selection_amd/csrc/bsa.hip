// BSA flat block selection, the comparison baseline of the PISA reading page
// (§02 eq. (1); Table 1 row 5; §7.3 Figure 3): every query scores every
// eligible leaf summary, the scores are written in full, then a Top-K pass
// keeps the forced blocks plus the best K-#F others (ties to the lower index).
//
// Scores: s[t, i] = scale * sum over the group's heads of q_h,t . kbar_i
// (eq. (1) summed over the group's heads).
// bf16 inputs: the leaf summaries are split once into three bf16 planes
// (hi + mid + lo carries the fp32 value).  The score is linear in the query,
// so for a group of G > 1 heads the heads' queries are added in fp32 first and
// the sum enters as two bf16 parts (hi + lo): the MFMA count does not grow
// with G.  A workgroup owns 128 queries (32 per wave, held as MFMA A operands
// in registers) and walks the leaves 32 at a
// time up to its causal limit; the three planes of each 32-leaf tile are
// staged in LDS (double-buffered) and shared by the four waves.  Each output
// row segment is a coalesced 128-byte store.  fp32 inputs use an LDS-tiled
// FMA kernel.
// Top-K runs one wavefront per query row (<= 4096 scores held in registers):
// the K-#F-th largest of the 64 lane maxima (cross-lane bitonic sort) bounds
// the answer from below, the scores at or above it are compacted into LDS and
// ranked exactly on 64-bit (score, index) keys, and the kept leaves are put in
// ascending order by one more cross-lane sort.
#include <algorithm>

#include "pisa_common.h"
#include "pisa_launch.h"

namespace pisa {

constexpr int kBsaTile = 64;
constexpr int kBsaDk = 32;
// Row length held in registers by the Top-K pass: the longest row of the
// general pass; rows of the MFMA path are taken in segments of this length.
constexpr int kBsaMaxLeaves = 4096;

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
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int kMfmaQ = 128;  // queries per workgroup (32 per wave)
constexpr int kMfmaL = 32;   // leaves per tile

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

// The row of query t holds eq. (1) scores of its rankable leaves; its forced
// leaves (§5.3: current, and with forcing the first and the previous) and the
// entries from its causal bound up to the next multiple of 4 hold -inf, so
// that the Top-K pass reads whole 16-byte groups without masks.
//
// The pass waits on its score stores, so occupancy is what moves it: three
// workgroups per CU at d = 128 (their LDS tiles take 153 KB) and four at
// d = 64, which caps the registers at 168 and 128 (128K: 0.75-0.80 ->
// 0.67 ms against two per CU).
template <int D, int G>
__global__ __launch_bounds__(256, D == 64 ? 4 : 3) void bsa_scores_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ planes, float* __restrict__ S,
    int heads_q, int heads_kv, int n_tok, int block, int m1, int causal, int force, float scale,
    size_t plane_stride) {
  constexpr int KSTEPS = D / 16;
  constexpr int ROW = D + 8;                 // padded LDS row (bf16)
  constexpr int V16 = D / 8;                 // 16-byte pieces per row
  constexpr int PIECES = 3 * kMfmaL * V16;   // per tile
  constexpr int PER_THREAD = (PIECES + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16_t bs[2][3][kMfmaL * ROW];
  const int bh = blockIdx.y;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int t0 = blockIdx.x * kMfmaQ;
  const int t_last = min(t0 + kMfmaQ, n_tok) - 1;
  const int lim_last = causal ? t_last / block : m1 - 1;
  const int n_tiles = lim_last / kMfmaL + 1;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  __builtin_assume(tid < 256);  // the launch's block size: fetch/put guards fold when 256 | PIECES
  const int col = lane & 31, kh = lane >> 5;
  const int tq0 = t0 + 32 * wave;
  // A operands: this lane's query row (clamped).  Eq. (1) summed over the
  // group is linear in the query, so a group's heads are added first (fp32)
  // and the sum enters as bf16 hi and lo parts: 2 operands for any G.
  constexpr int NQ = G == 1 ? 1 : 2;
  const int tq = min(tq0 + col, n_tok - 1);
  bf16x8_t a[NQ][KSTEPS];
  if constexpr (G == 1) {
    const bf16_t* qr = q + (((size_t)b * heads_q + (size_t)kvh) * n_tok + tq) * D + 8 * kh;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) a[0][s] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qr + 16 * s));
  } else {
    // One head's row at a time (heads in order), so that the loads of all
    // G rows are never live together.
    float sum[KSTEPS][8] = {};
#pragma unroll 1
    for (int h = 0; h < G; ++h) {
      const bf16_t* qr = q + (((size_t)b * heads_q + (size_t)kvh * G + h) * n_tok + tq) * D + 8 * kh;
      u32x4_t w[KSTEPS];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) w[s] = *reinterpret_cast<const u32x4_t*>(qr + 16 * s);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[s][2 * e] += __uint_as_float(w[s][e] << 16);
          sum[s][2 * e + 1] += __uint_as_float(w[s][e] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hi = (__bf16)sum[s][e];
        a[0][s][e] = hi;
        a[1][s][e] = (__bf16)(sum[s][e] - (float)hi);
      }
  }
  const bf16_t* pb = planes + (size_t)bh * m1 * D;
  u32x4_t stage[PER_THREAD];
  auto fetch = [&](int lt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int x = tid + 256 * i;
      const int p = x / (kMfmaL * V16), rem = x % (kMfmaL * V16);
      const int leaf = min(lt * kMfmaL + rem / V16, m1 - 1);
      stage[i] = x < PIECES ? *reinterpret_cast<const u32x4_t*>(pb + p * plane_stride +
                                                                (size_t)leaf * D + 8 * (rem % V16))
                            : u32x4_t{0, 0, 0, 0};
    }
  };
  auto put = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int x = tid + 256 * i;
      const int p = x / (kMfmaL * V16), rem = x % (kMfmaL * V16);
      if (x < PIECES)
        *reinterpret_cast<u32x4_t*>(&bs[buf][p][(rem / V16) * ROW + 8 * (rem % V16)]) = stage[i];
    }
  };
  // The tile loop decides its stores and masks without branches: the
  // causal bound of row t is t >> log2(C) (C is a power of two).
  const bool cz = causal != 0, fz = force != 0;
  const int cshift = 31 - __builtin_clz(block);
  fetch(0);
  put(0);
  __syncthreads();
  for (int lt = 0; lt < n_tiles; ++lt) {
    const int buf = lt & 1;
    if (lt + 1 < n_tiles) fetch(lt + 1);
    f32x16_t acc = {};
#pragma unroll
    for (int p = 2; p >= 0; --p)
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8_t bb =
            as_bf16x8(*reinterpret_cast<const u32x4_t*>(&bs[buf][p][col * ROW + 16 * s + 8 * kh]));
#pragma unroll
        for (int h = 0; h < NQ; ++h)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][s], bb, acc, 0, 0, 0);
      }
    // acc[i] = S[query tq0 + (i/4)*8 + 4kh + i%4][leaf lt*32 + col]
    const int leaf = lt * kMfmaL + col;
    const bool leaf_ok = leaf < m1;
    float* const srow0 = S + ((size_t)bh * n_tok + tq0 + 4 * kh) * m1 + leaf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = tq0 + (i / 4) * 8 + 4 * kh + (i % 4);
      const int lim = cz ? t >> cshift : m1 - 1;
      const bool forced = cz & ((leaf == lim) | (fz & ((leaf == 0) | (leaf == lim - 1))));
      const bool keep = (t < n_tok) & leaf_ok & (leaf < ((lim + 4) & ~3));
      const float val = (leaf <= lim) & !forced ? acc[i] * scale : neg_inf();
      if (keep)  // streamed out: read once, by the Top-K pass
        __builtin_nontemporal_store(val, srow0 + (size_t)((i / 4) * 8 + (i % 4)) * m1);
    }
    if (lt + 1 < n_tiles) {
      put(buf ^ 1);  // the other buffer was last read one tile ago
      __syncthreads();
    }
  }
}

// 64-bit rank key: higher score first, lower index first on equal scores.
__device__ __forceinline__ uint32_t ord32(float s) {
  const uint32_t b = __float_as_uint(s);
  return b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u);
}

// Bitonic sort of one value per lane across the wave, descending.
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t y = __shfl_xor(x, j, kWave);
      const bool desc = (lane & k) == 0 || k == kWave;
      const bool lower = (lane & j) == 0;
      x = (desc == lower) ? max(x, y) : min(x, y);
    }
  return x;
}
__device__ __forceinline__ uint64_t wave_sort_desc64(uint64_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = (uint64_t(uint32_t(__shfl_xor(int(x >> 32), j, kWave))) << 32) |
                         uint32_t(__shfl_xor(int(uint32_t(x)), j, kWave));
      const bool desc = (lane & k) == 0 || k == kWave;
      const bool lower = (lane & j) == 0;
      x = (desc == lower) ? (x > y ? x : y) : (x < y ? x : y);
    }
  return x;
}

template <int VPL>  // scores per lane (row length <= 64 * VPL), VPL % 4 == 0
__global__ __launch_bounds__(256) void bsa_topk_kernel(const float* __restrict__ S,
                                                       int32_t* __restrict__ idx,
                                                       float* __restrict__ score, int n_tok,
                                                       int block, int m1, int topk, int causal,
                                                       int force) {
  __shared__ uint64_t cand[4][kWave + 1];  // entry kWave takes non-candidates
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
  // Forced leaves (§5.3): current, and with forcing the first and previous.
  const int f1 = (cz && fz) ? 0 : -1;
  const int f2 = (cz && fz && cur >= 2) ? cur - 1 : -1;
  const int n_forced = cz ? 1 + (fz ? (cur >= 2 ? 2 : 1) : 0) : 0;
  const int keep_n = topk - n_forced;
  // Row in registers: element i = 256 r + 4 lane + e (16-byte loads).
  const float* srow = S + row * m1;
  uint32_t key[VPL];
  uint32_t lmax = 0;
#pragma unroll
  for (int r = 0; r < VPL / 4; ++r) {
    const int i0 = 256 * r + 4 * lane;
    float4 x4 = make_float4(0.f, 0.f, 0.f, 0.f);
    // (reads up to 3 floats past the row; the workspace has slack for the last row)
    if (i0 < n_el) x4 = *reinterpret_cast<const float4*>(srow + i0);
    const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      const bool rankable =
          (i < n_el) & !(cz & ((i == cur) | (i == f1) | (i == f2)));
      key[4 * r + e] = rankable ? ord32(xs[e]) | 1u : 0u;  // rankable keys are never 0
      lmax = max(lmax, key[4 * r + e]);
    }
  }
  bool chosen = false;
  uint64_t mine = 0;
  if (keep_n > 0) {
    // Lower bound on the keep_n-th best key: the keep_n-th best lane maximum.
    // (at least 1: unrankable entries have key 0)
    const uint32_t sorted = wave_sort_desc(lmax);
    const uint32_t thr = max(1u, uint32_t(__builtin_amdgcn_readlane(sorted, keep_n - 1)));
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < VPL; ++r) cnt += key[r] >= thr ? 1 : 0;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    if (total <= kWave) {
      int off = incl - cnt;
#pragma unroll
      for (int r = 0; r < VPL; ++r) {
        const int i = 256 * (r / 4) + 4 * lane + (r % 4);
        const bool c = key[r] >= thr;
        cand[wave][c ? off : kWave] = (uint64_t(key[r]) << 32) | uint32_t(0xffffffffu - uint32_t(i));
        off += c ? 1 : 0;
      }
      wave_lds_sync();
      const uint64_t ck = lane < total ? cand[wave][lane] : 0ull;
      wave_lds_sync();
      const uint64_t srt = wave_sort_desc64(ck);
      chosen = lane < keep_n;
      mine = srt;
    } else {
      // Rare: many scores at the bound.  Extract the keep_n best one at a time
      // (largest key, then the lowest index holding it).
      for (int kk = 0; kk < keep_n; ++kk) {
        uint32_t best = 0;
#pragma unroll
        for (int r = 0; r < VPL; ++r) best = max(best, key[r]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) best = max(best, uint32_t(__shfl_xor(int(best), o, kWave)));
        int bi = 0x7fffffff;
#pragma unroll
        for (int r = 0; r < VPL; ++r)
          bi = key[r] == best ? min(bi, 256 * (r / 4) + 4 * lane + (r % 4)) : bi;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) bi = min(bi, __shfl_xor(bi, o, kWave));
#pragma unroll
        for (int r = 0; r < VPL; ++r)
          key[r] = 256 * (r / 4) + 4 * lane + (r % 4) == bi ? 0u : key[r];
        if (lane == kk) {
          chosen = true;
          mine = (uint64_t(best) << 32) | uint32_t(0xffffffffu - uint32_t(bi));
        }
      }
    }
  }
  // Kept leaves: chosen candidates in lanes < keep_n, forced leaves appended,
  // then ascending order by one more sort (key = ~index puts small first).
  int node = chosen ? int(0xffffffffu - uint32_t(mine)) : -1;
  if (cz) {
    if (lane == keep_n) node = cur;
    if (fz && lane == keep_n + 1 && cur >= 1) node = 0;
    if (fz && lane == keep_n + 2 && cur >= 2) node = cur - 1;
  }
  const uint32_t o_sorted = wave_sort_desc(node >= 0 ? 0xffffffffu - uint32_t(node) : 0u);
  const int out = o_sorted ? int(0xffffffffu - o_sorted) : -1;
  if (lane < topk) {
    idx_row[lane] = out;
    if (score_row) {
      const bool forced = cz & ((out == cur) | (out == f1) | (out == f2));
      score_row[lane] = out < 0 ? neg_inf() : (forced ? pos_inf() : srow[out]);
    }
  }
}

// Top-K over rows written by bsa_scores_mfma_kernel (forced leaves and the
// padding to a multiple of 4 already hold -inf; M1 % 4 == 0), LPR lanes per
// query row (32: two rows per wavefront; 64: one), VPL scores per lane:
//   1. the row in registers (16-byte loads up to the causal bound);
//   2. the (K-#F)-th largest lane maximum, by a bitonic sort across the row's
//      lanes, bounds the answer from below;
//   3. each lane marks its scores at or above that bound in a bitmask; the
//      marked entries (rarely more than a few per lane) are gathered through
//      LDS as 64-bit (score, ~index) keys and sorted exactly: higher score
//      first, lower index first on ties;
//   4. the kept leaves plus the forced ones are put in ascending order by one
//      more sort and written.
// A row whose marked entries exceed LPR falls back to extracting the best
// entries one at a time.  Rows longer than LPR * VPL scores (past 4096 leaf
// blocks, one row per wavefront) run steps 1-3 per segment of that length and
// merge each segment's sorted keys into the running best LPR.
__device__ __forceinline__ uint32_t xlane_u32(uint32_t v, int j) {
  return uint32_t(__shfl_xor(int(v), j, kWave));
}
template <int LPR>
__device__ __forceinline__ float row_sort_desc(float x, int hl) {
#pragma unroll
  for (int k = 2; k <= LPR; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float y = __shfl_xor(x, j, kWave);
      const bool desc = (hl & k) == 0 || k == LPR;
      const bool lower = (hl & j) == 0;
      x = (desc == lower) ? fmaxf(x, y) : fminf(x, y);
    }
  return x;
}
template <int LPR>
__device__ __forceinline__ uint64_t row_sort_desc64(uint64_t x, int hl) {
#pragma unroll
  for (int k = 2; k <= LPR; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = (uint64_t(xlane_u32(uint32_t(x >> 32), j)) << 32) | xlane_u32(uint32_t(x), j);
      const bool desc = (hl & k) == 0 || k == LPR;
      const bool lower = (hl & j) == 0;
      x = (desc == lower) ? (x > y ? x : y) : (x < y ? x : y);
    }
  return x;
}
template <int LPR>
__device__ __forceinline__ uint32_t row_sort_desc32(uint32_t x, int hl) {
#pragma unroll
  for (int k = 2; k <= LPR; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t y = xlane_u32(x, j);
      const bool desc = (hl & k) == 0 || k == LPR;
      const bool lower = (hl & j) == 0;
      x = (desc == lower) ? max(x, y) : min(x, y);
    }
  return x;
}

// lanes per row (32 or 64), scores per lane (% 4 == 0), rows longer than LPR * VPL.
// Rows held as 64 scores per lane (1025 to 4096 leaves) run four waves per
// SIMD (128 VGPRs, a few spilled): the pass waits on its row loads, and more
// waves keep more of them in flight (Top-K at 128K 0.66 -> 0.56-0.62 ms
// against three waves per SIMD; about 3% at 256K).
template <int LPR, int VPL, bool kLong>
__global__ __launch_bounds__(256, (VPL == 64 && !kLong) ? 4 : 1) void bsa_topk_rows_kernel(
                                                            const float* __restrict__ S,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ score, int n_tok,
                                                            int block, int m1, int topk,
                                                            int causal, int force) {
  constexpr int ROWS = 256 / LPR;  // rows per workgroup
  constexpr int NM = (VPL + 31) / 32;  // 32-bit candidate masks per lane
  __shared__ uint64_t cand[ROWS][LPR + 1];  // entry LPR takes non-candidates
  const int lane = lane_id();
  const int hl = lane & (LPR - 1);
  const int slot = threadIdx.x / LPR;
  const int t = blockIdx.x * ROWS + slot;
  const bool live = t < n_tok;
  const int bh = blockIdx.y;
  const size_t row = (size_t)bh * n_tok + (live ? t : n_tok - 1);
  const float* srow = S + row * m1;
  const int cur = (live ? t : n_tok - 1) / block;
  const bool cz = causal != 0, fz = force != 0;
  const int n_el = cz ? cur + 1 : m1;
  const bool keep_all = n_el <= topk;
  const int n_forced = cz ? 1 + (fz ? (cur >= 2 ? 2 : 1) : 0) : 0;
  const int keep_n = keep_all ? 0 : topk - n_forced;
  // A row longer than LPR * VPL scores (one row per wavefront: LPR = 64) is
  // taken in segments of that length; the sorted keys of each segment are
  // merged into the running list, lane hl holding the hl-th best so far.
  constexpr int SEG = LPR * VPL;
  bool chosen = false;
  uint64_t mine = 0;
  static_assert(!kLong || LPR == 64, "segments need one row per wavefront");
  for (int s0 = 0; s0 == 0 || (kLong && s0 < n_el); s0 += SEG) {
    // 1. The segment: element i = s0 + 4 LPR g + 4 hl + e (g < VPL / 4, e < 4).
    float x[VPL];
    float lmax = neg_inf();
#pragma unroll
    for (int g = 0; g < VPL / 4; ++g) {
      const int i0 = s0 + 4 * LPR * g + 4 * hl;
      float4 v = make_float4(neg_inf(), neg_inf(), neg_inf(), neg_inf());
      if (!keep_all && i0 < n_el) v = *reinterpret_cast<const float4*>(srow + i0);
      x[4 * g] = v.x; x[4 * g + 1] = v.y; x[4 * g + 2] = v.z; x[4 * g + 3] = v.w;
      lmax = fmaxf(lmax, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
    // 2. Lower bound: the keep_n-th largest lane maximum of the segment.
    const float srt = row_sort_desc<LPR>(lmax, hl);
    const int kk = max(keep_n, 1) - 1;
    const float thr = __shfl(srt, (lane & ~(LPR - 1)) + kk, kWave);
    // 3. Marked entries (>= thr and rankable, i.e. > -inf).
    uint32_t m[NM];
#pragma unroll
    for (int w = 0; w < NM; ++w) m[w] = 0u;
#pragma unroll
    for (int r = 0; r < VPL; ++r)
      m[r / 32] |= (x[r] >= thr && x[r] > neg_inf()) ? (1u << (r % 32)) : 0u;
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < NM; ++w) cnt += __popc(m[w]);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) {
      const int y = __shfl_up(incl, o, LPR);
      if (hl >= o) incl += y;
    }
    const int total = __shfl(incl, (lane & ~(LPR - 1)) + LPR - 1, kWave);
    bool seg_chosen = false;
    uint64_t seg_key = 0;
    if (keep_n > 0 && total <= LPR) {
      int off = incl - cnt;
      bool more = cnt > 0;
      // marked entries, one per lane per round (their scores are re-read: L2)
      while (__ballot(more) != 0) {
        if (more) {
          int w = 0;
#pragma unroll
          for (int ww = NM - 1; ww >= 0; --ww) w = m[ww] != 0u ? ww : w;
          uint32_t mw = m[0];
#pragma unroll
          for (int ww = 1; ww < NM; ++ww) mw = w == ww ? m[ww] : mw;
          const int r = 32 * w + __builtin_ctz(mw);
          const int i = s0 + 4 * LPR * (r / 4) + 4 * hl + (r % 4);
          cand[slot][off] = (uint64_t(ord32(srow[i])) << 32) | uint32_t(0xffffffffu - uint32_t(i));
          ++off;
          mw &= mw - 1u;
#pragma unroll
          for (int ww = 0; ww < NM; ++ww) m[ww] = w == ww ? mw : m[ww];
          more = false;
#pragma unroll
          for (int ww = 0; ww < NM; ++ww) more |= m[ww] != 0u;
        }
      }
      wave_lds_sync();
      const uint64_t ck = hl < total ? cand[slot][hl] : 0ull;
      wave_lds_sync();
      seg_key = row_sort_desc64<LPR>(ck, hl);
      seg_chosen = hl < keep_n;
    } else if (keep_n > 0) {
      // Rare: many entries at the bound.  The keep_n best, one at a time
      // (largest score, then the lowest index holding it).
      uint32_t key[VPL];
#pragma unroll
      for (int r = 0; r < VPL; ++r) key[r] = x[r] > neg_inf() ? ord32(x[r]) | 1u : 0u;
      for (int q = 0; q < keep_n; ++q) {
        uint32_t best = 0;
#pragma unroll
        for (int r = 0; r < VPL; ++r) best = max(best, key[r]);
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) best = max(best, xlane_u32(best, o));
        int bi = 0x7fffffff;
#pragma unroll
        for (int r = 0; r < VPL; ++r)
          bi = key[r] == best ? min(bi, s0 + 4 * LPR * (r / 4) + 4 * hl + (r % 4)) : bi;
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) bi = min(bi, __shfl_xor(bi, o, kWave));
#pragma unroll
        for (int r = 0; r < VPL; ++r)
          key[r] = s0 + 4 * LPR * (r / 4) + 4 * hl + (r % 4) == bi ? 0u : key[r];
        if (hl == q) {
          seg_chosen = true;
          seg_key = (uint64_t(ord32(srow[bi])) << 32) | uint32_t(0xffffffffu - uint32_t(bi));
        }
      }
    }
    if (s0 == 0) {
      chosen = seg_chosen;
      mine = seg_key;
    } else {
      // Merge: the running list and the segment's, both descending with 0
      // past their ends and keys distinct.  The larger of run[hl] and
      // seg[LPR - 1 - hl] is a bitonic sequence holding the best LPR of
      // both; a bitonic merge sorts it descending.
      const uint64_t a = chosen ? mine : 0ull;
      const uint64_t sk = seg_chosen ? seg_key : 0ull;
      const int src = (lane & ~(LPR - 1)) + LPR - 1 - hl;
      const uint64_t rv = (uint64_t(uint32_t(__shfl(int(uint32_t(sk >> 32)), src, kWave))) << 32) |
                          uint32_t(__shfl(int(uint32_t(sk)), src, kWave));
      uint64_t v = a > rv ? a : rv;
#pragma unroll
      for (int j = LPR / 2; j > 0; j >>= 1) {
        const uint64_t y = (uint64_t(xlane_u32(uint32_t(v >> 32), j)) << 32) | xlane_u32(uint32_t(v), j);
        v = ((hl & j) == 0) ? (v > y ? v : y) : (v < y ? v : y);
      }
      mine = v;
      chosen = hl < keep_n && v != 0ull;
    }
  }
  // 4. Kept leaves (lanes < keep_n), forced leaves appended, ascending.
  int node = chosen ? int(0xffffffffu - uint32_t(mine)) : -1;
  if (keep_all) {
    node = hl < n_el ? hl : -1;
  } else if (cz) {
    if (hl == keep_n) node = cur;
    if (fz && hl == keep_n + 1 && cur >= 1) node = 0;
    if (fz && hl == keep_n + 2 && cur >= 2) node = cur - 1;
  }
  const uint32_t o_sorted = row_sort_desc32<LPR>(node >= 0 ? 0xffffffffu - uint32_t(node) : 0u, hl);
  const int out = o_sorted ? int(0xffffffffu - o_sorted) : -1;
  if (live && hl < topk) {
    idx[row * topk + hl] = out;
    if (score) {
      const bool unranked = keep_all || (cz & ((out == cur) | (fz & ((out == 0) | (out == cur - 1)))));
      score[row * topk + hl] = out < 0 ? neg_inf() : (unranked ? pos_inf() : srow[out]);
    }
  }
}

// Score matrix plus 16 bytes of slack for the Top-K pass's 16-byte row reads.
static size_t scores_bytes(const LaunchShape& s) {
  return ((size_t)s.batch * s.heads_kv * s.seq_len * s.lv.size[0] * sizeof(float) + 16 + 255) &
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

template <int LPR, int VPL, bool kLong = false>
static hipError_t launch_bsa_topk_rows_t(const LaunchShape& s, const float* S, int32_t* idx,
                                         float* score, hipStream_t st) {
  constexpr int ROWS = 256 / LPR;
  dim3 grid((s.seq_len + ROWS - 1) / ROWS, s.batch * s.heads_kv);
  prof::Scope ps("bsa_topk", st);
  hipLaunchKernelGGL((bsa_topk_rows_kernel<LPR, VPL, kLong>), grid, dim3(256), 0, st, S, idx, score,
                     s.seq_len, s.block, s.lv.size[0], s.topk, s.causal ? 1 : 0, s.force ? 1 : 0);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_bsa_mfma_t(const LaunchShape& s, const void* q, const float* pyr,
                                    float* S, bf16_t* planes, hipStream_t st) {
  const int m1 = s.lv.size[0];
  const size_t n = (size_t)s.batch * s.heads_kv * m1 * D;
  {
    prof::Scope ps("bsa_split", st);
    hipLaunchKernelGGL(bsa_split_kernel, dim3((unsigned)std::min<size_t>(65536, (n + 255) / 256)),
                       dim3(256), 0, st, pyr, planes, s.lv.rows, m1, D, n);
  }
  dim3 grid((s.seq_len + kMfmaQ - 1) / kMfmaQ, s.batch * s.heads_kv);
  prof::Scope ps("bsa_scores", st);
  hipLaunchKernelGGL((bsa_scores_mfma_kernel<D, G>), grid, dim3(256), 0, st,
                     static_cast<const bf16_t*>(q), planes, S, s.heads_q, s.heads_kv, s.seq_len,
                     s.block, m1, s.causal ? 1 : 0, s.force ? 1 : 0, s.scale, n);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bsa_mfma_d(const LaunchShape& s, const void* q, const float* pyr,
                                    float* S, bf16_t* planes, hipStream_t st) {
  switch (s.group) {
    case 1: return launch_bsa_mfma_t<D, 1>(s, q, pyr, S, planes, st);
    case 2: return launch_bsa_mfma_t<D, 2>(s, q, pyr, S, planes, st);
    case 4: return launch_bsa_mfma_t<D, 4>(s, q, pyr, S, planes, st);
    case 8: return launch_bsa_mfma_t<D, 8>(s, q, pyr, S, planes, st);
    default: return launch_bsa_mfma_t<D, 16>(s, q, pyr, S, planes, st);
  }
}

hipError_t launch_bsa(const LaunchShape& s, const void* q, const float* pyr, int32_t* idx,
                      float* score, void* ws, hipStream_t st) {
  float* S = static_cast<float*>(ws);
  hipError_t e;
  const int m1 = s.lv.size[0];
  // MFMA scores for bf16 with a power-of-two group; else fp32 FMA tiles.
  if (s.bf16 && (s.group & (s.group - 1)) == 0) {
    bf16_t* planes = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + scores_bytes(s));
    e = s.head_dim == 128 ? launch_bsa_mfma_d<128>(s, q, pyr, S, planes, st)
                          : launch_bsa_mfma_d<64>(s, q, pyr, S, planes, st);
    if (e != hipSuccess) return e;
    // Rows written by the MFMA kernel (forced leaves and padding at -inf).
    if (m1 % 4 == 0) {
      if (m1 <= 32 * 16) return launch_bsa_topk_rows_t<32, 16>(s, S, idx, score, st);
      if (m1 <= 32 * 32) return launch_bsa_topk_rows_t<32, 32>(s, S, idx, score, st);
      if (m1 <= 32 * 64) return launch_bsa_topk_rows_t<32, 64>(s, S, idx, score, st);
      constexpr int V = kBsaMaxLeaves / kWave;
      if (m1 <= kBsaMaxLeaves) return launch_bsa_topk_rows_t<64, V>(s, S, idx, score, st);
      return launch_bsa_topk_rows_t<64, V, true>(s, S, idx, score, st);
    }
  } else if (s.bf16) {
    e = s.head_dim == 128 ? launch_bsa_scores_t<bf16_t, 128>(s, q, pyr, S, st)
                          : launch_bsa_scores_t<bf16_t, 64>(s, q, pyr, S, st);
  } else {
    e = s.head_dim == 128 ? launch_bsa_scores_t<float, 128>(s, q, pyr, S, st)
                          : launch_bsa_scores_t<float, 64>(s, q, pyr, S, st);
  }
  if (e != hipSuccess) return e;
  if (m1 <= 4 * kWave) return launch_bsa_topk_t<4>(s, S, idx, score, st);
  if (m1 <= 16 * kWave) return launch_bsa_topk_t<16>(s, S, idx, score, st);
  if (m1 <= 32 * kWave) return launch_bsa_topk_t<32>(s, S, idx, score, st);
  return launch_bsa_topk_t<kBsaMaxLeaves / kWave>(s, S, idx, score, st);
}

}  // namespace pisa
