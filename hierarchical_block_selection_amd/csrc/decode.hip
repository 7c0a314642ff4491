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
    int heads_kv, int capacity, int block, int topk, int group, int force, int variant,
    float scale_log2, LevelTable lv) {
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
                                              true, force != 0, scale_log2, nbuf, false, variant);
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

namespace {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecMaxK = 16;  // 2K candidates fit one 32-lane half-wave

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// One Top-K decision over the candidates held by lanes 0..31 (lane j = slot
// j, ascending nodes): keep all when at most K are valid, else the forced
// ones plus the best K - #F rankable ones.  Returns the kept-slot mask.
__device__ __forceinline__ uint32_t decide32(bool valid, bool forced, float score, int topk) {
  const int lane = lane_id();
  const uint32_t vm = uint32_t(__ballot(valid & (lane < 32)));
  if (__popc(vm) <= topk) return vm;
  const bool fz = valid & forced & (lane < 32);
  const uint32_t fm = uint32_t(__ballot(fz));
  const int keep_n = topk - __popc(fm);
  const bool rankable = valid & !forced & (lane < 32);
  // best rankable score of the decision (xor shuffles stay inside 32-lane halves)
  float smax = rankable ? score : neg_inf();
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) smax = fmaxf(smax, __shfl_xor(smax, o, kWave));
  uint32_t key = rankable ? rank_key_rel(score, smax, lane) : 0u;
  // bitonic sort, descending, inside each 32-lane half
#pragma unroll
  for (int k = 2; k <= 32; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t y = uint32_t(__shfl_xor(int(key), j, kWave));
      const bool desc = ((lane & k) == 0) || k == 32;
      const bool lower = (lane & j) == 0;
      key = (desc == lower) ? max(key, y) : min(key, y);
    }
  uint32_t km = fm;
  for (int i = 0; i < keep_n; ++i) {
    const uint32_t kk = uint32_t(__builtin_amdgcn_readlane(int(key), i));
    km |= 1u << (31 - (kk & 31u));
  }
  return km;
}

// One decode step for one (sequence, KV head) per workgroup (bf16, C = 64,
// K <= 16): the descent of the PISA reading page §4.2 at t = cache_len - 1
// over the cache's pyramid (§5.1 single fused stage, §5.3 forcing), then
// eq. (2) over the kept blocks for every query head of the group.
//   levels L..2: the 2 * #A child summaries (fp32) are scored by all threads
//                (4 threads per row), one wave ranks the candidates;
//   leaves:      the raw keys of every candidate leaf go through bf16 MFMA
//                (keys x heads), exact LSE per head, summed over the group;
//   attention:   the kept leaves are split over the waves, each running an
//                online softmax (logits again on MFMA, P V on the vector
//                units, lanes over the head dimension); the waves' partial
//                results are merged through LDS.
template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_wg_kernel(
    const int32_t* __restrict__ cache_len, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, const float* __restrict__ pyr,
    int32_t* __restrict__ idx, float* __restrict__ score, bf16_t* __restrict__ out,
    float* __restrict__ lse, int heads_q, int heads_kv, int capacity, int topk, int force,
    float scale_log2, LevelTable lv) {
  constexpr int C = 64;
  constexpr int KSTEPS = D / 16;
  constexpr int TPR = kDecThreads / 64;  // threads per child row (64 rows)
  constexpr int DP = D / TPR;             // dims per thread in the child-summary dots
  constexpr int DL = D / kWave;       // output dims per lane in P V
  __shared__ float q_s[G][D];
  __shared__ float z_s[64][G];
  __shared__ float leaf_s[32];
  __shared__ int kept_s[kDecMaxK + 1];
  __shared__ int nk_s;
  __shared__ float lg_s[32][C][G];  // candidate logits (log2 units), later probabilities
  __shared__ float cm_s[32][G];      // candidate max logit per head
  __shared__ int kept_j_s[kDecMaxK];
  __shared__ float po_s[kDecWaves][G][D];
  __shared__ float pl_s[kDecWaves][G];
  __shared__ float mh_s[G];
  const int bh = blockIdx.x;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int n = cache_len[b];
  const size_t head0 = (size_t)b * heads_q + (size_t)kvh * G;
  int32_t* idx_row = idx + (size_t)bh * topk;
  float* score_row = score ? score + (size_t)bh * topk : nullptr;
  if (n < 1 || n > capacity) {  // no valid cache: empty selection, zero output
    if (tid < topk) {
      idx_row[tid] = -1;
      if (score_row) score_row[tid] = neg_inf();
    }
    for (int x = tid; x < G * D; x += kDecThreads) out[head0 * D + x] = 0;
    if (lse && tid < G) lse[head0 + tid] = neg_inf();
    return;
  }
  const int t = n - 1, cur = t / C;
  const bool fz = force != 0;
  for (int x = tid; x < G * D; x += kDecThreads) q_s[x / D][x % D] = bf16_to_f32(q[head0 * D + x]);
  if (tid == 0) {
    kept_s[0] = 0;
    nk_s = 1;
  }
  // MFMA B operands: column h < G is query head h (zero elsewhere).
  const int col = lane & 31, kh = lane >> 5;
  bf16x8_t bq[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < G) v = *reinterpret_cast<const uint4*>(q + (head0 + col) * D + 16 * s + 8 * kh);
    bq[s] = as_bf16x8(v);
  }
  __syncthreads();
  const float* pb = pyr + (size_t)bh * lv.rows * D;
  const bf16_t* kb = kc + (size_t)bh * capacity * D;
  const bf16_t* vb = vc + (size_t)bh * capacity * D;

  // Levels L..2.
  for (int l = lv.n; l >= 2; --l) {
    const int sh = l - 1;
    const int size_l = lv.size[l - 1];
    const int lim = cur >> sh;
    const int x_max = min(size_l - 1, lim);
    const int nk = nk_s;
    int n_valid = 0;
    for (int i = 0; i < nk; ++i) {
      const int c = 2 * kept_s[i];
      n_valid += int(c <= x_max) + int(c + 1 <= x_max);
    }
    const int m_child = lv.size[l - 2];
    if (n_valid > topk) {
      // child row r of candidate r / 2; TPR threads per row
      const int r = tid / TPR, part = tid % TPR;
      const int j = r >> 1;
      const int cnode = 2 * kept_s[min(j >> 1, kDecMaxK)] + (j & 1);
      const int crow = 2 * cnode + (r & 1);
      const bool live = (j < n_valid) & (crow < m_child);
      const float* xr = pb + ((size_t)lv.off[l - 2] + (live ? crow : 0)) * D + part * DP;
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < DP; c4 += 4) {
        const float4 x = *reinterpret_cast<const float4*>(xr + c4);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float* qh = &q_s[h][part * DP + c4];
          acc[h] += qh[0] * x.x + qh[1] * x.y + qh[2] * x.z + qh[3] * x.w;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float v = acc[h];
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) v += __shfl_xor(v, o, kWave);
        if (part == 0) z_s[r][h] = live ? v * scale_log2 : neg_inf();
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int j = lane & 31;
      const int node = 2 * kept_s[min(j >> 1, kDecMaxK)] + (j & 1);
      const bool valid = (lane < 32) & (j < n_valid);
      uint32_t km;
      if (n_valid > topk) {
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float a = z_s[2 * j][h], c = z_s[2 * j + 1][h];
          const float mx = fmaxf(a, c), mn = fminf(a, c);
          sc += mx + fast_log2(1.f + fast_exp2(mn - mx));
        }
        const int prev = cur >= 1 ? (cur - 1) >> sh : -1;
        const bool forced = (node == lim) | (fz & ((node == 0) | (node == prev)));
        km = decide32(valid, forced, sc, topk);
      } else {
        km = uint32_t(__ballot(valid));
      }
      const bool k = (lane < 32) & ((km >> j) & 1u);
      wave_lds_sync();
      if (k) kept_s[min(int(__popc(km & ((1u << j) - 1u))), kDecMaxK)] = node;
      if (lane == 0) nk_s = min(int(__popc(km)), kDecMaxK);
    }
    __syncthreads();
  }

  // Leaf level: candidates are the leaves under the kept level-2 nodes.
  const int nk2 = nk_s;
  int n_valid = 0;
  for (int i = 0; i < nk2; ++i) {
    const int c = 2 * kept_s[i];
    n_valid += int(c <= cur) + int(c + 1 <= cur);
  }
  const bool ranked = n_valid > topk;
  {
    // Wave w scores candidates w * PER .. ; the raw keys of two candidates are
    // requested together (a candidate past the list loads a valid leaf and
    // its result is dropped).  The logits stay in LDS for the attention.
    constexpr int PER = 32 / kDecWaves;
    const int last_leaf = 2 * kept_s[(n_valid - 1) >> 1] + ((n_valid - 1) & 1);
#pragma unroll
    for (int jj = 0; jj < PER; jj += 2) {
      uint4 kr[2][2][KSTEPS];
      int leaf2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = wave * PER + jj + u;
        leaf2[u] = j < n_valid ? 2 * kept_s[j >> 1] + (j & 1) : last_leaf;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int tok = min(leaf2[u] * C + 32 * rb + col, capacity - 1);
          const bf16_t* kp = kb + (size_t)tok * D + 8 * kh;
#pragma unroll
          for (int s2 = 0; s2 < KSTEPS; ++s2) kr[u][rb][s2] = *reinterpret_cast<const uint4*>(kp + 16 * s2);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = wave * PER + jj + u;
        const int leaf = leaf2[u];
        f32x16_t acc[2] = {};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int s2 = 0; s2 < KSTEPS; ++s2)
            acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[u][rb][s2]), bq[s2],
                                                              acc[rb], 0, 0, 0);
        // lane: head col, keys (i/4)*8 + 4kh + i%4 (+32 in acc[1])
        float m = neg_inf();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = leaf * C + 32 * rb + (i / 4) * 8 + 4 * kh + (i % 4);
            acc[rb][i] = tok <= t ? acc[rb][i] * scale_log2 : neg_inf();
            m = fmaxf(m, acc[rb][i]);
          }
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        if (col < G && j < n_valid) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              lg_s[j][32 * rb + (i / 4) * 8 + 4 * kh + (i % 4)][col] = acc[rb][i];
          if (kh == 0) cm_s[j][col] = m;
        }
        float se = 0.f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) se += fast_exp2(acc[rb][i] - m);
        se += __shfl_xor(se, 32, kWave);
        float v = col < G ? m + fast_log2(se) : 0.f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o, kWave);
        if (lane == 0 && j < n_valid) leaf_s[j] = v;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int j = lane & 31;
    const int leaf = 2 * kept_s[min(j >> 1, kDecMaxK)] + (j & 1);
    const bool valid = (lane < 32) & (j < n_valid);
    const bool forced = (leaf == cur) | (fz & ((leaf == 0) | (leaf == cur - 1)));
    const float sc = ranked && valid ? leaf_s[j] : 0.f;
    const uint32_t km = ranked ? decide32(valid, forced, sc, topk) : uint32_t(__ballot(valid));
    const bool k = (lane < 32) & ((km >> j) & 1u);
    const int pos = __popc(km & ((1u << j) - 1u));
    const int nsel = min(int(__popc(km)), kDecMaxK);
    wave_lds_sync();
    if (k && pos < kDecMaxK) {
      kept_s[pos] = leaf;
      kept_j_s[pos] = j;
      idx_row[pos] = leaf;
      if (score_row) score_row[pos] = (ranked && !forced) ? sc * kLn2 : pos_inf();
    }
    if (lane >= nsel && lane < topk) {
      idx_row[lane] = -1;
      if (score_row) score_row[lane] = neg_inf();
    }
    if (lane == 0) nk_s = nsel;
  }
  __syncthreads();

  // Attention over the kept leaves, from the logits kept in LDS: one shared
  // maximum per head, so the waves' partial sums add without rescaling.
  // Wave w takes kept leaves w, w + kDecWaves; their value rows are all
  // requested before use.
  const int nsel = nk_s;
  float Mh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Mh[h] = neg_inf();
    for (int i = 0; i < nsel; ++i) Mh[h] = fmaxf(Mh[h], cm_s[kept_j_s[i]][h]);
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (tid == h) mh_s[h] = Mh[h];
  float lsum[G], o[G][DL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[h][e] = 0.f;
  }
  constexpr int PERW = (kDecMaxK + kDecWaves - 1) / kDecWaves;
  uint32_t vw[PERW][C];
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const int i = min(wave + u * kDecWaves, nsel - 1);
    const int leaf = kept_s[i];
    // rows after t (probability 0) repeat row t, which is inside the cache
    const int last = t - leaf * C;  // >= 0: a kept leaf is never in the future
    const bf16_t* vr = vb + (size_t)leaf * C * D + lane * DL;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      const int rr = min(r, last);
      if constexpr (DL == 2)
        vw[u][r] = *reinterpret_cast<const uint32_t*>(vr + (size_t)rr * D);
      else
        vw[u][r] = uint32_t(vr[(size_t)rr * D]) << 16;
    }
  }
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const int i = wave + u * kDecWaves;
    if (i >= nsel) break;
    const int j = kept_j_s[i];
    // probabilities in place: lane = key, every head
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pv = fast_exp2(lg_s[j][lane][h] - Mh[h]);
      lg_s[j][lane][h] = pv;
      lsum[h] += pv;
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float vv[DL];
      if constexpr (DL == 2) {
        vv[0] = __uint_as_float(vw[u][r] << 16);
        vv[1] = __uint_as_float(vw[u][r] & 0xffff0000u);
      } else {
        vv[0] = __uint_as_float(vw[u][r]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = lg_s[j][r][h];
#pragma unroll
        for (int e = 0; e < DL; ++e) o[h][e] += pr * vv[e];
      }
    }
  }
  // Merge the waves' partial sums.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = lsum[h];
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
#pragma unroll
    for (int e = 0; e < DL; ++e) po_s[wave][h][lane * DL + e] = o[h][e];
    if (lane == 0) pl_s[wave][h] = v;
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kDecThreads) {
    const int h = x / D, d = x % D;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      L += pl_s[w][h];
      O += po_s[w][h][d];
    }
    out[(head0 + h) * D + d] = f32_to_bf16(L > 0.f ? O / L : 0.f);
    if (lse && d == 0) lse[head0 + h] = L > 0.f ? (mh_s[h] + fast_log2(L)) * kLn2 : neg_inf();
  }
}

bool decode_wg_supported(const LaunchShape& s) {
  const bool g_ok = s.group == 1 || s.group == 2 || s.group == 4 || s.group == 8;
  return s.bf16 && s.block == 64 && (s.head_dim == 64 || s.head_dim == 128) && g_ok &&
         s.topk <= kDecMaxK && s.causal && s.lv.n >= 2 && s.variant == 0;
}

template <int D, int G>
hipError_t launch_decode_wg(const LaunchShape& s, const int32_t* cache_len, const void* q,
                            const void* kc, const void* vc, const float* pyr, int32_t* idx,
                            float* score, void* out, float* lse, hipStream_t st) {
  prof::Scope ps("decode", st);
  hipLaunchKernelGGL((decode_wg_kernel<D, G>), dim3(s.batch * s.heads_kv), dim3(kDecThreads), 0,
                     st, cache_len, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(kc),
                     static_cast<const bf16_t*>(vc), pyr, idx, score, static_cast<bf16_t*>(out),
                     lse, s.heads_q, s.heads_kv, s.seq_len, s.topk, s.force ? 1 : 0,
                     s.scale * kLog2e, s.lv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_wg_d(const LaunchShape& s, const int32_t* cache_len, const void* q,
                              const void* kc, const void* vc, const float* pyr, int32_t* idx,
                              float* score, void* out, float* lse, hipStream_t st) {
  switch (s.group) {
    case 1: return launch_decode_wg<D, 1>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
    case 2: return launch_decode_wg<D, 2>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
    case 4: return launch_decode_wg<D, 4>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
    default: return launch_decode_wg<D, 8>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
  }
}

}  // namespace

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
                     s.variant, s.scale * kLog2e, s.lv);
  return hipGetLastError();
}

size_t decode_ws_bytes(const LaunchShape&) { return 0; }

hipError_t launch_decode(const LaunchShape& s, const int32_t* cache_len, const void* q,
                         const void* kc, const void* vc, const float* pyr, int32_t* idx,
                         float* score, void* out, float* lse, void* /*ws*/, hipStream_t st) {
  if (decode_wg_supported(s))
    return s.head_dim == 128
               ? launch_decode_wg_d<128>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st)
               : launch_decode_wg_d<64>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
  if (s.bf16)
    return s.head_dim == 128
               ? launch_decode_t<bf16_t, 128>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st)
               : launch_decode_t<bf16_t, 64>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
  return s.head_dim == 128
             ? launch_decode_t<float, 128>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st)
             : launch_decode_t<float, 64>(s, cache_len, q, kc, vc, pyr, idx, score, out, lse, st);
}

}  // namespace pisa
