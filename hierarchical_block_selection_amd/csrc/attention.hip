// Block-sparse attention over the selected leaf blocks (PISA reading page §02
// eq. (2), causal mask of §5.3).
//
// bf16, C = 64 (block path): a (query row, selected block) pair moves only the
// query (d bf16) and a partial result instead of the block's 2*C*d key/value
// bytes.  Pairs are bucketed by block; one workgroup per (block, <= 256 pairs)
// keeps K_b (row-major) and V_b (transposed) in LDS and, per 32 (query, head)
// columns, runs S = K_b Q^T and O = P V_b as bf16 MFMA 32x32x16 with fp32
// accumulation, masks keys after t, and writes the block's normalised output
// (bf16) and its log2-sum-exp.  A combine pass merges the K partials of each
// row with the usual max-rescaled weights.  V is stored transposed so that the
// probabilities held in the QK^T accumulators feed the PV product directly:
// the key order inside the PV reduction is permuted to match the accumulator
// layout, which leaves the sum unchanged.
//
// Other cases (fp32, other C): per-query form, one wavefront per (batch, query
// head, position) running attend_wave over the K blocks.
#include "attn_core.h"
#include "bucket.h"
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
  prof::Scope ps("attn_query", st);
  hipLaunchKernelGGL((attn_query_kernel<T, D>), grid, dim3(kAttnWaves * kWave), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     idx, static_cast<T*>(out), lse, s.heads_q, s.heads_kv, s.seq_len, s.block,
                     s.topk, s.group, s.causal ? 1 : 0, s.scale * kLog2e);
  return hipGetLastError();
}

namespace {

constexpr int kAttnBlock = 64;
constexpr int kAttnThreads = 256;
constexpr int kAttnPairsPerItem = 256;
constexpr int kAttnCols = 32;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

struct AttnWs {
  size_t counts, offsets, cursors, item_offsets, pairs, part_o, part_lse, total;
  int n_buckets, max_items;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool block_path(const LaunchShape& s) {
  // (query, slot) pair ids are int32
  const int64_t slots = (int64_t)s.batch * s.heads_kv * s.seq_len * s.topk;
  return s.bf16 && s.block == kAttnBlock && (s.head_dim == 64 || s.head_dim == 128) &&
         (s.group & (s.group - 1)) == 0 && s.group <= kMaxGroup && slots < INT32_MAX;
}

AttnWs attn_layout(const LaunchShape& s) {
  AttnWs w;
  const size_t slots = (size_t)s.batch * s.heads_kv * s.seq_len * s.topk;
  w.n_buckets = s.batch * s.heads_kv * s.lv.size[0];
  w.max_items = bucket::max_items(slots, w.n_buckets, kAttnPairsPerItem);
  size_t off = 0;
  w.counts = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.cursors = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.item_offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.pairs = off; off = align256(off + sizeof(int) * slots);
  w.part_o = off; off = align256(off + sizeof(bf16_t) * slots * s.group * s.head_dim);
  w.part_lse = off; off = align256(off + sizeof(float) * slots * s.group);
  w.total = off;
  return w;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int* __restrict__ item_offsets, const int* __restrict__ offsets,
    const int* __restrict__ pairs, bf16_t* __restrict__ part_o, float* __restrict__ part_lse,
    int n_buckets, int heads_q, int heads_kv, int n_tok, int topk, int group, int m1, int causal,
    float scale_log2) {
  constexpr int C = kAttnBlock;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int KROW = D + 8;  // padded rows against LDS bank conflicts
  constexpr int VROW = C + 8;
  constexpr int NW = kAttnThreads / kWave;
  __shared__ __attribute__((aligned(16))) bf16_t ks[C * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t vt[D * VROW];
  constexpr int OROW = D + 8;  // padded output staging row (bf16)
  __shared__ float inv_l[NW][kAttnCols];
  __shared__ int pid_s[NW][kAttnCols];
  __shared__ __attribute__((aligned(16))) bf16_t obuf[NW][kAttnCols * OROW];
  int bucket, start, len;
  if (!bucket::locate_item(item_offsets, offsets, n_buckets, blockIdx.x, kAttnPairsPerItem,
                           &bucket, &start, &len))
    return;
  const int bh = bucket / m1, blk = bucket % m1;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tok0 = blk * C;
  const int n_keys = min(C, n_tok - tok0);
  const bf16_t* kb = k + ((size_t)bh * n_tok + tok0) * D;
  const bf16_t* vb = v + ((size_t)bh * n_tok + tok0) * D;
  for (int x = threadIdx.x; x < C * (D / 8); x += kAttnThreads) {
    const int r = x / (D / 8), c = (x % (D / 8)) * 8;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (r < n_keys) {
      kv = *reinterpret_cast<const uint4*>(kb + (size_t)r * D + c);
      vv = *reinterpret_cast<const uint4*>(vb + (size_t)r * D + c);
    }
    *reinterpret_cast<uint4*>(&ks[r * KROW + c]) = kv;
    const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(c + 2 * e) * VROW + r] = bf16_t(w4[e] & 0xffffu);
      vt[(c + 2 * e + 1) * VROW + r] = bf16_t(w4[e] >> 16);
    }
  }
  __syncthreads();

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = lane & 31, khalf = lane >> 5;
  const int per_chunk = kAttnCols / group;
  const int n_chunks = (len + per_chunk - 1) / per_chunk;
  const int h = col % group;
  auto load_chunk = [&](int ch, bf16x8_t (&bq)[KSTEPS], int& pair_id, int& t) {
    const int p = ch * per_chunk + col / group;
    pair_id = -1;
    t = 0;
    if (ch < n_chunks && p < len) {
      pair_id = pairs[start + p];
      t = (int)(((size_t)pair_id / topk) % n_tok);
      const bf16_t* qrow = q + (((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t) * D;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        bq[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * khalf));
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  };
  bf16x8_t bq[KSTEPS];
  int pair_id, t;
  load_chunk(wave, bq, pair_id, t);
  bf16_t* ostage = &obuf[wave][0];
  for (int ch = wave; ch < n_chunks; ch += NW) {
    bf16x8_t bn[KSTEPS];
    int pair_next, t_next;
    load_chunk(ch + NW, bn, pair_next, t_next);  // prefetch the next chunk
    f32x16_t s0 = {}, s1 = {};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8_t a0 =
          as_bf16x8(*reinterpret_cast<const uint4*>(&ks[col * KROW + 16 * s + 8 * khalf]));
      const bf16x8_t a1 =
          as_bf16x8(*reinterpret_cast<const uint4*>(&ks[(32 + col) * KROW + 16 * s + 8 * khalf]));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bq[s], s1, 0, 0, 0);
    }
    // Lane holds raw logits of key rows (i/4)*8 + khalf*4 + i%4 (+32 in s1) for column col.
    int lim = n_keys - 1;
    if (causal) lim = min(lim, t - tok0);
    if (pair_id < 0) lim = -1;
    const bool any_masked = __ballot(lim < C - 1) != 0;
    if (any_masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = (i / 4) * 8 + khalf * 4 + (i % 4);
        s0[i] = r <= lim ? s0[i] : neg_inf();
        s1[i] = r + 32 <= lim ? s1[i] : neg_inf();
      }
    }
    float m = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fmaxf(s0[i], s1[i]));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    const float ms = m == neg_inf() ? 0.f : m * scale_log2;  // column without keys
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = fast_exp2(fmaf(s0[i], scale_log2, -ms));
      s1[i] = fast_exp2(fmaf(s1[i], scale_log2, -ms));
      l += s0[i] + s1[i];
    }
    l += __shfl_xor(l, 32, kWave);
    // O = P V: A = P (rows = columns of S), k-step s covers 16 keys.
    f32x16_t o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t pa;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = s < 2 ? s0[8 * s + j] : s1[8 * (s - 2) + j];
        pa[j] = __builtin_bit_cast(__bf16, f32_to_bf16(x));
      }
      const int kbase = 32 * (s / 2) + 16 * (s % 2) + 4 * khalf;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const bf16_t* vrow = &vt[(32 * db + col) * VROW + kbase];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        const bf16x8_t vbop = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vbop, o[db], 0, 0, 0);
      }
    }
    if (khalf == 0) {
      inv_l[wave][col] = l > 0.f ? 1.f / l : 0.f;
      pid_s[wave][col] = pair_id;
      if (pair_id >= 0) part_lse[(size_t)pair_id * group + h] = ms + fast_log2(l);
    }
    wave_lds_sync();
    // o[db][i] = O[row (i/4)*8 + khalf*4 + i%4][d = 32*db + col] -> LDS [row][d] (bf16)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (i / 4) * 8 + khalf * 4 + (i % 4);
      const float inv = inv_l[wave][r];
#pragma unroll
      for (int db = 0; db < DBLK; ++db) ostage[r * OROW + 32 * db + col] = f32_to_bf16(o[db][i] * inv);
    }
    wave_lds_sync();
    // 16-byte stores: each row is D bf16 = D/8 chunks.
    constexpr int CH_PER_ROW = D / 8;
#pragma unroll
    for (int x = lane; x < 32 * CH_PER_ROW; x += kWave) {
      const int r = x / CH_PER_ROW, c8 = (x % CH_PER_ROW) * 8;
      const int pr = pid_s[wave][r];
      if (pr >= 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(&ostage[r * OROW + c8]);
        *reinterpret_cast<uint4*>(part_o + ((size_t)pr * group + (r % group)) * D + c8) = v;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bq[s] = bn[s];
    pair_id = pair_next;
    t = t_next;
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ part_o,
    const float* __restrict__ part_lse, bf16_t* __restrict__ out, float* __restrict__ lse_out,
    int heads_q, int heads_kv, int n_tok, int topk, int group, int m1, size_t n_rows) {
  constexpr int EPL = D / 16;  // elements per lane (16 lanes per row)
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 16;
  if (row >= n_rows) return;
  const int sub = threadIdx.x & 15;
  const size_t u = row / group;
  const int h = (int)(row % group);
  const int t = (int)(u % n_tok);
  const size_t bh = u / n_tok;
  const int b = (int)(bh / heads_kv), kvh = (int)(bh % heads_kv);
  const int32_t* ir = idx + u * topk;
  float M = neg_inf();
  for (int j = 0; j < topk; ++j) {
    const int x = ir[j];
    if (x >= 0 && x < m1) M = fmaxf(M, part_lse[(u * topk + j) * group + h]);
  }
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float W = 0.f;
  if (M != neg_inf()) {
    for (int j = 0; j < topk; ++j) {
      const int x = ir[j];
      if (x < 0 || x >= m1) continue;
      const size_t pi = (u * topk + j) * group + h;
      const float w = fast_exp2(part_lse[pi] - M);
      W += w;
      const bf16_t* src = part_o + pi * D + sub * EPL;
      float vals[8];
      if (EPL == 8) {
        load16(src, vals);
      } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(src);
        vals[0] = __uint_as_float(raw.x << 16);
        vals[1] = __uint_as_float(raw.x & 0xffff0000u);
        vals[2] = __uint_as_float(raw.y << 16);
        vals[3] = __uint_as_float(raw.y & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += w * vals[e];
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  bf16_t* dst = out + (((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t) * D + sub * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = f32_to_bf16(acc[e] * inv);
  if (lse_out && sub == 0) {
    lse_out[((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t] =
        W > 0.f ? (M + fast_log2(W)) * kLn2 : neg_inf();
  }
}

template <int D>
hipError_t launch_block_path(const LaunchShape& s, const void* q, const void* k, const void* v,
                             const int32_t* idx, void* out, float* lse, void* ws, hipStream_t st) {
  const AttnWs lay = attn_layout(s);
  char* base = static_cast<char*>(ws);
  int* counts = reinterpret_cast<int*>(base + lay.counts);
  int* offsets = reinterpret_cast<int*>(base + lay.offsets);
  int* cursors = reinterpret_cast<int*>(base + lay.cursors);
  int* item_offsets = reinterpret_cast<int*>(base + lay.item_offsets);
  int* pairs = reinterpret_cast<int*>(base + lay.pairs);
  bf16_t* part_o = reinterpret_cast<bf16_t*>(base + lay.part_o);
  float* part_lse = reinterpret_cast<float*>(base + lay.part_lse);
  const int m1 = s.lv.size[0];
  hipError_t e;
  {
    prof::Scope ps("attn_sort", st);
    e = bucket::sort_pairs(idx, s.batch * s.heads_kv, s.seq_len, s.topk, m1,
                                    kAttnPairsPerItem, counts, offsets, cursors, item_offsets,
                                    pairs, false, st);
  }
  if (e != hipSuccess) return e;
  {
  prof::Scope ps("attn_partial", st);
  hipLaunchKernelGGL((attn_partial_kernel<D>), dim3(lay.max_items), dim3(kAttnThreads), 0, st,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), item_offsets, offsets, pairs, part_o,
                     part_lse, lay.n_buckets, s.heads_q, s.heads_kv, s.seq_len, s.topk, s.group,
                     m1, s.causal ? 1 : 0, s.scale * kLog2e);
  }
  prof::Scope ps("attn_combine", st);
  const size_t rows = (size_t)s.batch * s.heads_kv * s.seq_len * s.group;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)((rows * 16 + 255) / 256)),
                     dim3(256), 0, st, idx, part_o, part_lse, static_cast<bf16_t*>(out), lse,
                     s.heads_q, s.heads_kv, s.seq_len, s.topk, s.group, m1, rows);
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_bytes(const LaunchShape& s) { return block_path(s) ? attn_layout(s).total : 0; }

hipError_t launch_attn(const LaunchShape& s, const void* q, const void* k, const void* v,
                       const int32_t* idx, void* out, float* lse, void* ws, hipStream_t st) {
  if (block_path(s))
    return s.head_dim == 128 ? launch_block_path<128>(s, q, k, v, idx, out, lse, ws, st)
                             : launch_block_path<64>(s, q, k, v, idx, out, lse, ws, st);
  if (s.bf16)
    return s.head_dim == 128 ? launch_attn_t<bf16_t, 128>(s, q, k, v, idx, out, lse, st)
                             : launch_attn_t<bf16_t, 64>(s, q, k, v, idx, out, lse, st);
  return s.head_dim == 128 ? launch_attn_t<float, 128>(s, q, k, v, idx, out, lse, st)
                           : launch_attn_t<float, 64>(s, q, k, v, idx, out, lse, st);
}

}  // namespace pisa
