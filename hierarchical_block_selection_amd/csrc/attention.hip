// Block-sparse attention over the selected leaf blocks (PISA reading page §02
// eq. (2), causal mask of §5.3).
//
// bf16, C = 64 (block path): a (query row, selected block) pair moves only the
// query (d bf16) and a partial result instead of the block's 2*C*d key/value
// bytes.  Pairs are bucketed by block; one workgroup per (block, <= 1024
// (pair, head) rows) keeps K_b (row-major) and V_b (transposed) in LDS and,
// per 32 (query, head) columns, runs S = K_b Q^T and O = P V_b as bf16 MFMA
// 32x32x16 with fp32 accumulation, masks keys after t, and writes the
// block's normalised output (bf16) and its log2-sum-exp.  A combine pass
// merges the K partials of each row with the usual max-rescaled weights.  V is stored transposed so that the
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
constexpr int kAttnRows = 128;   // (pair, head) rows per batch
constexpr int kAttnBatches = 8;  // batches per work item
constexpr int kAttnCols = 32;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

struct AttnWs {
  size_t counts, offsets, cursors, item_offsets, pairs, inv, part_o, part_lse, total;
  int n_buckets, max_items;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool block_path(const LaunchShape& s) {
  // pairs are stored as (row << 5) | slot in an int32; slot ids index int32 maps
  const int64_t rows = (int64_t)s.batch * s.heads_kv * s.seq_len;
  return s.bf16 && s.block == kAttnBlock && (s.head_dim == 64 || s.head_dim == 128) &&
         (s.group & (s.group - 1)) == 0 && s.group <= kMaxGroup && rows < (int64_t(1) << 26);
}

AttnWs attn_layout(const LaunchShape& s) {
  AttnWs w;
  const size_t slots = (size_t)s.batch * s.heads_kv * s.seq_len * s.topk;
  w.n_buckets = s.batch * s.heads_kv * s.lv.size[0];
  w.max_items = bucket::max_items(slots, w.n_buckets, kAttnRows / s.group * kAttnBatches);
  size_t off = 0;
  w.counts = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.cursors = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.item_offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.pairs = off; off = align256(off + sizeof(int) * slots);
  w.inv = off; off = align256(off + sizeof(int) * slots);
  w.part_o = off; off = align256(off + sizeof(bf16_t) * slots * s.group * s.head_dim);
  w.part_lse = off; off = align256(off + sizeof(float) * slots * s.group);
  w.total = off;
  return w;
}

// One workgroup per work item: leaf block blk of KV head bh and up to
// kAttnBatches batches of kAttnRows / G of the (query, slot) pairs that
// selected it.  K_blk (row-major) and V_blk (transposed) sit in LDS for the
// whole item; in every batch wave w takes the 32-column chunk w of the
// batch's (pair, head) rows, loading its query rows at the batch's start
// (no register prefetch: at 168 VGPRs and 53 KB of LDS three workgroups
// share a CU and cover each other's loads).  Per chunk:
//   S^T = K_blk Q^T   (MFMA A = keys from LDS, B = queries; a lane holds the
//                      logits of 32 keys for one column)
//   P   = exp2(S * scale - m) in fp32, row sum l, then bf16
//   O^T = V_blk^T P^T (MFMA A = V^T from LDS, B = P straight from the S
//                      accumulators; the key order inside this reduction is
//                      permuted to match the accumulator layout)
// Each lane then holds 16 output dims of its own column and scales them by
// 1/l; the chunk's rows (contiguous in bucket order) pass through an LDS tile
// and leave as 1 KB store instructions, with each column's log2-sum-exp.
template <int D, int G, int NCH, int KSTEPS>
__device__ __forceinline__ void attn_fetch(bf16x8_t (&bq)[NCH][KSTEPS], int (&pid)[NCH],
                                           int (&tq)[NCH], const int* __restrict__ pairs,
                                           int start, int len, int bt, int wave, int col, int kh,
                                           const bf16_t* __restrict__ qh, int bh, int n_tok,
                                           int topk) {
  constexpr int NW = kAttnThreads / kWave;
  const int rows = len * G;
  const int h = col % G;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int r = min(bt * kAttnRows + (wave + NW * c) * kAttnCols + col, rows - 1);
    pid[c] = pairs[start + r / G];
    tq[c] = (pid[c] >> 5) - bh * n_tok;  // pair = (row << 5) | slot
    const bf16_t* qrow = qh + ((size_t)h * n_tok + tq[c]) * D + 8 * kh;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bq[c][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * s));
  }
}

template <int D, int G>
__global__ __launch_bounds__(kAttnThreads, 3) void attn_partial_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int* __restrict__ item_offsets, const int* __restrict__ offsets,
    const int* __restrict__ pairs, bf16_t* __restrict__ part_o, float* __restrict__ part_lse,
    int n_buckets, int heads_q, int heads_kv, int n_tok, int topk, int m1, int causal,
    float scale_log2) {
  constexpr int C = kAttnBlock;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int KROW = D + 8;  // padded rows (bf16) against LDS bank conflicts
  constexpr int VROW = C + 4;
  constexpr int NW = kAttnThreads / kWave;
  constexpr int PAIRS = kAttnRows / G;             // pairs per batch
  constexpr int NCH = kAttnRows / kAttnCols / NW;  // chunks per wave and batch
  __shared__ __attribute__((aligned(16))) bf16_t ks[C * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t vt[D * VROW];
  constexpr int OROW = D / 2 + 8;  // padded output tile row (bf16): half of d per pass
  __shared__ __attribute__((aligned(16))) bf16_t os[NW][kAttnCols * OROW];
  int bucket, start, len;
  if (!bucket::locate_item(item_offsets, offsets, n_buckets, blockIdx.x, PAIRS * kAttnBatches,
                           &bucket, &start, &len))
    return;
  const int bh = bucket / m1, blk = bucket % m1;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tok0 = blk * C;
  const int n_keys = min(C, n_tok - tok0);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int col = lane & 31, kh = lane >> 5;
  const int h = col % G;
  const bf16_t* qh = q + ((size_t)b * heads_q + (size_t)kvh * G) * n_tok * D;
  // First batch's query rows (in flight while K and V are staged).
  bf16x8_t bq[NCH][KSTEPS];
  int pid[NCH], tq[NCH];
  attn_fetch<D, G, NCH, KSTEPS>(bq, pid, tq, pairs, start, len, 0, wave, col, kh, qh, bh, n_tok,
                                topk);
  const bf16_t* kb = k + ((size_t)bh * n_tok + tok0) * D;
  const bf16_t* vb = v + ((size_t)bh * n_tok + tok0) * D;
  for (int x = tid; x < C * (D / 8); x += kAttnThreads) {
    const int r = x / (D / 8), c = (x % (D / 8)) * 8;
    const int rr = min(r, n_keys - 1);  // rows past the sequence end: masked below
    const uint4 kv = *reinterpret_cast<const uint4*>(kb + (size_t)rr * D + c);
    const uint4 vv = *reinterpret_cast<const uint4*>(vb + (size_t)rr * D + c);
    *reinterpret_cast<uint4*>(&ks[r * KROW + c]) = kv;
    const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(c + 2 * e) * VROW + r] = bf16_t(w4[e] & 0xffffu);
      vt[(c + 2 * e + 1) * VROW + r] = bf16_t(w4[e] >> 16);
    }
  }
  __syncthreads();

  const int rows = len * G;
  const int n_batches = (len + PAIRS - 1) / PAIRS;
  for (int bt = 0; bt < n_batches; ++bt) {
    if (bt > 0)
      attn_fetch<D, G, NCH, KSTEPS>(bq, pid, tq, pairs, start, len, bt, wave, col, kh, qh, bh,
                                    n_tok, topk);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int r0 = bt * kAttnRows + (wave + NW * c) * kAttnCols;
      if (r0 >= rows) break;
      const bool live = r0 + col < rows;
      f32x16_t s0 = {}, s1 = {};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8_t a0 = as_bf16x8(*reinterpret_cast<const uint4*>(&ks[col * KROW + 16 * s + 8 * kh]));
        const bf16x8_t a1 =
            as_bf16x8(*reinterpret_cast<const uint4*>(&ks[(32 + col) * KROW + 16 * s + 8 * kh]));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq[c][s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bq[c][s], s1, 0, 0, 0);
      }
      // Lane holds logits of keys (i/4)*8 + 4kh + i%4 (s0) and 32 + that (s1).
      int lim = n_keys - 1;
      if (causal) lim = min(lim, tq[c] - tok0);
      if (__ballot(lim < C - 1) != 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (i / 4) * 8 + 4 * kh + (i % 4);
          s0[i] = r <= lim ? s0[i] : neg_inf();
          s1[i] = r + 32 <= lim ? s1[i] : neg_inf();
        }
      }
      float m = fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s1[0], s1[1]));
#pragma unroll
      for (int i = 2; i < 16; i += 2)
        m = fmaxf(m, fmaxf(fmaxf(s0[i], s0[i + 1]), fmaxf(s1[i], s1[i + 1])));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      const float ms = m == neg_inf() ? 0.f : m * scale_log2;  // a column without keys
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = fast_exp2(fmaf(s0[i], scale_log2, -ms));
        s1[i] = fast_exp2(fmaf(s1[i], scale_log2, -ms));
        l += s0[i] + s1[i];
      }
      l += __shfl_xor(l, 32, kWave);
      // B operands P^T: step st covers keys 32(st/2) + 16(st%2) + 8(j/4) + 4kh + j%4.
      bf16x8_t pb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[st][j] = (__bf16)(st < 2 ? s0[8 * st + j] : s1[8 * (st - 2) + j]);
      f32x16_t o[DBLK];
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        o[db] = f32x16_t{};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16_t* vrow = &vt[(32 * db + col) * VROW + 32 * (st / 2) + 16 * (st % 2) + 4 * kh];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[st], o[db], 0, 0, 0);
        }
      }
      // o[db][i] = O[column][d = 32 db + (i/4)*8 + 4kh + i%4].  Partials are
      // stored in bucket order (row start * G + r of the sorted pairs): the
      // chunk's 32 rows are one contiguous run, written through an LDS tile
      // (half of d per pass) as 16-byte pieces, 1 KB per store instruction.
      const float inv = l > 0.f ? 1.f / l : 0.f;
      bf16_t* tile = &os[wave][0];
      if (live && kh == 0) part_lse[(size_t)start * G + r0 + col] = ms + fast_log2(l);
      const int n_live = min(kAttnCols, rows - r0);  // rows of this chunk that exist
      bf16_t* dst = part_o + ((size_t)start * G + r0) * D;
      // two passes, each over half of d
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int dh = 0; dh < DBLK / 2; ++dh)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
            bf16x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[hf * (DBLK / 2) + dh][4 * g4 + e] * inv);
            *reinterpret_cast<uint2*>(&tile[col * OROW + 32 * dh + 8 * g4 + 4 * kh]) =
                __builtin_bit_cast(uint2, w);
          }
        wave_lds_sync();
        constexpr int PIECES = kAttnCols * D / 16;  // 16-byte pieces of the half chunk
#pragma unroll
        for (int x = lane; x < PIECES; x += kWave) {
          const int rr = x / (D / 16), c8 = (x % (D / 16)) * 8;
          if (rr < n_live)
            // streamed out: read once, by the combine
            __builtin_nontemporal_store(
                *reinterpret_cast<const u32x4_t*>(&tile[rr * OROW + c8]),
                reinterpret_cast<u32x4_t*>(dst + (size_t)rr * D + hf * (D / 2) + c8));
        }
        wave_lds_sync();
      }
    }
  }
}

// Merge the K partials of each (query, head) row: weights exp2(lse_j - M)
// over the selected blocks, 16 lanes per row.  Slot j of row u sits at
// position pos_of[u * K + j] of the bucket order.  The row's positions and
// LSEs, then up to 16 partials (16-byte loads), are all requested before any
// is used.  Slots that are -1 or out of range have no position (rows need
// not be sorted, so slot 0 may be one of them): they read position 0, which
// is always inside the partial buffers, with weight 0 and their loaded values
// replaced by zeros.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const int32_t* __restrict__ idx, const int* __restrict__ pos_of, const bf16_t* __restrict__ part_o,
    const float* __restrict__ part_lse, bf16_t* __restrict__ out, float* __restrict__ lse_out,
    int heads_q, int heads_kv, int n_tok, int topk, int group, int m1, size_t n_rows) {
  constexpr int EPL = D / 16;  // elements per lane (16 lanes per row)
  constexpr int B = 16;        // slots per batch
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 16;
  if (row >= n_rows) return;
  const int sub = threadIdx.x & 15;
  const size_t u = row / group;
  const int h = (int)(row % group);
  const int t = (int)(u % n_tok);
  const size_t bh = u / n_tok;
  const int b = (int)(bh / heads_kv), kvh = (int)(bh % heads_kv);
  const int32_t* ir = idx + u * topk;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float M = neg_inf(), W = 0.f;
  for (int j0 = 0; j0 < topk; j0 += B) {
    float lj[B];
    int pj[B];
#pragma unroll
    for (int jj = 0; jj < B; ++jj) {
      const int j = min(j0 + jj, topk - 1);
      const int x = ir[j];
      const bool ok = j0 + jj < topk && x >= 0 && x < m1;
      // a slot that is not live was never given a position: use position 0
      const int p = pos_of[u * topk + j];
      pj[jj] = ok ? p : 0;
      const float lv = part_lse[(size_t)pj[jj] * group + h];
      lj[jj] = ok ? lv : neg_inf();
    }
    float mb = M;
#pragma unroll
    for (int jj = 0; jj < B; ++jj) mb = fmaxf(mb, lj[jj]);
    if (mb == neg_inf()) continue;
    // rescale what earlier batches accumulated
    const float r = M == neg_inf() ? 0.f : fast_exp2(M - mb);
    W *= r;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= r;
    M = mb;
    uint32_t raw[B][EPL / 2];  // bf16 pairs, unpacked when used
#pragma unroll
    for (int jj = 0; jj < B; ++jj) {
      const bf16_t* src = part_o + ((size_t)pj[jj] * group + h) * D + sub * EPL;
      if (EPL == 8) {
        const u32x4_t v4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
        raw[jj][0] = v4.x; raw[jj][1] = v4.y; raw[jj][2] = v4.z; raw[jj][3] = v4.w;
      } else {
        const uint2 v2 = *reinterpret_cast<const uint2*>(src);
        raw[jj][0] = v2.x; raw[jj][1] = v2.y;
      }
    }
#pragma unroll
    for (int jj = 0; jj < B; ++jj) {
      const bool live = lj[jj] != neg_inf();
      const float w = live ? fast_exp2(lj[jj] - M) : 0.f;
      // a slot without a partial read position 0, which need not hold one
      // (no pair at all, or not yet written): take zeros, never 0 * garbage
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) raw[jj][e] = live ? raw[jj][e] : 0u;
      W += w;
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) {
        acc[2 * e] += w * __uint_as_float(raw[jj][e] << 16);
        acc[2 * e + 1] += w * __uint_as_float(raw[jj][e] & 0xffff0000u);
      }
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  bf16_t* dst = out + (((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t) * D + sub * EPL;
  if (EPL == 8) {
    typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8v;
    bf16x8v o8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<uint4*>(dst) = __builtin_bit_cast(uint4, o8);
  } else {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4v;
    bf16x4v o4;
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, o4);
  }
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
  int* inv = reinterpret_cast<int*>(base + lay.inv);
  bf16_t* part_o = reinterpret_cast<bf16_t*>(base + lay.part_o);
  float* part_lse = reinterpret_cast<float*>(base + lay.part_lse);
  const int m1 = s.lv.size[0];
  hipError_t e;
  {
    prof::Scope ps("attn_sort", st);
    e = bucket::sort_pairs(idx, s.batch * s.heads_kv, s.seq_len, s.topk, m1,
                           kAttnRows / s.group * kAttnBatches, counts, offsets, cursors,
                           item_offsets, pairs, inv, false, st);
  }
  if (e != hipSuccess) return e;
  {
    prof::Scope ps("attn_partial", st);
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const float sl = s.scale * kLog2e;
    const int cz = s.causal ? 1 : 0;
#define PISA_AP(G)                                                                             \
  hipLaunchKernelGGL((attn_partial_kernel<D, G>), dim3(lay.max_items), dim3(kAttnThreads), 0, st, \
                     qb, kb, vb, item_offsets, offsets, pairs, part_o, part_lse, lay.n_buckets,  \
                     s.heads_q, s.heads_kv, s.seq_len, s.topk, m1, cz, sl)
    switch (s.group) {
      case 1: PISA_AP(1); break;
      case 2: PISA_AP(2); break;
      case 4: PISA_AP(4); break;
      case 8: PISA_AP(8); break;
      default: PISA_AP(16); break;
    }
#undef PISA_AP
  }
  prof::Scope ps("attn_combine", st);
  const size_t rows = (size_t)s.batch * s.heads_kv * s.seq_len * s.group;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)((rows * 16 + 255) / 256)),
                     dim3(256), 0, st, idx, inv, part_o, part_lse, static_cast<bf16_t*>(out), lse,
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
