// Backward of the block-sparse attention with the block lists held fixed
// (PISA reading page §5.3 "backward": the selected indices do not move and
// gradients flow only through the attention entries they select; the forward
// is eq. (2) of §02 with the causal mask of §5.3).
//
// With the forward's row LSE (natural log) and output O, for every query head
// and row i and every token j of the row's blocks:
//   P_ij  = exp(scale q_i.k_j - lse_i)
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i.v_j - D_i),      D_i = dO_i.O_i
//   dQ_i  = scale sum_j dS_ij k_j,       dK_j = scale sum_i dS_ij q_i
// where the sums over i run over every query head of the KV group.
//
// bf16, C = 64, a power-of-two group (any other shape: the general kernel
// below replaces step 3 with fp32 vector math, same items and reductions):
//  1. delta:   D_i per (query head, row), fp32;
//  2. the (row, slot) pairs are bucketed by leaf block with the stable
//     counting sort of bucket.h (each block's pairs in row order), in work
//     items of at most 2048 (pair, head) columns;
//  3. one workgroup per work item keeps its block's K and V as MFMA operands
//     in registers and walks the item's columns 32 at a time.  Wave w owns the
//     block's keys 16w..16w+15:
//       S, dP  [32 columns x 16 keys]  MFMA 16x16x32 (A = Q / dO rows from LDS,
//                                      B = K / V rows from registers)
//       P, dS  in the accumulators (masked entries are 0)
//       dV^T += dO^T P,  dK^T += Q^T dS  (the contraction runs over the chunk's
//                                         columns; Q^T and dO^T come from LDS)
//       dQ^T  = K^T dS^T for the wave's quarter of d (dS passes through LDS;
//               computed one chunk later, so each chunk needs two barriers)
//     Each column's dQ over this block goes (bf16) through an LDS tile and
//     leaves as whole rows, in bucket order.  At the end the block's dK, dV
//     go straight to the outputs when its bucket is one work item, else to a
//     per-item fp32 partial;
//  4. dq combine: the row's K partials summed in slot order, times scale;
//  5. dkv reduce: blocks of several work items sum their partials in item
//     order; blocks that no row selected get zeros.
// No floating-point atomics: the results are bitwise reproducible.
#include <algorithm>

#include "bucket.h"
#include "pisa_common.h"
#include "pisa_launch.h"

namespace pisa {
namespace {

constexpr int kBwdBlock = 64;     // C
constexpr int kBwdThreads = 256;  // 4 waves, one per 16 keys of the block
constexpr int kBwdCols = 32;      // (pair, head) columns per chunk
constexpr int kBwdItemCols = 2048;  // (pair, head) columns per work item
constexpr int kGenItemCols = 256;   // columns per work item of the general kernel

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
// Word i (0..3, may differ per lane) of v.
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  const uint32_t a = (i & 1) ? v.y : v.x;
  const uint32_t b = (i & 1) ? v.w : v.z;
  return (i & 2) ? b : a;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// bf16, C = 64, a power-of-two group: the MFMA kernel; every other shape
// the general one.
bool mfma_path(const LaunchShape& s) {
  return s.bf16 && s.block == kBwdBlock && (s.group & (s.group - 1)) == 0;
}

struct BwdWs {
  size_t counts, offsets, cursors, item_offsets, wgc, pairs, inv, delta, part_dq, part_kv, total;
  int n_buckets, max_items, per_item;
};

BwdWs bwd_layout(const LaunchShape& s) {
  BwdWs w;
  const bool mf = mfma_path(s);
  const size_t slots = (size_t)s.batch * s.heads_kv * s.seq_len * s.topk;
  w.n_buckets = s.batch * s.heads_kv * s.lv.size[0];
  w.per_item = (mf ? kBwdItemCols : kGenItemCols) / s.group;
  w.max_items = bucket::max_items(slots, w.n_buckets, w.per_item);
  size_t off = 0;
  w.counts = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.cursors = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.item_offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.wgc = off;
  off = align256(off + sizeof(int) * bucket::stable_wgc_ints(s.batch * s.heads_kv, s.seq_len, s.lv.size[0]));
  w.pairs = off; off = align256(off + sizeof(int) * slots);
  w.inv = off; off = align256(off + sizeof(int) * slots);
  w.delta = off; off = align256(off + sizeof(float) * s.batch * s.heads_q * s.seq_len);
  w.part_dq = off;
  off = align256(off + (mf ? sizeof(bf16_t) : sizeof(float)) * slots * s.group * s.head_dim);
  w.part_kv = off; off = align256(off + sizeof(float) * w.max_items * 2 * s.block * s.head_dim);
  w.total = off;
  return w;
}

// D_i = dO_i . O_i (fp32) for every (batch, query head, row); 16 lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const T* __restrict__ out,
                                                             const T* __restrict__ dout,
                                                             float* __restrict__ delta,
                                                             size_t n_rows) {
  constexpr int EPL = D / 16;  // elements per lane
  constexpr int VEC = Vec16<T>::n;
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 16;
  if (row >= n_rows) return;
  const int sub = threadIdx.x & 15;
  float o[EPL], g[EPL];
  if (EPL % VEC == 0) {
#pragma unroll
    for (int c = 0; c < EPL; c += VEC) {
      load16(out + row * D + sub * EPL + c, o + c);
      load16(dout + row * D + sub * EPL + c, g + c);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      o[e] = to_f32(out[row * D + sub * EPL + e]);
      g[e] = to_f32(dout[row * D + sub * EPL + e]);
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc = fmaf(o[e], g[e], acc);
#pragma unroll
  for (int o2 = 8; o2 >= 1; o2 >>= 1) acc += __shfl_xor(acc, o2, 16);
  if (sub == 0) delta[row] = acc;
}

// One chunk's staging: R = D / 32 columns x 8 dims per (thread, tensor);
// threads 0..127 carry Q, threads 128..255 carry dO.  Column r of the item is
// pair r / G, query head r % G; columns past the item's end repeat its last
// column (their results are masked).
template <int D, int G>
struct ChunkRegs {
  static constexpr int R = D / 32;
  uint4 x[R];
  // per-column metadata, threads 0..31 (column = tid)
  float lse2, dl;
  int lim;
};

template <int D, int G>
__device__ __forceinline__ void chunk_fetch(ChunkRegs<D, G>& cr, int chunk, const int* tok_s,
                                            int rows, const bf16_t* __restrict__ qh,
                                            const bf16_t* __restrict__ doh,
                                            const float* __restrict__ lse_h,
                                            const float* __restrict__ delta_h, int n_tok,
                                            int tok0, int n_keys, bool causal) {
  constexpr int R = D / 32;
  constexpr int PIECES = D / 8;  // 16-byte pieces per row
  const int tid = threadIdx.x;
  const int tt = tid & 127;
  const int c8 = (tt % PIECES) * 8;
  const int cg = tt / PIECES;  // columns R*cg .. R*cg + R - 1
  const bf16_t* src = tid < 128 ? qh : doh;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = min(chunk * kBwdCols + R * cg + i, rows - 1);
    const int t = tok_s[r / G];
    const int h = r % G;
    cr.x[i] = *reinterpret_cast<const uint4*>(src + ((size_t)h * n_tok + t) * D + c8);
  }
  if (tid < kBwdCols) {
    const int r0 = chunk * kBwdCols + tid;
    const int r = min(r0, rows - 1);
    const int t = tok_s[r / G];
    const int h = r % G;
    cr.lse2 = lse_h[(size_t)h * n_tok + t] * kLog2e;
    cr.dl = delta_h[(size_t)h * n_tok + t];
    int lim = n_keys - 1;
    if (causal) lim = min(lim, t - tok0);
    cr.lim = r0 < rows ? lim : -1;
  }
}

template <int D>
struct BwdLds {
  static constexpr int KROW = D + 8;          // [column][d] rows (bf16)
  static constexpr int TROW = kBwdBlock + 8;  // K^T [d][key]
  static constexpr int CT = kBwdCols + 4;     // Q^T, dO^T [d][column]
  static constexpr int SROW = kBwdBlock + 8;  // dS [column][key]
  bf16_t qs[kBwdCols * KROW];
  bf16_t os[kBwdCols * KROW];
  bf16_t qt[D * CT];
  bf16_t ot[D * CT];
  float lse2[kBwdCols];
  float dl[kBwdCols];
  int lim[kBwdCols];
  int tok[kBwdItemCols];  // query position of each pair of the work item
  // K^T is read into registers once, before the first chunk; its space then
  // holds two chunks' dS and dQ rows (chunk c is written while chunk c - 1's
  // are still being read).
  union {
    bf16_t kt[D * TROW];
    struct {
      bf16_t ds[2][kBwdCols * SROW];
      bf16_t dqt[2][kBwdCols * KROW];  // a chunk's dQ rows, stored out whole
    } c;
  } u;
};

template <int D, int G>
__device__ __forceinline__ void chunk_stage(const ChunkRegs<D, G>& cr, BwdLds<D>& L) {
  constexpr int R = D / 32;
  constexpr int PIECES = D / 8;
  constexpr int KROW = BwdLds<D>::KROW, CT = BwdLds<D>::CT;
  const int tid = threadIdx.x;
  const int tt = tid & 127;
  const int c8 = (tt % PIECES) * 8;
  const int cg = tt / PIECES;
  bf16_t* rows = tid < 128 ? L.qs : L.os;
  bf16_t* tr = tid < 128 ? L.qt : L.ot;
#pragma unroll
  for (int i = 0; i < R; ++i)
    *reinterpret_cast<uint4*>(&rows[(R * cg + i) * KROW + c8]) = cr.x[i];
  // transposed: dims c8..c8+7, columns R*cg..R*cg+R-1 (R consecutive bf16).
  // Lane p writes dim c8 + (e + p) % 8 at step e: without the rotation the
  // lanes of one store would sit 8 rows apart, on the same few banks.
  const int p = tt % PIECES;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ee = (e + p) & 7;
    uint32_t h[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t w = word(cr.x[i], ee >> 1);
      h[i] = (ee & 1) ? (w >> 16) : (w & 0xffffu);
    }
    bf16_t* dst = &tr[(c8 + ee) * CT + R * cg];
    if (R == 4)
      *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    else
      *reinterpret_cast<uint32_t*>(dst) = h[0] | (h[1] << 16);
  }
  if (tid < kBwdCols) {
    L.lse2[tid] = cr.lse2;
    L.dl[tid] = cr.dl;
    L.lim[tid] = cr.lim;
  }
}

// One workgroup per work item (block blk of KV head bh, up to kBwdItemCols /
// G pairs).  MFMA 16x16x32 bf16 operand layout: A[i][k] at lane i + 16 (k/8),
// element k % 8; B[k][j] at lane j + 16 (k/8), element k % 8; the fp32 result
// D[i][j] at lane j + 16 (i/4), element i % 4.
template <int D, int G>
__global__ __launch_bounds__(kBwdThreads, 2) void attn_bwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ item_offsets,
    const int* __restrict__ offsets, const int* __restrict__ pairs, bf16_t* __restrict__ part_dq,
    float* __restrict__ part_kv, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int n_buckets,
    int heads_q, int heads_kv, int n_tok, int m1, int causal, float scale, float scale_log2) {
  constexpr int C = kBwdBlock;
  constexpr int DS = D / 32;   // 32-deep k-steps over d
  constexpr int MT = D / 16;   // 16-row tiles over d
  constexpr int QMT = D / 64;  // dQ tiles over d per wave
  constexpr int TROW = BwdLds<D>::TROW, KROW = BwdLds<D>::KROW, CT = BwdLds<D>::CT,
                SROW = BwdLds<D>::SROW;
  __shared__ __attribute__((aligned(16))) BwdLds<D> L;

  int bucket, start, len;
  if (!bucket::locate_item(item_offsets, offsets, n_buckets, blockIdx.x, kBwdItemCols / G,
                           &bucket, &start, &len))
    return;
  const int bh = bucket / m1, blk = bucket % m1;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tok0 = blk * C;
  const int n_keys = min(C, n_tok - tok0);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int li = lane & 15, g = lane >> 4;
  const int rows = len * G;
  const int n_chunks = (rows + kBwdCols - 1) / kBwdCols;
  const size_t head0 = (size_t)b * heads_q + (size_t)kvh * G;
  const bf16_t* qh = q + head0 * n_tok * D;
  const bf16_t* doh = dout + head0 * n_tok * D;
  const float* lse_h = lse + head0 * n_tok;
  const float* delta_h = delta + head0 * n_tok;
  for (int i = tid; i < len; i += kBwdThreads)
    L.tok[i] = (pairs[start + i] >> 5) - bh * n_tok;  // pair = (row << 5) | slot
  __syncthreads();

  // Two chunks in flight: chunk c + 2 is requested while chunk c computes.
  ChunkRegs<D, G> cra, crb;
  chunk_fetch<D, G>(cra, 0, L.tok, rows, qh, doh, lse_h, delta_h, n_tok, tok0, n_keys, causal != 0);
  if (n_chunks > 1)
    chunk_fetch<D, G>(crb, 1, L.tok, rows, qh, doh, lse_h, delta_h, n_tok, tok0, n_keys,
                      causal != 0);

  // This wave's keys as B operands (K rows for S, V rows for dP), rows past
  // the sequence end repeat the last key (masked below).
  const bf16_t* kb = k + ((size_t)bh * n_tok + tok0) * D;
  const bf16_t* vb = v + ((size_t)bh * n_tok + tok0) * D;
  const int my_key = 16 * w + li;
  bf16x8_t kop[DS], vop[DS];
  {
    const int kr = min(my_key, n_keys - 1);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kop[s] = as_bf16x8(*reinterpret_cast<const uint4*>(kb + (size_t)kr * D + 32 * s + 8 * g));
      vop[s] = as_bf16x8(*reinterpret_cast<const uint4*>(vb + (size_t)kr * D + 32 * s + 8 * g));
    }
  }
  // K^T through LDS once per item.
  for (int x = tid; x < C * (D / 8); x += kBwdThreads) {
    const int r = x / (D / 8), c = (x % (D / 8)) * 8;
    const uint4 kv = *reinterpret_cast<const uint4*>(kb + (size_t)min(r, n_keys - 1) * D + c);
    const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      L.u.kt[(c + 2 * e) * TROW + r] = bf16_t(w4[e] & 0xffffu);
      L.u.kt[(c + 2 * e + 1) * TROW + r] = bf16_t(w4[e] >> 16);
    }
  }
  __syncthreads();
  // dQ's A operands: K^T rows of this wave's d tiles, both 32-key steps.
  bf16x8_t ktop[QMT][2];
#pragma unroll
  for (int m = 0; m < QMT; ++m)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      ktop[m][ks] = as_bf16x8(
          *reinterpret_cast<const uint4*>(&L.u.kt[(16 * (QMT * w + m) + li) * TROW + 32 * ks + 8 * g]));

  f32x4_t dk_acc[MT], dv_acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    dk_acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dv_acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // dQ^T of chunk cp for d tiles QMT*w.., all 32 columns; lane (column
  // 16ct + li, g) receives dQ[column][16 (QMT w + m) + 4g + e], which goes to
  // the chunk's dQ tile.
  auto dq_phase = [&](int cp) {
    const bf16_t* dsb = L.u.c.ds[cp & 1];
    bf16_t* dqt = L.u.c.dqt[cp & 1];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int col = 16 * ct + li;
      bf16x8_t bs[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        bs[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&dsb[col * SROW + 32 * ks + 8 * g]));
#pragma unroll
      for (int m = 0; m < QMT; ++m) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ktop[m][0], bs[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ktop[m][1], bs[1], acc, 0, 0, 0);
        bf16x4_t o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)acc[e];
        *reinterpret_cast<uint2*>(&dqt[col * KROW + 16 * (QMT * w + m) + 4 * g]) =
            __builtin_bit_cast(uint2, o4);
      }
    }
  };
  // Whole dQ rows of chunk cp leave as 16-byte pieces (1 KB per store
  // instruction); each is read once, by the dq combine.
  auto store_phase = [&](int cp) {
    const bf16_t* dqt = L.u.c.dqt[cp & 1];
#pragma unroll
    for (int j = 0; j < kBwdCols * (D / 8) / kBwdThreads; ++j) {
      const int x = tid + kBwdThreads * j;
      const int row = x / (D / 8), c8 = (x % (D / 8)) * 8;
      const int r = cp * kBwdCols + row;
      if (r < rows)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4_t*>(&dqt[row * KROW + c8]),
            reinterpret_cast<u32x4_t*>(part_dq + ((size_t)start * G + r) * D + c8));
    }
  };
  // Per chunk two barriers: after the staging (A) and after this chunk's
  // reads of the staged rows (X).  Chunk c's dQ is computed after barrier A
  // of chunk c + 1 (its dS is complete by then) and stored after barrier X.
  auto chunk = [&](int ch, ChunkRegs<D, G>& cr) {
    chunk_stage<D, G>(cr, L);
    __syncthreads();
    if (ch + 2 < n_chunks)
      chunk_fetch<D, G>(cr, ch + 2, L.tok, rows, qh, doh, lse_h, delta_h, n_tok, tok0, n_keys,
                        causal != 0);
    if (ch > 0) dq_phase(ch - 1);
    // S and dP for columns 16ct + 4g + e, key my_key.
    f32x4_t sacc[2], pacc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      sacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8_t aq =
            as_bf16x8(*reinterpret_cast<const uint4*>(&L.qs[(16 * ct + li) * KROW + 32 * s + 8 * g]));
        const bf16x8_t ao =
            as_bf16x8(*reinterpret_cast<const uint4*>(&L.os[(16 * ct + li) * KROW + 32 * s + 8 * g]));
        sacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kop[s], sacc[ct], 0, 0, 0);
        pacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, vop[s], pacc[ct], 0, 0, 0);
      }
    }
    // P and dS; the B operands of dV^T / dK^T hold columns {4g..4g+3,
    // 16+4g..16+4g+3} in k-slots 8g..8g+7 (the same permutation is used for
    // the A operands read from Q^T / dO^T).
    bf16x8_t pb, sb;
    bf16_t* dsb = L.u.c.ds[ch & 1];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 16 * ct + 4 * g + e;
        const bool ok = my_key <= L.lim[col];
        const float p = ok ? fast_exp2(fmaf(sacc[ct][e], scale_log2, -L.lse2[col])) : 0.f;
        const float dsv = p * (pacc[ct][e] - L.dl[col]);
        pb[4 * ct + e] = (__bf16)p;
        sb[4 * ct + e] = (__bf16)dsv;
        dsb[col * SROW + my_key] = __builtin_bit_cast(bf16_t, (__bf16)dsv);
      }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bf16_t* orow = &L.ot[(16 * m + li) * CT];
      const bf16_t* qrow = &L.qt[(16 * m + li) * CT];
      const uint2 o0 = *reinterpret_cast<const uint2*>(orow + 4 * g);
      const uint2 o1 = *reinterpret_cast<const uint2*>(orow + 16 + 4 * g);
      const uint2 q0 = *reinterpret_cast<const uint2*>(qrow + 4 * g);
      const uint2 q1 = *reinterpret_cast<const uint2*>(qrow + 16 + 4 * g);
      dv_acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(make_uint4(o0.x, o0.y, o1.x, o1.y)), pb, dv_acc[m], 0, 0, 0);
      dk_acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(make_uint4(q0.x, q0.y, q1.x, q1.y)), sb, dk_acc[m], 0, 0, 0);
    }
    __syncthreads();
    if (ch > 0) store_phase(ch - 1);
  };
  for (int ch = 0; ch < n_chunks; ch += 2) {
    chunk(ch, cra);
    if (ch + 1 < n_chunks) chunk(ch + 1, crb);
  }
  dq_phase(n_chunks - 1);
  __syncthreads();
  store_phase(n_chunks - 1);

  // dK (times scale) and dV of keys my_key: lane holds d = 16m + 4g + e.
  const int n_items = item_offsets[bucket + 1] - item_offsets[bucket];
  if (n_items == 1) {
    if (my_key < n_keys) {
      bf16_t* kd = dk + ((size_t)bh * n_tok + tok0 + my_key) * D;
      bf16_t* vd = dv + ((size_t)bh * n_tok + tok0 + my_key) * D;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        bf16x4_t a4, b4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a4[e] = (__bf16)(dk_acc[m][e] * scale);
          b4[e] = (__bf16)dv_acc[m][e];
        }
        *reinterpret_cast<uint2*>(kd + 16 * m + 4 * g) = __builtin_bit_cast(uint2, a4);
        *reinterpret_cast<uint2*>(vd + 16 * m + 4 * g) = __builtin_bit_cast(uint2, b4);
      }
    }
  } else {
    float* pk = part_kv + ((size_t)blockIdx.x * 2) * C * D + (size_t)my_key * D;
    float* pv = pk + (size_t)C * D;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      f32x4_t a4 = dk_acc[m] * scale;
      *reinterpret_cast<f32x4_t*>(pk + 16 * m + 4 * g) = a4;
      *reinterpret_cast<f32x4_t*>(pv + 16 * m + 4 * g) = dv_acc[m];
    }
  }
}

// dq of each (query head, row): scale times the sum of its slots' partials in
// slot order (16 lanes per row, loads of up to 16 slots in flight).  Slots
// without a position (index < 0 or past the last block) add nothing.
// Partials P are bf16 (MFMA kernel) or fp32 (general kernel).
template <typename P, typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const int32_t* __restrict__ idx, const int* __restrict__ pos_of,
    const P* __restrict__ part_dq, T* __restrict__ dq, int heads_q, int heads_kv, int n_tok,
    int topk, int group, int m1, float scale, size_t n_rows) {
  constexpr int EPL = D / 16;
  constexpr int B = 16;
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 16;
  if (row >= n_rows) return;
  const int sub = threadIdx.x & 15;
  const size_t u = row / group;
  const int h = (int)(row % group);
  const int t = (int)(u % n_tok);
  const size_t bh = u / n_tok;
  const int b = (int)(bh / heads_kv), kvh = (int)(bh % heads_kv);
  const int32_t* ir = idx + u * topk;
  constexpr bool kBf = sizeof(P) == 2;
  constexpr int WPL = kBf ? EPL / 2 : EPL;  // 32-bit words per lane and slot
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < topk; j0 += B) {
    uint32_t raw[B][WPL];  // unpacked when used
    bool live[B];
#pragma unroll
    for (int jj = 0; jj < B; ++jj) {
      const int j = min(j0 + jj, topk - 1);
      const int xj = ir[j];
      live[jj] = j0 + jj < topk && xj >= 0 && xj < m1;
      // requested with the block index, not after it (a dead slot's entry is
      // never written and never used): position 0 always exists
      const int pj = pos_of[u * topk + j];
      const int p = live[jj] ? pj : 0;
      const uint32_t* src =
          reinterpret_cast<const uint32_t*>(part_dq + ((size_t)p * group + h) * D + sub * EPL);
      if (WPL % 4 == 0) {
#pragma unroll
        for (int c = 0; c < WPL; c += 4) {
          const u32x4_t v4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + c));
          raw[jj][c] = v4.x; raw[jj][c + 1] = v4.y; raw[jj][c + 2] = v4.z; raw[jj][c + 3] = v4.w;
        }
      } else {
        const uint2 v2 = *reinterpret_cast<const uint2*>(src);
        raw[jj][0] = v2.x; raw[jj][1] = v2.y;
      }
    }
#pragma unroll
    for (int jj = 0; jj < B; ++jj) {
      if (!live[jj]) continue;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        if (kBf) {
          acc[2 * w] += __uint_as_float(raw[jj][w] << 16);
          acc[2 * w + 1] += __uint_as_float(raw[jj][w] & 0xffff0000u);
        } else {
          acc[w] += __uint_as_float(raw[jj][w]);
        }
      }
    }
  }
  T* dst = dq + (((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t) * D + sub * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) store_from_f32(dst + e, acc[e] * scale);
}

// The blocks whose dK and dV the reduction below writes: those whose bucket
// is split over several work items, and those with no pair (zeros), in
// increasing order.  One workgroup; the list length goes to *n_list.
__global__ __launch_bounds__(1024) void attn_bwd_dkv_plan_kernel(
    const int* __restrict__ item_offsets, int* __restrict__ list, int* __restrict__ n_list,
    int n_buckets) {
  constexpr int NW = 1024 / kWave;
  __shared__ int wave_n[NW];
  __shared__ int base_s;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (threadIdx.x == 0) base_s = 0;
  __syncthreads();
  for (int b0 = 0; b0 < n_buckets; b0 += 1024) {
    const int b = b0 + (int)threadIdx.x;
    const bool f = b < n_buckets && item_offsets[b + 1] - item_offsets[b] != 1;
    const uint64_t m = __ballot(f);
    if (lane == 0) wave_n[wave] = __popcll(m);
    __syncthreads();
    int before = base_s;
    for (int x = 0; x < wave; ++x) before += wave_n[x];
    if (f) list[before + lanes_below(m)] = b;
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int x = 0; x < NW; ++x) tot += wave_n[x];
      base_s += tot;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_list = base_s;
}

// dK, dV rows of the listed blocks: the sum of their items' partials in item
// order (no item: zeros).  A block's C * D / 4 * 2 (key, 4 dims, K or V)
// units form slices of 256, one thread per unit; the grid walks the list's
// slices, so a block split over many items still spreads over many
// workgroups while blocks of one item launch nothing.  C keys per block (CF >
// 0 fixes C at compile time).
template <typename T, int D, int CF>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(
    const int* __restrict__ item_offsets, const int* __restrict__ list,
    const int* __restrict__ n_list, const float* __restrict__ part_kv, T* __restrict__ dk,
    T* __restrict__ dv, int n_tok, int m1, int c_rt) {
  constexpr int Q4 = D / 4;
  const int C = CF > 0 ? CF : c_rt;
  const int slices = C * Q4 * 2 / 256;  // C >= 16 and D >= 64: a whole number
  const int n = *n_list * slices;
  for (int sl = blockIdx.x; sl < n; sl += gridDim.x) {
    const int bucket = list[sl / slices];
    const int id = (sl % slices) * 256 + (int)threadIdx.x;
    const int d4 = id % Q4;
    const int key = (id / Q4) % C;
    const int which = id / Q4 / C;
    const int bh = bucket / m1, blk = bucket % m1;
    const int tok = blk * C + key;
    if (tok >= n_tok) continue;
    const int i0 = item_offsets[bucket], n_items = item_offsets[bucket + 1] - i0;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float* src = part_kv + ((size_t)i0 * 2 + which) * C * D + (size_t)key * D + 4 * d4;
    constexpr int U = 8;
    for (int i = 0; i < n_items; i += U) {
      f32x4_t x[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        x[u] = *reinterpret_cast<const f32x4_t*>(src + (size_t)min(i + u, n_items - 1) * 2 * C * D);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i + u < n_items) acc += x[u];
    }
    T* dst = (which ? dv : dk) + ((size_t)bh * n_tok + tok) * D + 4 * d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_from_f32(dst + e, acc[e]);
  }
}

// General backward kernel (any dtype, C <= 64, any group), fp32 vector math,
// the same work items as the MFMA kernel.  One workgroup per item keeps the
// block's K and V in LDS as fp32 and walks the item's (pair, head) columns one
// at a time:
//   s_j, g_j = q . k_j, dO . v_j   4 threads per key, lanes over d
//   P_j, dS_j                      one thread per key (masked entries 0)
//   dK, dV += dS_j q, P_j dO       each thread owns C*D/256 (key, dim)
//                                  entries of the block in registers
//   dQ column = sum_j dS_j k_j     (fp32 partial, bucket order)
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int* __restrict__ item_offsets, const int* __restrict__ offsets,
    const int* __restrict__ pairs, float* __restrict__ part_dq, float* __restrict__ part_kv,
    T* __restrict__ dk, T* __restrict__ dv, int n_buckets, int heads_q, int heads_kv, int n_tok,
    int C, int m1, int G, int causal, float scale, float scale_log2) {
  constexpr int KP = D + 1;      // padded fp32 rows
  constexpr int NG = 256 / D;    // key groups of the dQ sums
  constexpr int RMAX = 64 * D / 256;  // (key, dim) entries per thread at C = 64
  __shared__ float ks[64 * KP], vs[64 * KP];
  __shared__ float qv[D], gv[D];
  __shared__ float sp[64], sd[64];
  __shared__ float red[NG][D];
  __shared__ int tok_s[kGenItemCols];
  int bucket, start, len;
  if (!bucket::locate_item(item_offsets, offsets, n_buckets, blockIdx.x, kGenItemCols / G,
                           &bucket, &start, &len))
    return;
  const int bh = bucket / m1, blk = bucket % m1;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tok0 = blk * C;
  const int n_keys = min(C, n_tok - tok0);
  const int tid = threadIdx.x;
  const int rows = len * G;
  const size_t head0 = (size_t)b * heads_q + (size_t)kvh * G;
  const T* kb = k + ((size_t)bh * n_tok + tok0) * D;
  const T* vb = v + ((size_t)bh * n_tok + tok0) * D;
  for (int i = tid; i < len; i += 256) tok_s[i] = (pairs[start + i] >> 5) - bh * n_tok;
  for (int x = tid; x < C * D; x += 256) {
    const int j = x / D, d = x % D;
    const size_t src = (size_t)min(j, n_keys - 1) * D + d;
    ks[j * KP + d] = to_f32(kb[src]);
    vs[j * KP + d] = to_f32(vb[src]);
  }
  float ak[RMAX], av[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) ak[r] = av[r] = 0.f;
  const int kj = tid / 4, part = tid % 4;
  const int dd = tid % D, grp = tid / D;
  __syncthreads();
  for (int r = 0; r < rows; ++r) {
    const int h = r % G;
    const int t = tok_s[r / G];
    const size_t qrow = ((head0 + h) * n_tok + t) * D;
    for (int d = tid; d < D; d += 256) {
      qv[d] = to_f32(q[qrow + d]);
      gv[d] = to_f32(dout[qrow + d]);
    }
    __syncthreads();
    float sv = 0.f, gd = 0.f;
    if (kj < C) {
#pragma unroll 8
      for (int i = 0; i < D / 4; ++i) {
        const int d = part + 4 * i;
        sv = fmaf(qv[d], ks[kj * KP + d], sv);
        gd = fmaf(gv[d], vs[kj * KP + d], gd);
      }
    }
    sv += __shfl_xor(sv, 1, kWave);
    sv += __shfl_xor(sv, 2, kWave);
    gd += __shfl_xor(gd, 1, kWave);
    gd += __shfl_xor(gd, 2, kWave);
    if (part == 0 && kj < C) {
      int lim = n_keys - 1;
      if (causal) lim = min(lim, t - tok0);
      const float* lse_h = lse + (head0 + h) * n_tok;
      const float p = kj <= lim ? fast_exp2(fmaf(sv, scale_log2, -lse_h[t] * kLog2e)) : 0.f;
      sp[kj] = p;
      sd[kj] = p * (gd - delta[(head0 + h) * n_tok + t]);
    }
    __syncthreads();
#pragma unroll
    for (int r2 = 0; r2 < RMAX; ++r2) {
      const int e = tid + 256 * r2;
      if (e < C * D) {
        const int j = e / D, d = e % D;
        ak[r2] = fmaf(sd[j], qv[d], ak[r2]);
        av[r2] = fmaf(sp[j], gv[d], av[r2]);
      }
    }
    float acc = 0.f;
    for (int j = grp; j < C; j += NG) acc = fmaf(sd[j], ks[j * KP + dd], acc);
    red[grp][dd] = acc;
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) sum += red[g2][tid];
      part_dq[((size_t)start * G + r) * D + tid] = sum;
    }
    __syncthreads();
  }
  const int n_items = item_offsets[bucket + 1] - item_offsets[bucket];
#pragma unroll
  for (int r2 = 0; r2 < RMAX; ++r2) {
    const int e = tid + 256 * r2;
    if (e >= C * D) continue;
    const int j = e / D, d = e % D;
    if (n_items == 1) {
      if (j < n_keys) {
        store_from_f32(dk + ((size_t)bh * n_tok + tok0 + j) * D + d, ak[r2] * scale);
        store_from_f32(dv + ((size_t)bh * n_tok + tok0 + j) * D + d, av[r2]);
      }
    } else {
      float* pk = part_kv + ((size_t)blockIdx.x * 2) * C * D;
      pk[e] = ak[r2] * scale;
      pk[(size_t)C * D + e] = av[r2];
    }
  }
}

template <typename T, int D>
hipError_t launch_bwd(const LaunchShape& s, const void* q, const void* k, const void* v,
                      const int32_t* idx, const void* out, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
  const BwdWs lay = bwd_layout(s);
  const bool mf = mfma_path(s);
  char* base = static_cast<char*>(ws);
  int* counts = reinterpret_cast<int*>(base + lay.counts);
  int* offsets = reinterpret_cast<int*>(base + lay.offsets);
  int* cursors = reinterpret_cast<int*>(base + lay.cursors);
  int* item_offsets = reinterpret_cast<int*>(base + lay.item_offsets);
  int* wgc = reinterpret_cast<int*>(base + lay.wgc);
  int* pairs = reinterpret_cast<int*>(base + lay.pairs);
  int* inv = reinterpret_cast<int*>(base + lay.inv);
  float* delta = reinterpret_cast<float*>(base + lay.delta);
  void* part_dq = base + lay.part_dq;
  float* part_kv = reinterpret_cast<float*>(base + lay.part_kv);
  const int m1 = s.lv.size[0];
  const size_t q_rows = (size_t)s.batch * s.heads_q * s.seq_len;
  const T* qt = static_cast<const T*>(q);
  const T* kt = static_cast<const T*>(k);
  const T* vt = static_cast<const T*>(v);
  const T* gt = static_cast<const T*>(dout);
  T* dkt = static_cast<T*>(dk);
  T* dvt = static_cast<T*>(dv);
  {
    prof::Scope ps("attn_bwd_delta", st);
    hipLaunchKernelGGL((attn_bwd_delta_kernel<T, D>), dim3((unsigned)((q_rows * 16 + 255) / 256)),
                       dim3(256), 0, st, static_cast<const T*>(out), gt, delta, q_rows);
  }
  hipError_t e;
  {
    prof::Scope ps("attn_bwd_sort", st);
    e = bucket::sort_pairs_stable(idx, s.batch * s.heads_kv, s.seq_len, s.topk, m1, lay.per_item,
                                  counts, offsets, cursors, item_offsets, wgc, pairs, inv, st);
  }
  if (e != hipSuccess) return e;
  const int cz = s.causal ? 1 : 0;
  const float sl = s.scale * kLog2e;
  if (mf) {
    prof::Scope ps("attn_bwd_main", st);
    const bf16_t* qb = reinterpret_cast<const bf16_t*>(qt);
    const bf16_t* kb = reinterpret_cast<const bf16_t*>(kt);
    const bf16_t* vb = reinterpret_cast<const bf16_t*>(vt);
    const bf16_t* gb = reinterpret_cast<const bf16_t*>(gt);
    bf16_t* dkb = reinterpret_cast<bf16_t*>(dkt);
    bf16_t* dvb = reinterpret_cast<bf16_t*>(dvt);
    bf16_t* pq = static_cast<bf16_t*>(part_dq);
#define PISA_BWD(G)                                                                            \
  hipLaunchKernelGGL((attn_bwd_kernel<D, G>), dim3(lay.max_items), dim3(kBwdThreads), 0, st, qb, \
                     kb, vb, gb, lse, delta, item_offsets, offsets, pairs, pq, part_kv, dkb, dvb, \
                     lay.n_buckets, s.heads_q, s.heads_kv, s.seq_len, m1, cz, s.scale, sl)
    switch (s.group) {
      case 1: PISA_BWD(1); break;
      case 2: PISA_BWD(2); break;
      case 4: PISA_BWD(4); break;
      case 8: PISA_BWD(8); break;
      default: PISA_BWD(16); break;
    }
#undef PISA_BWD
  } else {
    prof::Scope ps("attn_bwd_general", st);
    hipLaunchKernelGGL((attn_bwd_generic_kernel<T, D>), dim3(lay.max_items), dim3(256), 0, st, qt,
                       kt, vt, gt, lse, delta, item_offsets, offsets, pairs,
                       static_cast<float*>(part_dq), part_kv, dkt, dvt, lay.n_buckets, s.heads_q,
                       s.heads_kv, s.seq_len, s.block, m1, s.group, cz, s.scale, sl);
  }
  {
    prof::Scope ps("attn_bwd_dkv", st);
    // counts and cursors are free once the sort is done: the list of blocks
    // to reduce goes to cursors, its length to counts[0]
    hipLaunchKernelGGL(attn_bwd_dkv_plan_kernel, dim3(1), dim3(1024), 0, st, item_offsets,
                       cursors, counts, lay.n_buckets);
    const size_t slices = (size_t)lay.n_buckets * s.block * (D / 4) * 2 / 256;
    const dim3 grid((unsigned)std::min<size_t>(slices, 8192));
    if (s.block == kBwdBlock)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, D, kBwdBlock>), grid, dim3(256), 0, st,
                         item_offsets, cursors, counts, part_kv, dkt, dvt, s.seq_len, m1,
                         s.block);
    else
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, D, 0>), grid, dim3(256), 0, st, item_offsets,
                         cursors, counts, part_kv, dkt, dvt, s.seq_len, m1, s.block);
  }
  prof::Scope ps("attn_bwd_dq", st);
  const size_t rows = (size_t)s.batch * s.heads_kv * s.seq_len * s.group;
  const dim3 grid((unsigned)((rows * 16 + 255) / 256));
  if (mf)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<bf16_t, T, D>), grid, dim3(256), 0, st, idx, inv,
                       static_cast<const bf16_t*>(part_dq), static_cast<T*>(dq), s.heads_q,
                       s.heads_kv, s.seq_len, s.topk, s.group, m1, s.scale, rows);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<float, T, D>), grid, dim3(256), 0, st, idx, inv,
                       static_cast<const float*>(part_dq), static_cast<T*>(dq), s.heads_q,
                       s.heads_kv, s.seq_len, s.topk, s.group, m1, s.scale, rows);
  return hipGetLastError();
}

}  // namespace

bool attn_bwd_supported(const LaunchShape& s) {
  const int64_t rows = (int64_t)s.batch * s.heads_kv * s.seq_len;
  return (s.head_dim == 64 || s.head_dim == 128) && s.block <= kBwdBlock &&
         s.group <= kMaxGroup && rows < (int64_t(1) << 26) &&
         s.lv.size[0] <= bucket::kMaxLocalBuckets;
}

size_t attn_bwd_ws_bytes(const LaunchShape& s) {
  return attn_bwd_supported(s) ? bwd_layout(s).total : 0;
}

hipError_t launch_attn_bwd(const LaunchShape& s, const void* q, const void* k, const void* v,
                           const int32_t* idx, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, void* ws,
                           hipStream_t st) {
  if (s.bf16)
    return s.head_dim == 128
               ? launch_bwd<bf16_t, 128>(s, q, k, v, idx, out, lse, dout, dq, dk, dv, ws, st)
               : launch_bwd<bf16_t, 64>(s, q, k, v, idx, out, lse, dout, dq, dk, dv, ws, st);
  return s.head_dim == 128
             ? launch_bwd<float, 128>(s, q, k, v, idx, out, lse, dout, dq, dk, dv, ws, st)
             : launch_bwd<float, 64>(s, q, k, v, idx, out, lse, dout, dq, dk, dv, ws, st);
}

}  // namespace pisa
