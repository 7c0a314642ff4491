// Two-stage PISA selection for bf16 inputs (PISA reading page §05, Algorithm
// 1 and §5.1: the intermediate levels run per query, then key blocks are
// loaded once and scored for every query that needs them).
//
// The split is placed one level higher than the pages' (which score the leaf
// level in stage 2): here stage 2 works per kept level-3 node n (4 leaves,
// 4C raw keys).  Its MFMA pass gives q.k for every key under n; the mean of a
// leaf's logits equals the leaf summary's logit (eq. (4) is a mean and the dot
// product is linear), so one pass yields both the level-2 scores of n's two
// children (eq. (7) over child summaries) and the exact leaf LSEs (eq. (7) at
// level 1).  Each query then needs K (not 2K) key groups and the level-2
// summary gathers disappear from stage 1.
//
//   stage 1   levels L..3 of the descent, kept level-3 nodes -> s1_nodes[u][K]:
//             K <= 16: one lane per query (select_lpq.h); K <= 32: one
//             wavefront per (b, kv head, t) (stage1_kernel below).
//   scan      one workgroup: bucket offsets and the stage-2 work list.
//   scatter   pairs (row << 5 | slot) into per-node buckets.
//   stage 2   one workgroup per (node, <= 1024 / G pairs): each wave holds one
//             leaf's keys in registers, the pairs' query rows pass through LDS
//             in batches; bf16 MFMA 32x32x16 (keys x queries), per-leaf LSE
//             and mean.
//   final     level-2 and leaf decisions from the stage-2 scores, ascending
//             leaf list out: one lane per query (K <= 16) or one wavefront
//             per query (final_kernel below).
// Pair order inside a bucket depends on atomics, but every pair's scores are
// computed by the same instruction sequence whatever its position, so the
// outputs are bitwise reproducible.
#include <algorithm>
#include <cstdlib>
#include <cfloat>
#include <type_traits>

#include "bucket.h"
#include "pisa_common.h"
#include "pisa_launch.h"
#include "select_core.h"
#include "select_lpq.h"

namespace pisa {

namespace {

constexpr int kSplitLevel = 3;   // stage 1 decides levels L..3
constexpr int kS1Waves = 4;
constexpr int kS2Threads = 256;
constexpr int kS2Rows = 64;       // (pair, head) rows per stage-2 batch (default, G = 1)
constexpr int kS2RowsGrouped = 128;  // default for G > 1 (measured: 9-13% faster there)
constexpr int kS2ItemRows = 1024; // (pair, head) rows per stage-2 work item (default)

// Tuning overrides of the stage-2 work decomposition (read per call):
//   PISA_S2_ITEM_ROWS   (pair, head) rows served by one load of a level-3
//                       node's keys: a power of two in [64, 4096];
//   PISA_S2_BATCH_ROWS  rows staged in LDS per batch: 32, 64 or 128
//                       (default 64 for one head per KV head, else 128).
// and of stage 1:
//   PISA_S1_TILE_ROWS   child rows per window of the union tiles (16 heads
//                       per KV head): a multiple of 64 in [64, 8192], default
//                       8192; smaller windows only serve tests of the window
//                       loop at moderate lengths.
// Other values fall back to the defaults.  The workspace size follows the
// item size, so set them before pisa_workspace_bytes.
int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == 0 && x > 0 && x < (1 << 20)) ? int(x) : dflt;
}
int s2_item_rows() {
  const int x = env_int("PISA_S2_ITEM_ROWS", kS2ItemRows);
  return (x >= 64 && x <= 4096 && (x & (x - 1)) == 0) ? x : kS2ItemRows;
}
int s2_batch_rows(int group) {
  const int dflt = group == 1 ? kS2Rows : kS2RowsGrouped;
  const int x = env_int("PISA_S2_BATCH_ROWS", dflt);
  return (x == 32 || x == 64 || x == 128) ? x : dflt;
}
int s1_tile_rows() {
  const int x = env_int("PISA_S1_TILE_ROWS", lpq::kTileRows);
  return (x >= 64 && x <= lpq::kTileRows && x % 64 == 0) ? x : lpq::kTileRows;
}
constexpr int kS2Cols = 32;      // MFMA 32x32x16: 32 (query, head) columns
constexpr int kScoreStride = 8;  // floats per pair: 4 leaf LSE, 2 level-2, 2 pad

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

struct Ws {
  int* counts;        // [n_buckets]
  int* offsets;       // [n_buckets + 1]
  int* cursors;       // [n_buckets]
  int* item_offsets;  // [n_buckets + 1]
  int* s1_nodes;      // [U * K]
  int* pairs;         // [U * K]
  float* scores;      // [U * K * kScoreStride]
  bf16_t* plane_hi;   // [B * Hkv * R * d] bf16 hi part of the pyramid
  bf16_t* plane_lo;   // [B * Hkv * R * d] bf16 lo part
};

struct WsLayout {
  size_t counts, offsets, cursors, item_offsets, s1_nodes, pairs, scores, plane_hi, plane_lo,
      total;
  int n_buckets, max_items;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout ws_layout(const LaunchShape& s) {
  WsLayout w;
  const size_t units = (size_t)s.batch * s.heads_kv * s.seq_len;
  const int m3 = s.lv.n >= kSplitLevel ? s.lv.size[kSplitLevel - 1] : 1;
  w.n_buckets = s.batch * s.heads_kv * m3;
  w.max_items = bucket::max_items(units * s.topk, w.n_buckets, s2_item_rows() / s.group);
  size_t off = 0;
  w.counts = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.cursors = off; off = align256(off + sizeof(int) * w.n_buckets);
  w.item_offsets = off; off = align256(off + sizeof(int) * (w.n_buckets + 1));
  w.s1_nodes = off; off = align256(off + sizeof(int) * units * s.topk);
  w.pairs = off; off = align256(off + sizeof(int) * units * s.topk);
  w.scores = off; off = align256(off + sizeof(float) * units * s.topk * kScoreStride);
  const size_t plane = (size_t)s.batch * s.heads_kv * s.lv.rows * s.head_dim * sizeof(bf16_t);
  w.plane_hi = off; off = align256(off + plane);
  w.plane_lo = off; off = align256(off + plane);
  w.total = off;
  return w;
}

Ws ws_bind(const WsLayout& l, void* base) {
  char* b = static_cast<char*>(base);
  return {reinterpret_cast<int*>(b + l.counts), reinterpret_cast<int*>(b + l.offsets),
          reinterpret_cast<int*>(b + l.cursors), reinterpret_cast<int*>(b + l.item_offsets),
          reinterpret_cast<int*>(b + l.s1_nodes), reinterpret_cast<int*>(b + l.pairs),
          reinterpret_cast<float*>(b + l.scores), reinterpret_cast<bf16_t*>(b + l.plane_hi),
          reinterpret_cast<bf16_t*>(b + l.plane_lo)};
}

// ---------------------------------------------------------------------------
// Stage 1
// ---------------------------------------------------------------------------

// Eq. (7) scores of up to 64 candidates (lane j owns candidate j) at an
// intermediate level, coalesced: each child summary row (fp32, D floats) is
// read by 8 lanes holding D/8 columns each; the group's query columns for
// those lanes sit in registers.  Returns this lane's candidate score (nats).
template <int D, int GM>
__device__ __forceinline__ float score_level_coalesced(const float* __restrict__ child_rows,
                                                       int m_child, int node, bool rankable,
                                                       const float (&qreg)[GM][D / 8],
                                                       int group, float scale_log2,
                                                       float* dots /* LDS [GM][128] */) {
  constexpr int CPL = D / 8;  // columns per lane
  const int lane = lane_id();
  const uint64_t rm = ballot(rankable);
  // rows: candidate j -> child rows 2j (always exists) and 2j+1 (if < m_child)
  const int n_cand = 64 - __builtin_clzll(rm | 1ull);  // highest rankable lane + 1
  const int n_rows = 2 * n_cand;
  const int sub = lane >> 3, part = lane & 7;
  constexpr int BATCH = 4;  // passes of 8 rows whose loads are issued together
  for (int r0 = 0; r0 < n_rows; r0 += 8 * BATCH) {
    float4 x[BATCH][CPL / 4];
    bool live[BATCH];
#pragma unroll
    for (int pp = 0; pp < BATCH; ++pp) {
      const int r = r0 + 8 * pp + sub;
      const int cand = r >> 1;
      const int cnode = __shfl(node, cand & 63, kWave);
      live[pp] = r < n_rows && ((rm >> (cand & 63)) & 1ull) && (2 * cnode + (r & 1) < m_child);
      const float* row = child_rows + (size_t)(live[pp] ? 2 * cnode + (r & 1) : 0) * D + part * CPL;
#pragma unroll
      for (int c = 0; c < CPL / 4; ++c)
        x[pp][c] = live[pp] ? *reinterpret_cast<const float4*>(row + 4 * c) : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int pp = 0; pp < BATCH; ++pp) {
      const int r = r0 + 8 * pp + sub;
      float acc[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        acc[h] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL / 4; ++c)
          acc[h] += qreg[h][4 * c] * x[pp][c].x + qreg[h][4 * c + 1] * x[pp][c].y +
                    qreg[h][4 * c + 2] * x[pp][c].z + qreg[h][4 * c + 3] * x[pp][c].w;
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < group) {
          float v = acc[h];
          v += __shfl_xor(v, 1, kWave);
          v += __shfl_xor(v, 2, kWave);
          v += __shfl_xor(v, 4, kWave);
          if (part == 0 && r < 128) dots[h * 128 + r] = v;
        }
      }
    }
  }
  wave_lds_sync();
  float total = neg_inf();
  if (rankable) {
    const bool has1 = 2 * node + 1 < m_child;
    total = 0.f;
    for (int h = 0; h < group; ++h) {
      const float z0 = dots[h * 128 + 2 * lane] * scale_log2;
      if (has1) {
        const float z1 = dots[h * 128 + 2 * lane + 1] * scale_log2;
        const float m = fmaxf(z0, z1);
        total += m + log2f(exp2f(z0 - m) + exp2f(z1 - m));
      } else {
        total += z0;
      }
    }
    total *= kLn2;
  }
  wave_lds_sync();
  return total;
}

template <typename T, int D, int GM>
__global__ __launch_bounds__(kS1Waves * kWave) void stage1_kernel(
    const T* __restrict__ q, const float* __restrict__ pyr, int* __restrict__ s1_nodes,
    int heads_q, int heads_kv, int n_tok, int block, int topk, int group, int causal, int force,
    float scale_log2, LevelTable lv) {
  constexpr int CPL = D / 8;
  __shared__ int nbuf_all[kS1Waves][kWave];
  __shared__ float dots_all[kS1Waves][GM * 128];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * kS1Waves + wave;
  if (t >= n_tok) return;
  const int bh = blockIdx.y;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int lane = lane_id();
  int* nbuf = nbuf_all[wave];
  float* dots = dots_all[wave];
  // The group's query columns for this lane's 8-lane part.
  float qreg[GM][CPL];
  const int part = lane & 7;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < group) {
      const T* qrow = q + (((size_t)b * heads_q + (size_t)kvh * group + h) * n_tok + t) * D +
                      part * CPL;
      constexpr int VEC = Vec16<T>::n;
#pragma unroll
      for (int c = 0; c < CPL; c += VEC) load16(qrow + c, &qreg[h][c]);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) qreg[h][c] = 0.f;
    }
  }
  const float* pb = pyr + (size_t)bh * lv.rows * D;
  const bool cz = causal != 0, fz = force != 0;
  const int cur = t / block;
  int node = lane == 0 ? 0 : -1;
  bool keep = false;
  for (int l = lv.n; l >= kSplitLevel; --l) {
    const int sh = l - 1;
    const int lim = cur >> sh;
    bool valid = node >= 0 && (!cz || node <= lim);
    const uint64_t vm = ballot(valid);
    const int ncand = __popcll(vm);
    if (valid) nbuf[lanes_below(vm)] = node;
    wave_lds_sync();
    node = lane < ncand ? nbuf[lane] : -1;
    wave_lds_sync();
    valid = lane < ncand;
    const bool forced = valid && cz &&
                        (node == lim || (fz && (node == 0 || (cur >= 1 && node == ((cur - 1) >> sh)))));
    if (ncand <= topk) {
      keep = valid;
    } else {
      const int keep_n = topk - __popcll(ballot(forced));
      const bool rankable = valid && !forced;
      const float s = score_level_coalesced<D, GM>(pb + (size_t)lv.off[l - 2] * D, lv.size[l - 2],
                                               node, rankable, qreg, group, scale_log2, dots);
      const uint64_t rm = ballot(rankable);
      int rank = 0;
      uint64_t it = rm;
      while (it) {
        const int j = __builtin_ctzll(it);
        it &= it - 1;
        rank += ranks_before(readlane_f(s, j), readlane_i(node, j), s, node) ? 1 : 0;
      }
      keep = forced || (rankable && rank < keep_n);
    }
    if (l > kSplitLevel) {
      const uint64_t km = ballot(keep);
      const int p = lanes_below(km);
      const int m_child = lv.size[l - 2];
      if (keep && p < topk) {  // p < K unless NaN inputs broke the order
        nbuf[2 * p] = 2 * node;
        nbuf[2 * p + 1] = (2 * node + 1 < m_child) ? 2 * node + 1 : -1;
      }
      wave_lds_sync();
      node = lane < 2 * min(__popcll(km), topk) ? nbuf[lane] : -1;
      wave_lds_sync();
      keep = false;
    }
  }
  // Kept level-3 nodes: compact into s1_nodes[u][0..nk), -1 after.
  const uint64_t km = ballot(keep);
  const int nk = __popcll(km);
  const size_t u = (size_t)bh * n_tok + t;
  int* out = s1_nodes + u * topk;
  if (keep) out[lanes_below(km)] = node;
  if (lane >= nk && lane < topk) out[lane] = -1;
}

// ---------------------------------------------------------------------------
// Stage 2
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Stage-2 batches of ROWS (pair, head) rows: row r of a batch's LDS tile holds
// the query row of pair r / G, head r % G (D bf16, rows padded to D + 8 so
// that the MFMA operand reads of 32 consecutive rows spread over the banks).
// Rows past the item repeat its last pair.  Thread x of the workgroup loads
// pieces x + i * kS2Threads (i < LOADS) of the tile into registers one batch
// ahead and writes them to LDS when the batch starts.
template <int D, int G, int ROWS>
struct S2Tile {
  static constexpr int PIECES = D / 8;                      // 16-byte pieces per row
  static constexpr int LOADS = ROWS * PIECES / kS2Threads;  // pieces per thread
  static constexpr int PAIRS = ROWS / G;
  static constexpr int QROW = D + 8;  // padded row (bf16): 32 rows' 16-byte reads spread over banks
  static_assert(LOADS >= 1 && ROWS % 32 == 0 && PAIRS >= 1, "stage-2 tile shape");

  // Pair ids of the rows this thread's pieces of batch bt belong to.
  __device__ __forceinline__ static void pair_ids(int (&pid)[LOADS], const int* __restrict__ pairs,
                                                  int start, int len, int bt) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = (threadIdx.x + i * kS2Threads) / PIECES;
      pid[i] = pairs[start + min(bt * PAIRS + r / G, len - 1)];
    }
  }

  __device__ __forceinline__ static void load(u32x4_t (&v)[LOADS], const int (&pid)[LOADS],
                                              const bf16_t* __restrict__ qh, int bh, int n_tok) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int x = threadIdx.x + i * kS2Threads;
      const int r = x / PIECES, p = x % PIECES;
      const int t = (pid[i] >> 5) - bh * n_tok;  // pair = (row << 5) | slot
      v[i] = *reinterpret_cast<const u32x4_t*>(qh + ((size_t)(r % G) * n_tok + t) * D + 8 * p);
    }
  }

  __device__ __forceinline__ static void store(bf16_t* tile, const u32x4_t (&v)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int x = threadIdx.x + i * kS2Threads;
      const int r = x / PIECES, p = x % PIECES;
      *reinterpret_cast<u32x4_t*>(tile + r * QROW + 8 * p) = v[i];
    }
  }

  // Piece p of row r (an MFMA operand).
  __device__ __forceinline__ static bf16x8_t read(const bf16_t* tile, int r, int p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(tile + r * QROW + 8 * p));
  }
};

// One workgroup per work item: level-3 node n of KV head bh and up to
// item_pairs of its (query, slot) pairs; wavefront w owns leaf 4n + w and
// keeps its 64 raw keys as MFMA A operands in registers for the whole item.
// The item's pairs run in batches of ROWS / G.  Batch bt's query rows were
// loaded into registers during batch bt - 1; per batch:
//   1. they go to one of two LDS tiles and the loads of batch bt + 1 start;
//      an LDS-only barrier (no wait for the loads or for earlier score
//      stores: only the registers' uses wait for their loads);
//   2. each wave walks the batch's rows 32 columns at a time: S = K_leaf . Q^T
//      on bf16 MFMA 32x32x16 (a lane holds 32 keys of one column), then the
//      exact leaf LSE (eq. (7) at level 1: max, sum of exp2) and the mean
//      logit, which equals q . kbar_leaf (eq. (4) is a mean), go to LDS;
//   3. after an LDS-only barrier every thread finishes one pair: the four
//      leaf LSEs and the two level-2 scores LSE(mean_2c, mean_2c+1), each
//      summed over the group's heads (eq. (11)), in nats.
template <int D, int G, int ROWS>
__global__ __launch_bounds__(kS2Threads, (G == 1 || D == 64) ? 3 : 2) void stage2_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const int* __restrict__ item_offsets, const int* __restrict__ offsets,
    const int* __restrict__ pairs, float* __restrict__ scores, int n_buckets, int heads_q,
    int heads_kv, int n_tok, int topk, int m3, float scale_log2, int item_pairs) {
  using Tile = S2Tile<D, G, ROWS>;
  constexpr int KSTEPS = D / 16;
  constexpr int PAIRS = Tile::PAIRS;
  constexpr int LEAF = 64;  // keys per leaf (C = 64)
  __shared__ __attribute__((aligned(16))) bf16_t tile_a[ROWS * Tile::QROW];
  __shared__ __attribute__((aligned(16))) bf16_t tile_b[ROWS * Tile::QROW];
  __shared__ float xs[4][2][ROWS];  // [leaf][lse, mean][row], log2 units
  int bucket, start, len;
  if (!bucket::locate_item(item_offsets, offsets, n_buckets, blockIdx.x, item_pairs, &bucket,
                           &start, &len))
    return;
  const int bh = bucket / m3, node = bucket % m3;
  const int b = bh / heads_kv, kvh = bh % heads_kv;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int col = lane & 31, kh = lane >> 5;
  const bf16_t* qh = q + ((size_t)b * heads_q + (size_t)kvh * G) * n_tok * D;
  const int n_batches = (len + PAIRS - 1) / PAIRS;

  // Batch 0's rows, and the pair ids of batch 1 (rows and the pair each
  // finishing thread owns).
  int pid[Tile::LOADS];
  u32x4_t stage[Tile::LOADS];
  Tile::pair_ids(pid, pairs, start, len, 0);
  Tile::load(stage, pid, qh, bh, n_tok);
  int fin_pid = pairs[start + min(tid, len - 1)];
  Tile::pair_ids(pid, pairs, start, len, 1);

  const int leaf_tok0 = (4 * node + wave) * LEAF;
  const int n_keys = max(0, min(LEAF, n_tok - leaf_tok0));  // keys of this wave's leaf
  // A operands: key rows leaf_tok0 + 32 rb + col (rows past the sequence end
  // repeat its last key; they are masked below).
  const bf16_t* kb = k + (size_t)bh * n_tok * D;
  bf16x8_t ka[2][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = min(leaf_tok0 + 32 * rb + col, n_tok - 1);
    const bf16_t* kr = kb + (size_t)row * D + 8 * kh;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) ka[rb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 16 * s));
  }
  const float inv_keys = n_keys > 0 ? 1.f / float(n_keys) : 0.f;
  // The keys and batch 0 are in before the loop: inside it, only the staged
  // registers' uses wait for the loads of the next batch.
  wait_vmcnt<0>();

  // One batch, compiled for a leaf with all C keys (no masking) and for the
  // sequence's last, partial leaf.  Waves of one workgroup may run different
  // copies; both pass the same barriers in the same order.
  auto batch = [&](auto full_tag, int bt, bf16_t* cur) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full_tag)::value;
    const int blen = min(PAIRS, len - bt * PAIRS);  // pairs in this batch
    // cur was last read two batches ago (both barriers of batch bt - 1 lie
    // between); xs was last read by batch bt - 1's finishing step, which
    // every thread completes before the barrier below.
    Tile::store(cur, stage);
    const int my_pid = fin_pid;
    // The next batch's loads are issued unconditionally (past the item's end
    // the clamped rows repeat its last pair, one cache line), so that every
    // batch issues the same memory operations and the waits for the staged
    // rows never have to cover the score stores that follow them.
    Tile::load(stage, pid, qh, bh, n_tok);
    fin_pid = pairs[start + min((bt + 1) * PAIRS + tid, len - 1)];
    Tile::pair_ids(pid, pairs, start, len, bt + 2);
    lds_barrier();

    const int n_chunks = (blen * G + 31) / 32;
    for (int ch = 0; ch < n_chunks; ++ch) {
      const int r = 32 * ch + col;
      f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8_t bq = Tile::read(cur, r, 2 * s + kh);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0][s], bq, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[1][s], bq, acc1, 0, 0, 0);
      }
      // Lane holds the logits of keys (i/4)*8 + 4kh + i%4 (acc0) and 32 + that (acc1).
      float sraw = 0.f, se = 0.f;
      if constexpr (!kFull) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = (i / 4) * 8 + 4 * kh + (i % 4);
          sraw += (kr < n_keys ? acc0[i] : 0.f) + (kr + 32 < n_keys ? acc1[i] : 0.f);
          acc0[i] = kr < n_keys ? acc0[i] : neg_inf();
          acc1[i] = kr + 32 < n_keys ? acc1[i] : neg_inf();
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) sraw += acc0[i] + acc1[i];
      }
      // The exps are taken relative to the mean logit, which the level-2
      // scores need anyway: the sum is >= 1 (some logit is >= the mean) and
      // only overflows when a logit exceeds the mean by ~128 (log2 units);
      // then the wave redoes the column relative to its maximum.
      sraw += __shfl_xor(sraw, 32, kWave);
      const float mean = sraw * inv_keys * scale_log2;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        se += fast_exp2(fmaf(acc0[i], scale_log2, -mean)) + fast_exp2(fmaf(acc1[i], scale_log2, -mean));
      se += __shfl_xor(se, 32, kWave);
      float ref = mean;
      if (__ballot(!(se <= FLT_MAX)) != 0) {
        float m = fmaxf(fmaxf(acc0[0], acc0[1]), fmaxf(acc1[0], acc1[1]));
#pragma unroll
        for (int i = 2; i < 16; i += 2)
          m = fmaxf(m, fmaxf(fmaxf(acc0[i], acc0[i + 1]), fmaxf(acc1[i], acc1[i + 1])));
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        ref = (kFull || n_keys > 0) ? m * scale_log2 : 0.f;
        se = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          se += fast_exp2(fmaf(acc0[i], scale_log2, -ref)) + fast_exp2(fmaf(acc1[i], scale_log2, -ref));
        se += __shfl_xor(se, 32, kWave);
      }
      if (kh == 0) {
        const bool has = kFull || n_keys > 0;
        xs[wave][0][r] = has ? ref + fast_log2(se) : neg_inf();
        xs[wave][1][r] = has ? mean : neg_inf();
      }
    }
    lds_barrier();  // xs complete

    // One pair per thread.
    if (tid < blen) {
      float o[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int hh = 0; hh < G; ++hh) {
        const int r = tid * G + hh;
#pragma unroll
        for (int f = 0; f < 4; ++f) o[f] += xs[f][0][r];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const float a = xs[2 * c2][1][r], bb = xs[2 * c2 + 1][1][r];
          const float mx = fmaxf(a, bb), mn = fminf(a, bb);
          // a missing leaf has mean -inf and drops out
          o[4 + c2] += mn == neg_inf() ? mx : mx + fast_log2(1.f + fast_exp2(mn - mx));
        }
      }
      float* dst = scores + ((size_t)(my_pid >> 5) * topk + (my_pid & 31)) * kScoreStride;
      *reinterpret_cast<float4*>(dst) =
          make_float4(o[0] * kLn2, o[1] * kLn2, o[2] * kLn2, o[3] * kLn2);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4] * kLn2, o[5] * kLn2, 0.f, 0.f);
    }
  };
  auto run = [&](auto full_tag) __attribute__((always_inline)) {
    for (int bt = 0; bt < n_batches; bt += 2) {
      batch(full_tag, bt, tile_a);
      if (bt + 1 < n_batches) batch(full_tag, bt + 1, tile_b);
    }
  };
  if (n_keys == LEAF)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// ---------------------------------------------------------------------------
// Final decisions at levels 2 and 1
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kS1Waves * kWave) void final_kernel(
    const int* __restrict__ s1_nodes, const float* __restrict__ scores, int32_t* __restrict__ idx,
    float* __restrict__ score_out, int n_tok, int block, int topk, int causal, int force, int m1,
    int m2) {
  __shared__ int nbuf_all[kS1Waves][kWave];
  __shared__ int sbuf_all[kS1Waves][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * kS1Waves + wave;
  if (t >= n_tok) return;
  const int bh = blockIdx.y;
  const int lane = lane_id();
  int* nbuf = nbuf_all[wave];
  int* sbuf = sbuf_all[wave];
  const size_t u = (size_t)bh * n_tok + t;
  const bool cz = causal != 0, fz = force != 0;
  const int cur = t / block;
  // Level-2 candidates: children of the kept level-3 nodes.  src = slot*8 + j
  // locates the candidate's score in scores[u][slot][j].
  int node = -1, src = -1;
  {
    const int slot = lane >> 1, c = lane & 1;
    const int n3 = slot < topk ? s1_nodes[u * topk + slot] : -1;
    if (n3 >= 0 && 2 * n3 + c < m2) {
      node = 2 * n3 + c;
      src = slot * kScoreStride + 4 + c;
    }
  }
  bool keep = false;
  float score = pos_inf();
  for (int l = 2; l >= 1; --l) {
    const int sh = l - 1;
    const int lim = cur >> sh;
    bool valid = node >= 0 && (!cz || node <= lim);
    const uint64_t vm = ballot(valid);
    const int ncand = __popcll(vm);
    if (valid) {
      nbuf[lanes_below(vm)] = node;
      sbuf[lanes_below(vm)] = src;
    }
    wave_lds_sync();
    node = lane < ncand ? nbuf[lane] : -1;
    src = lane < ncand ? sbuf[lane] : -1;
    wave_lds_sync();
    valid = lane < ncand;
    const bool forced = valid && cz &&
                        (node == lim || (fz && (node == 0 || (cur >= 1 && node == ((cur - 1) >> sh)))));
    if (ncand <= topk) {
      keep = valid;
      score = pos_inf();
    } else {
      const int keep_n = topk - __popcll(ballot(forced));
      const bool rankable = valid && !forced;
      const float s = rankable ? scores[u * topk * kScoreStride + src] : neg_inf();
      const uint64_t rm = ballot(rankable);
      int rank = 0;
      uint64_t it = rm;
      while (it) {
        const int j = __builtin_ctzll(it);
        it &= it - 1;
        rank += ranks_before(readlane_f(s, j), readlane_i(node, j), s, node) ? 1 : 0;
      }
      keep = forced || (rankable && rank < keep_n);
      score = forced ? pos_inf() : s;
    }
    if (l == 2) {
      // Expand kept level-2 nodes into leaves; leaf score index = slot*8 + 2*c + c'.
      const uint64_t km = ballot(keep);
      const int p = lanes_below(km);
      if (keep && p < topk) {  // p < K unless NaN inputs broke the order
        const int slot = src / kScoreStride, c = src % kScoreStride - 4;
        nbuf[2 * p] = 2 * node;
        sbuf[2 * p] = slot * kScoreStride + 2 * c;
        const bool has1 = 2 * node + 1 < m1;
        nbuf[2 * p + 1] = has1 ? 2 * node + 1 : -1;
        sbuf[2 * p + 1] = slot * kScoreStride + 2 * c + 1;
      }
      wave_lds_sync();
      const int n2 = 2 * min(__popcll(km), topk);
      node = lane < n2 ? nbuf[lane] : -1;
      src = lane < n2 ? sbuf[lane] : -1;
      wave_lds_sync();
      keep = false;
    }
  }
  SelectResult r{node, score, keep};
  write_selection(r, topk, idx + u * topk, score_out ? score_out + u * topk : nullptr);
}

template <typename T, int D, int GM>
hipError_t stage1_launch(const LaunchShape& s, const void* q, const float* pyr, const Ws& w,
                         hipStream_t st) {
  dim3 grid((s.seq_len + kS1Waves - 1) / kS1Waves, s.batch * s.heads_kv);
  prof::Scope ps("select_stage1", st);
  hipLaunchKernelGGL((stage1_kernel<T, D, GM>), grid, dim3(kS1Waves * kWave), 0, st,
                     static_cast<const T*>(q), pyr, w.s1_nodes, s.heads_q, s.heads_kv,
                     s.seq_len, s.block, s.topk, s.group, s.causal ? 1 : 0, s.force ? 1 : 0,
                     s.scale * kLog2e, s.lv);
  return hipGetLastError();
}

template <int D, int G>
hipError_t stage1_lpq_launch(const LaunchShape& s, const void* q, const float* pyr, const Ws& w,
                             hipStream_t st) {
  constexpr int T = kWave / G;  // queries per wave
  dim3 grid((s.seq_len + T * lpq::kWaves - 1) / (T * lpq::kWaves), s.batch * s.heads_kv);
  {
    prof::Scope ps("select_split_planes", st);
    const int heads = s.batch * s.heads_kv;
    const size_t head_len = (size_t)s.lv.rows * D, skip = (size_t)s.lv.size[0] * D;
    const size_t groups = (head_len - skip) / 8 * heads;
    if (groups > 0)
      hipLaunchKernelGGL(lpq::split_planes_kernel, dim3(bucket::grid_for(groups)), dim3(256), 0, st,
                         pyr, w.plane_hi, w.plane_lo, heads, head_len, skip, s.scale * kLog2e);
  }
  prof::Scope ps("select_stage1", st);
  hipLaunchKernelGGL((lpq::stage1_kernel<D, G>), grid, dim3(lpq::kWaves * kWave), 0, st,
                     static_cast<const bf16_t*>(q), w.plane_hi, w.plane_lo, w.s1_nodes,
                     s.heads_q, s.heads_kv, s.seq_len, s.block, s.topk, s.causal ? 1 : 0,
                     s.force ? 1 : 0, s.lv, kSplitLevel, s1_tile_rows());
  return hipGetLastError();
}

}  // namespace

bool select_two_stage_supported(const LaunchShape& s) {
  const bool pow2_group = (s.group & (s.group - 1)) == 0;
  // pairs are stored as (row << 5) | slot in an int32
  const int64_t rows = (int64_t)s.batch * s.heads_kv * s.seq_len;
  if (s.variant != 0) return false;  // LSE scores only
  return s.bf16 && s.block == 64 && (s.head_dim == 64 || s.head_dim == 128) &&
         s.lv.n >= kSplitLevel + 1 && pow2_group && s.topk <= 32 &&
         // the lane-per-query kernels (K <= 16) take every group size
         (s.group <= 4 || s.topk <= lpq::kMaxK) && rows < (int64_t(1) << 26);
}

size_t select_two_stage_ws_bytes(const LaunchShape& s) {
  return select_two_stage_supported(s) ? ws_layout(s).total : 0;
}

hipError_t launch_select_two_stage(const LaunchShape& s, const void* q, const void* k,
                                   const float* pyr, int32_t* idx, float* score, void* ws,
                                   hipStream_t st) {
  const WsLayout lay = ws_layout(s);
  const Ws w = ws_bind(lay, ws);
  const int m1 = s.lv.size[0], m2 = s.lv.size[1], m3 = s.lv.size[kSplitLevel - 1];
  hipError_t e;
  if (s.topk <= 16) {
    switch (s.group * 1000 + s.head_dim) {
      case 1128: e = stage1_lpq_launch<128, 1>(s, q, pyr, w, st); break;
      case 1064: e = stage1_lpq_launch<64, 1>(s, q, pyr, w, st); break;
      case 2128: e = stage1_lpq_launch<128, 2>(s, q, pyr, w, st); break;
      case 2064: e = stage1_lpq_launch<64, 2>(s, q, pyr, w, st); break;
      case 4128: e = stage1_lpq_launch<128, 4>(s, q, pyr, w, st); break;
      case 4064: e = stage1_lpq_launch<64, 4>(s, q, pyr, w, st); break;
      case 8128: e = stage1_lpq_launch<128, 8>(s, q, pyr, w, st); break;
      case 8064: e = stage1_lpq_launch<64, 8>(s, q, pyr, w, st); break;
      case 16128: e = stage1_lpq_launch<128, 16>(s, q, pyr, w, st); break;
      default: e = stage1_lpq_launch<64, 16>(s, q, pyr, w, st); break;
    }
  } else {
    e = s.group == 1 ? (s.head_dim == 128 ? stage1_launch<bf16_t, 128, 1>(s, q, pyr, w, st)
                                          : stage1_launch<bf16_t, 64, 1>(s, q, pyr, w, st))
                     : (s.head_dim == 128 ? stage1_launch<bf16_t, 128, 4>(s, q, pyr, w, st)
                                          : stage1_launch<bf16_t, 64, 4>(s, q, pyr, w, st));
  }
  if (e != hipSuccess) return e;
  {
    prof::Scope ps("select_sort", st);
    e = bucket::sort_pairs(w.s1_nodes, s.batch * s.heads_kv, s.seq_len, s.topk, m3,
                           s2_item_rows() / s.group,
                           w.counts, w.offsets, w.cursors, w.item_offsets, w.pairs, nullptr,
                           false, st);
  }
  if (e != hipSuccess) return e;
  {
    prof::Scope ps2("select_stage2", st);
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const float sl = s.scale * kLog2e;
    const int item_pairs = s2_item_rows() / s.group;
    const int rows = s2_batch_rows(s.group);
#define PISA_S2_ROWS(D, G, ROWS)                                                              \
  hipLaunchKernelGGL((stage2_kernel<D, G, ROWS>), dim3(lay.max_items), dim3(kS2Threads), 0, st, \
                     qb, kb, w.item_offsets, w.offsets, w.pairs, w.scores, lay.n_buckets,     \
                     s.heads_q, s.heads_kv, s.seq_len, s.topk, m3, sl, item_pairs)
#define PISA_S2(D, G)          \
  if (rows == 32) {            \
    PISA_S2_ROWS(D, G, 32);    \
  } else if (rows == 128) {    \
    PISA_S2_ROWS(D, G, 128);   \
  } else {                     \
    PISA_S2_ROWS(D, G, 64);    \
  }
    switch (s.group * 1000 + s.head_dim) {
      case 1128: PISA_S2(128, 1); break;
      case 1064: PISA_S2(64, 1); break;
      case 2128: PISA_S2(128, 2); break;
      case 2064: PISA_S2(64, 2); break;
      case 4128: PISA_S2(128, 4); break;
      case 4064: PISA_S2(64, 4); break;
      case 8128: PISA_S2(128, 8); break;
      case 8064: PISA_S2(64, 8); break;
      case 16128: PISA_S2(128, 16); break;
      default: PISA_S2(64, 16); break;
    }
#undef PISA_S2
#undef PISA_S2_ROWS
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof::Scope ps3("select_final", st);
  if (s.topk <= lpq::kMaxK) {
    const int per_group = lpq::kWaves * kWave;
    dim3 grid((s.seq_len + per_group - 1) / per_group, s.batch * s.heads_kv);
    const bool vec_out = (s.topk % 4) == 0 && (reinterpret_cast<uintptr_t>(idx) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(score) % 16) == 0;
    hipLaunchKernelGGL((lpq::final_kernel<kScoreStride>), grid, dim3(per_group), 0, st,
                       w.s1_nodes, w.scores, idx, score, s.seq_len, s.block, s.topk,
                       s.causal ? 1 : 0, s.force ? 1 : 0, m1, m2, vec_out ? 1 : 0);
  } else {
    dim3 grid((s.seq_len + kS1Waves - 1) / kS1Waves, s.batch * s.heads_kv);
    hipLaunchKernelGGL(final_kernel, grid, dim3(kS1Waves * kWave), 0, st, w.s1_nodes, w.scores,
                       idx, score, s.seq_len, s.block, s.topk, s.causal ? 1 : 0,
                       s.force ? 1 : 0, m1, m2);
  }
  return hipGetLastError();
}

}  // namespace pisa
