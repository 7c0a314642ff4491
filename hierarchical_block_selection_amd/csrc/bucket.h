// Counting sort of (row, slot) pairs into per-node buckets, used wherever a
// block of keys is loaded once and applied to every query that needs it.
//
// Input: node[u * K + slot] in [0, m) for live pairs (anything else is
// skipped), where row u belongs to head bh = u / n_tok; the pair's bucket is
// bh * m + node.  A pair is stored as (u << 5) | slot (K <= 32; callers keep
// u below 2^26).  A few buckets are very hot (the forced first block is in
// every row), so counting and scattering aggregate per workgroup in LDS and
// touch global counters once per (workgroup, bucket):
//   count:   grid (row chunks, heads); LDS histogram, then global adds;
//   scan:    one workgroup: exclusive bucket offsets, scatter cursors and
//            exclusive work-item offsets (ceil(count / per_item) items per
//            bucket); a consumer finds its item's bucket by binary search;
//   scatter: per workgroup, reserve a range in each touched bucket with one
//            global atomic, then place pairs with LDS atomics.  Order inside a
//            bucket is not fixed; consumers must not depend on it.  Optionally
//            the inverse map (pair id -> position) is written as well.
#pragma once

#include "pisa_common.h"

namespace pisa {
namespace bucket {

constexpr int kSortThreads = 1024;    // threads per count/scatter workgroup
constexpr int kRowsPerGroup = 512;    // least rows of one head per count/scatter workgroup
constexpr int kMaxRowsPerGroup = 2048;
constexpr int kMaxLocalBuckets = 8192;  // LDS histogram limit (two int arrays = 64 KB)
constexpr int kBatch = 16;  // slots per thread whose loads are issued together
constexpr int kStableRows = 128;  // rows per chunk of the stable sort (one wave scatters a chunk)

namespace {  // each translation unit keeps its own copy of these kernels

__global__ void fill_zero_kernel(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ __launch_bounds__(kSortThreads) void count_kernel(const int* __restrict__ node,
                                                    int* __restrict__ counts, int n_tok, int topk,
                                                    int m, int rpg) {
  extern __shared__ int hist[];  // [m]
  for (int i = threadIdx.x; i < m; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * rpg, t1 = min(t0 + rpg, n_tok);
  const int* src = node + ((size_t)bh * n_tok) * topk;
  const int i1 = t1 * topk;
  for (int ib = t0 * topk + threadIdx.x; ib < i1; ib += kBatch * blockDim.x) {
    int xs[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) xs[k] = src[min(ib + k * (int)blockDim.x, i1 - 1)];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (ib + k * (int)blockDim.x < i1 && xs[k] >= 0 && xs[k] < m) atomicAdd(&hist[xs[k]], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += blockDim.x)
    if (hist[i]) atomicAdd(&counts[(size_t)bh * m + i], hist[i]);
}

// Up to kScanLds buckets the counts pass through LDS, so that every global
// load and store of the scan is coalesced; beyond that each thread reads and
// writes its own contiguous range.
constexpr int kScanLds = 8192;
constexpr int kScanPer = kScanLds / 1024;  // buckets per thread when staged

__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ cursors,
                                                    int* __restrict__ item_offsets, int n_buckets,
                                                    int per_item) {
  __shared__ int part_pairs[1024 / kWave];  // per-wave totals
  __shared__ int part_items[1024 / kWave];
  extern __shared__ int c_s[];  // [n_buckets] when n_buckets <= kScanLds
  const bool staged = n_buckets <= kScanLds;
  const int tid = threadIdx.x;
  if (staged) {
    for (int i = tid; i < n_buckets; i += 1024) c_s[i] = counts[i];
    __syncthreads();
  }
  const int per = (n_buckets + 1023) / 1024;
  const int lo = min(tid * per, n_buckets), hi = min(lo + per, n_buckets);
  int sp = 0, si = 0;
  for (int i0 = lo; i0 < hi; i0 += 8) {  // 8 loads in flight
    int c8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = min(i0 + k, hi - 1);
      c8[k] = staged ? c_s[i] : counts[i];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (i0 + k < hi) {
        sp += c8[k];
        si += (c8[k] + per_item - 1) / per_item;
      }
  }
  // Exclusive prefix over the 1024 threads: inclusive scans inside each wave
  // (shuffles), then the 16 wave totals through LDS (one barrier).
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  int ip = sp, ii = si;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int a = __shfl_up(ip, o, kWave), c = __shfl_up(ii, o, kWave);
    if (lane >= o) {
      ip += a;
      ii += c;
    }
  }
  if (lane == kWave - 1) {
    part_pairs[wave] = ip;
    part_items[wave] = ii;
  }
  __syncthreads();
  int pos = ip - sp, ipos = ii - si;
  int tot_p = 0, tot_i = 0;
#pragma unroll
  for (int w = 0; w < 1024 / kWave; ++w) {
    const int a = part_pairs[w], c = part_items[w];
    pos += w < wave ? a : 0;
    ipos += w < wave ? c : 0;
    tot_p += a;
    tot_i += c;
  }
  if (tid == 1023) {
    offsets[n_buckets] = tot_p;
    item_offsets[n_buckets] = tot_i;
  }
  if (!staged) {
    for (int i = lo; i < hi; ++i) {
      const int c = counts[i];
      offsets[i] = pos;
      cursors[i] = pos;
      item_offsets[i] = ipos;
      pos += c;
      ipos += (c + per_item - 1) / per_item;
    }
    return;
  }
  // Staged: this thread's counts to registers, then its range of c_s becomes
  // the pair offsets (written out coalesced), then the item offsets.
  int cr[kScanPer];
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) cr[k] = lo + k < hi ? c_s[lo + k] : 0;
#pragma unroll
  for (int k = 0; k < kScanPer; ++k)
    if (lo + k < hi) {
      c_s[lo + k] = pos;
      pos += cr[k];
    }
  __syncthreads();
  for (int i = tid; i < n_buckets; i += 1024) {
    const int o = c_s[i];
    offsets[i] = o;
    cursors[i] = o;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kScanPer; ++k)
    if (lo + k < hi) {
      c_s[lo + k] = ipos;
      ipos += (cr[k] + per_item - 1) / per_item;
    }
  __syncthreads();
  for (int i = tid; i < n_buckets; i += 1024) item_offsets[i] = c_s[i];
}

inline size_t scan_lds_bytes(int n_buckets) {
  return n_buckets <= kScanLds ? sizeof(int) * (size_t)n_buckets : 0;
}

__global__ __launch_bounds__(kSortThreads) void scatter_kernel(const int* __restrict__ node,
                                                      int* __restrict__ cursors,
                                                      int* __restrict__ pairs,
                                                      int* __restrict__ inv, int n_tok, int topk,
                                                      int m, int rpg) {
  extern __shared__ int lds[];  // hist/base [m], local cursor [m]
  int* base = lds;
  int* cur = lds + m;
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    base[i] = 0;
    cur[i] = 0;
  }
  __syncthreads();
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * rpg, t1 = min(t0 + rpg, n_tok);
  const size_t row0 = (size_t)bh * n_tok;
  const int* src = node + row0 * topk;
  const int i1 = t1 * topk;
  for (int ib = t0 * topk + threadIdx.x; ib < i1; ib += kBatch * blockDim.x) {
    int xs[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) xs[k] = src[min(ib + k * (int)blockDim.x, i1 - 1)];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (ib + k * (int)blockDim.x < i1 && xs[k] >= 0 && xs[k] < m) atomicAdd(&base[xs[k]], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += blockDim.x)
    if (base[i]) base[i] = atomicAdd(&cursors[(size_t)bh * m + i], base[i]);
  __syncthreads();
  for (int ib = t0 * topk + threadIdx.x; ib < i1; ib += kBatch * blockDim.x) {
    int xs[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) xs[k] = src[min(ib + k * (int)blockDim.x, i1 - 1)];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = ib + k * (int)blockDim.x;
      const int x = xs[k];
      if (i < i1 && x >= 0 && x < m) {
        const int pos = base[x] + atomicAdd(&cur[x], 1);
        pairs[pos] = (int)(((row0 + i / topk) << 5) | (i % topk));
        if (inv) inv[row0 * topk + i] = pos;
      }
    }
  }
}

// Global-atomic fallbacks for more than kMaxLocalBuckets nodes per head.
__global__ void count_global_kernel(const int* __restrict__ node, int* __restrict__ counts,
                                    int n_tok, int topk, int m, size_t n_slots) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots;
       i += (size_t)gridDim.x * blockDim.x) {
    const int x = node[i];
    if (x < 0 || x >= m) continue;
    atomicAdd(&counts[(i / topk / n_tok) * m + x], 1);
  }
}

__global__ void scatter_global_kernel(const int* __restrict__ node, int* __restrict__ cursors,
                                      int* __restrict__ pairs, int* __restrict__ inv, int n_tok,
                                      int topk, int m, size_t n_slots) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots;
       i += (size_t)gridDim.x * blockDim.x) {
    const int x = node[i];
    if (x < 0 || x >= m) continue;
    const int pos = atomicAdd(&cursors[(i / topk / n_tok) * m + x], 1);
    pairs[pos] = (int)(((i / topk) << 5) | (i % topk));
    if (inv) inv[i] = pos;
  }
}

// Stable variant: each bucket lists its pairs in increasing (row, slot) order,
// so the pairs, their grouping into work items and every sum taken over them
// in that order are the same run to run.
//   count_wg:  per (chunk of kStableRows rows, head), the chunk's histogram
//              written out whole
//              to wgc[head][chunk][node] (no global atomics);
//   wg_prefix: per bucket, exclusive prefix of wgc over the chunks (in place)
//              and the bucket's total;
//   scatter_stable: one wave per (row chunk, head) walks its slots in order,
//              64 at a time; lanes holding the same node are ranked by lane
//              (ballot; LDS counters first single out the lanes whose node is
//              unique in the step), and a running base per node lives in LDS.
__global__ __launch_bounds__(256) void count_wg_kernel(const int* __restrict__ node,
                                                       int* __restrict__ wgc, int n_tok, int topk,
                                                       int m) {
  extern __shared__ int hist[];  // [m]
  for (int i = threadIdx.x; i < m; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * kStableRows, t1 = min(t0 + kStableRows, n_tok);
  const int* src = node + ((size_t)bh * n_tok) * topk;
  const int i1 = t1 * topk;
  for (int ib = t0 * topk + threadIdx.x; ib < i1; ib += kBatch * blockDim.x) {
    int xs[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) xs[k] = src[min(ib + k * (int)blockDim.x, i1 - 1)];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (ib + k * (int)blockDim.x < i1 && xs[k] >= 0 && xs[k] < m) atomicAdd(&hist[xs[k]], 1);
  }
  __syncthreads();
  int* dst = wgc + ((size_t)bh * gridDim.x + blockIdx.x) * m;
  for (int i = threadIdx.x; i < m; i += blockDim.x) dst[i] = hist[i];
}

// 16 buckets x 16 chunk segments per workgroup: each thread sums its
// segment, the segment offsets go through LDS, then each thread rewrites its
// segment as running prefixes.
constexpr int kPrefixBuckets = 16, kPrefixSegs = 16;
__global__ __launch_bounds__(256) void wg_prefix_kernel(int* __restrict__ wgc,
                                                        int* __restrict__ counts, int n_chunks,
                                                        int m, int n_buckets) {
  __shared__ int part[kPrefixSegs][kPrefixBuckets];
  const int bl = threadIdx.x % kPrefixBuckets, seg = threadIdx.x / kPrefixBuckets;
  const int bucket = blockIdx.x * kPrefixBuckets + bl;
  const bool ok = bucket < n_buckets;
  const int bh = ok ? bucket / m : 0, x = ok ? bucket % m : 0;
  int* col = wgc + (size_t)bh * n_chunks * m + x;
  const int per = (n_chunks + kPrefixSegs - 1) / kPrefixSegs;
  const int c0 = min(seg * per, n_chunks), c1 = min(c0 + per, n_chunks);
  int sum = 0;
  if (ok)
    for (int c = c0; c < c1; c += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) v[k] = col[(size_t)min(c + k, c1 - 1) * m];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (c + k < c1) sum += v[k];
    }
  part[seg][bl] = sum;
  __syncthreads();
  int run = 0;
  for (int s2 = 0; s2 < seg; ++s2) run += part[s2][bl];
  if (ok && seg == kPrefixSegs - 1) counts[bucket] = run + sum;
  if (ok)
    for (int c = c0; c < c1; c += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) v[k] = col[(size_t)min(c + k, c1 - 1) * m];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (c + k < c1) {
          col[(size_t)(c + k) * m] = run;
          run += v[k];
        }
    }
}

__global__ __launch_bounds__(64) void scatter_stable_kernel(
    const int* __restrict__ node, const int* __restrict__ offsets, const int* __restrict__ wgc,
    int* __restrict__ pairs, int* __restrict__ inv, int n_tok, int topk, int m) {
  extern __shared__ int base[];  // [m] next position of each node's pairs, then
                                 // [m / 4] byte counters of the current step
  unsigned* cnt4 = reinterpret_cast<unsigned*>(base + m);
  const int bh = blockIdx.y;
  const int* pre = wgc + ((size_t)bh * gridDim.x + blockIdx.x) * m;
  for (int i = threadIdx.x; i < m; i += blockDim.x) base[i] = offsets[(size_t)bh * m + i] + pre[i];
  for (int i = threadIdx.x; i < (m + 3) / 4; i += blockDim.x) cnt4[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * kStableRows, t1 = min(t0 + kStableRows, n_tok);
  const size_t row0 = (size_t)bh * n_tok;
  const int* src = node + row0 * topk;
  const int i1 = t1 * topk;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  // Steps of 64 slots, S at a time: their node loads are issued together and
  // their stores after the last of them (loads and stores share one counter,
  // so a store between two steps would hold up the next step's load).
  constexpr int S = 8;
  for (int ib0 = t0 * topk; ib0 < i1; ib0 += S * 64) {
    int xs[S], ps[S];
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int i = ib0 + u * 64 + lane;
      xs[u] = i < i1 ? src[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int x = xs[u];
      const bool live = x >= 0 && x < m;
      const int xc = live ? x : 0;
      const unsigned one = 1u << (8 * (xc & 3));
      // How many of the step's lanes hold x (order-free LDS adds); lanes
      // whose node is unique take rank 0 without the ranking loop below.
      if (live) atomicAdd(&cnt4[xc >> 2], one);
      wave_lds_sync();
      const int c = live ? (int)((cnt4[xc >> 2] >> (8 * (xc & 3))) & 0xffu) : 0;
      wave_lds_sync();
      if (live) atomicSub(&cnt4[xc >> 2], one);
      int rank = 0, cnt = c;
      uint64_t pending = __ballot(c > 1);  // lanes ranked by lane among equal nodes
      while (pending) {
        const int v = __builtin_amdgcn_readlane(x, (int)__builtin_ctzll(pending));
        const uint64_t same = __ballot(live && x == v);
        if (live && x == v) rank = __popcll(same & below);
        pending &= ~same;
      }
      const int b = base[xc];
      ps[u] = live ? b + rank : -1;
      wave_lds_sync();  // every lane has read base[] before the leaders move it
      if (live && rank == 0) base[x] += cnt;
      wave_lds_sync();
    }
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int i = ib0 + u * 64 + lane;
      if (ps[u] >= 0) {
        pairs[ps[u]] = (int)(((row0 + i / topk) << 5) | (i % topk));
        if (inv) inv[row0 * topk + i] = ps[u];
      }
    }
  }
}

}  // namespace

// Work item -> (bucket, first pair, pair count) from the scan's offsets.
// Called by every lane of a wave with the same item (the kernels call it
// first thing, with all lanes active).  The bucket is the largest b with
// item_offsets[b] <= item, found by a 64-way search: each round the wave's
// lanes probe 64 evenly spaced entries at once, so 2^18 buckets take three
// rounds of parallel loads instead of eighteen dependent ones.
__device__ __forceinline__ bool locate_item(const int* __restrict__ item_offsets,
                                            const int* __restrict__ offsets, int n_buckets,
                                            int item, int per_item, int* bucket, int* start,
                                            int* len) {
  if (item >= item_offsets[n_buckets]) return false;
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n_buckets;  // item_offsets[lo] <= item; answer in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) >> 6;
    const int probe = lo + lane * step;
    const bool ok = probe < hi && item_offsets[probe] <= item;
    const uint64_t m = __ballot(ok);  // a prefix of the lanes (item_offsets is sorted)
    const int last = 63 - __builtin_clzll(m);
    lo += last * step;
    hi = min(hi, lo + step);
  }
  const int k = item - item_offsets[lo];
  *bucket = lo;
  *start = offsets[lo] + k * per_item;
  *len = min(per_item, offsets[lo + 1] - *start);
  return true;
}

inline unsigned grid_for(size_t n, unsigned threads = 256, unsigned cap = 65536) {
  const size_t g = (n + threads - 1) / threads;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

// Zero counters, count, scan and scatter the live slots of node[] (one head =
// n_tok rows of topk slots).  Work items of per_item pairs are located with
// locate_item.  inv (nullable) receives each live pair's position in pairs[].
inline hipError_t sort_pairs(const int* node, int batch_heads, int n_tok, int topk, int m,
                             int per_item, int* counts, int* offsets, int* cursors,
                             int* item_offsets, int* pairs, int* inv, bool counts_ready,
                             hipStream_t st) {
  const int n_buckets = batch_heads * m;
  const size_t n_slots = (size_t)batch_heads * n_tok * topk;
  // Rows per count/scatter workgroup: fewer, larger workgroups place their
  // pairs with fewer global counter updates, as long as the grid still has a
  // few hundred of them.
  int rpg = kRowsPerGroup;
  while (rpg < kMaxRowsPerGroup &&
         (size_t)((n_tok + 2 * rpg - 1) / (2 * rpg)) * batch_heads >= 256)
    rpg *= 2;
  const dim3 grid((n_tok + rpg - 1) / rpg, batch_heads);
  const bool local = m <= kMaxLocalBuckets;
  if (!counts_ready) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n_buckets)), dim3(256), 0, st, counts,
                       n_buckets);
    if (local)
      hipLaunchKernelGGL(count_kernel, grid, dim3(kSortThreads), sizeof(int) * m, st, node, counts, n_tok,
                         topk, m, rpg);
    else
      hipLaunchKernelGGL(count_global_kernel, dim3(grid_for(n_slots)), dim3(256), 0, st, node,
                         counts, n_tok, topk, m, n_slots);
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), scan_lds_bytes(n_buckets), st, counts,
                     offsets, cursors, item_offsets, n_buckets, per_item);
  if (local)
    hipLaunchKernelGGL(scatter_kernel, grid, dim3(kSortThreads), 2 * sizeof(int) * m, st, node, cursors,
                       pairs, inv, n_tok, topk, m, rpg);
  else
    hipLaunchKernelGGL(scatter_global_kernel, dim3(grid_for(n_slots)), dim3(256), 0, st, node,
                       cursors, pairs, inv, n_tok, topk, m, n_slots);
  return hipGetLastError();
}

// Row chunks of the stable sort, and its per-chunk count matrix (ints).
inline int row_chunks(int n_tok) { return (n_tok + kStableRows - 1) / kStableRows; }
inline size_t stable_wgc_ints(int batch_heads, int n_tok, int m) {
  return (size_t)batch_heads * row_chunks(n_tok) * m;
}

// sort_pairs with each bucket in increasing (row, slot) order (m <=
// kMaxLocalBuckets; callers check).  wgc: stable_wgc_ints(...) ints.
inline hipError_t sort_pairs_stable(const int* node, int batch_heads, int n_tok, int topk, int m,
                                    int per_item, int* counts, int* offsets, int* cursors,
                                    int* item_offsets, int* wgc, int* pairs, int* inv,
                                    hipStream_t st) {
  const int n_buckets = batch_heads * m;
  const dim3 grid(row_chunks(n_tok), batch_heads);
  hipLaunchKernelGGL(count_wg_kernel, grid, dim3(256), sizeof(int) * m, st, node, wgc, n_tok, topk,
                     m);
  hipLaunchKernelGGL(wg_prefix_kernel, dim3((n_buckets + kPrefixBuckets - 1) / kPrefixBuckets),
                     dim3(256), 0, st, wgc, counts, (int)grid.x, m, n_buckets);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), scan_lds_bytes(n_buckets), st, counts,
                     offsets, cursors, item_offsets, n_buckets, per_item);
  hipLaunchKernelGGL(scatter_stable_kernel, grid, dim3(64), sizeof(int) * (m + (m + 3) / 4), st,
                     node, offsets, wgc, pairs, inv, n_tok, topk, m);
  return hipGetLastError();
}

// Upper bound of the number of work items (for grid sizing).
inline int max_items(size_t n_slots, int n_buckets, int per_item) {
  return (int)((n_slots + per_item - 1) / per_item) + n_buckets;
}

}  // namespace bucket
}  // namespace pisa
