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

constexpr int kRowsPerGroup = 512;    // rows of one head per count/scatter workgroup
constexpr int kMaxLocalBuckets = 8192;  // LDS histogram limit (two int arrays = 64 KB)
constexpr int kBatch = 16;  // slots per thread whose loads are issued together

namespace {  // each translation unit keeps its own copy of these kernels

__global__ void fill_zero_kernel(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ __launch_bounds__(256) void count_kernel(const int* __restrict__ node,
                                                    int* __restrict__ counts, int n_tok, int topk,
                                                    int m) {
  extern __shared__ int hist[];  // [m]
  for (int i = threadIdx.x; i < m; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * kRowsPerGroup, t1 = min(t0 + kRowsPerGroup, n_tok);
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

__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ cursors,
                                                    int* __restrict__ item_offsets, int n_buckets,
                                                    int per_item) {
  __shared__ int part_pairs[1024];
  __shared__ int part_items[1024];
  const int tid = threadIdx.x;
  const int per = (n_buckets + 1023) / 1024;
  const int lo = min(tid * per, n_buckets), hi = min(lo + per, n_buckets);
  int sp = 0, si = 0;
  for (int i0 = lo; i0 < hi; i0 += 8) {  // 8 loads in flight
    int c8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c8[k] = counts[min(i0 + k, hi - 1)];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (i0 + k < hi) {
        sp += c8[k];
        si += (c8[k] + per_item - 1) / per_item;
      }
  }
  part_pairs[tid] = sp;
  part_items[tid] = si;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = tid >= o ? part_pairs[tid - o] : 0;
    const int c = tid >= o ? part_items[tid - o] : 0;
    __syncthreads();
    part_pairs[tid] += a;
    part_items[tid] += c;
    __syncthreads();
  }
  int pos = tid ? part_pairs[tid - 1] : 0;
  int ipos = tid ? part_items[tid - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    const int c = counts[i];
    offsets[i] = pos;
    cursors[i] = pos;
    item_offsets[i] = ipos;
    pos += c;
    ipos += (c + per_item - 1) / per_item;
  }
  if (tid == 1023) {
    offsets[n_buckets] = part_pairs[1023];
    item_offsets[n_buckets] = part_items[1023];
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ node,
                                                      int* __restrict__ cursors,
                                                      int* __restrict__ pairs,
                                                      int* __restrict__ inv, int n_tok, int topk,
                                                      int m) {
  extern __shared__ int lds[];  // hist/base [m], local cursor [m]
  int* base = lds;
  int* cur = lds + m;
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    base[i] = 0;
    cur[i] = 0;
  }
  __syncthreads();
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * kRowsPerGroup, t1 = min(t0 + kRowsPerGroup, n_tok);
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

}  // namespace

// Work item -> (bucket, first pair, pair count) from the scan's offsets.
__device__ __forceinline__ bool locate_item(const int* __restrict__ item_offsets,
                                            const int* __restrict__ offsets, int n_buckets,
                                            int item, int per_item, int* bucket, int* start,
                                            int* len) {
  if (item >= item_offsets[n_buckets]) return false;
  int lo = 0, hi = n_buckets - 1;  // largest bucket with item_offsets[b] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (item_offsets[mid] <= item) lo = mid; else hi = mid - 1;
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
  const dim3 grid((n_tok + kRowsPerGroup - 1) / kRowsPerGroup, batch_heads);
  const bool local = m <= kMaxLocalBuckets;
  if (!counts_ready) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n_buckets)), dim3(256), 0, st, counts,
                       n_buckets);
    if (local)
      hipLaunchKernelGGL(count_kernel, grid, dim3(256), sizeof(int) * m, st, node, counts, n_tok,
                         topk, m);
    else
      hipLaunchKernelGGL(count_global_kernel, dim3(grid_for(n_slots)), dim3(256), 0, st, node,
                         counts, n_tok, topk, m, n_slots);
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, offsets, cursors,
                     item_offsets, n_buckets, per_item);
  if (local)
    hipLaunchKernelGGL(scatter_kernel, grid, dim3(256), 2 * sizeof(int) * m, st, node, cursors,
                       pairs, inv, n_tok, topk, m);
  else
    hipLaunchKernelGGL(scatter_global_kernel, dim3(grid_for(n_slots)), dim3(256), 0, st, node,
                       cursors, pairs, inv, n_tok, topk, m, n_slots);
  return hipGetLastError();
}

// Upper bound of the number of work items (for grid sizing).
inline int max_items(size_t n_slots, int n_buckets, int per_item) {
  return (int)((n_slots + per_item - 1) / per_item) + n_buckets;
}

}  // namespace bucket
}  // namespace pisa
