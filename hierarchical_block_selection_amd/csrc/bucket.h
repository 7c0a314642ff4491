// Counting sort of (row, slot) pairs into per-node buckets, used wherever a
// block of keys is loaded once and applied to every query that needs it.
//
// Input: node[u * K + slot] >= 0 for live pairs (-1 otherwise), where row u
// belongs to head bh = u / n_tok; the pair's bucket is bh * m + node.
//   count:   histogram of buckets (atomic adds on zeroed counters);
//   scan:    one workgroup: exclusive bucket offsets, scatter cursors and a
//            work list of (bucket, first pair, pair count <= per_item);
//   scatter: pair ids u * K + slot into their buckets (order inside a bucket
//            follows the atomics; consumers must not depend on it).
#pragma once

#include "pisa_common.h"

namespace pisa {
namespace bucket {
namespace {  // each translation unit keeps its own copy of these kernels

__global__ void fill_zero_kernel(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void count_kernel(const int* __restrict__ node, int* __restrict__ counts, int n_tok,
                             int topk, int m, size_t n_slots) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots;
       i += (size_t)gridDim.x * blockDim.x) {
    const int x = node[i];
    if (x < 0 || x >= m) continue;
    const size_t bh = i / topk / n_tok;
    atomicAdd(&counts[bh * m + x], 1);
  }
}

__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ cursors,
                                                    int* __restrict__ items,
                                                    int* __restrict__ n_items, int n_buckets,
                                                    int max_items, int per_item) {
  __shared__ int part_pairs[1024];
  __shared__ int part_items[1024];
  const int tid = threadIdx.x;
  const int per = (n_buckets + 1023) / 1024;
  const int lo = min(tid * per, n_buckets), hi = min(lo + per, n_buckets);
  int sp = 0, si = 0;
  for (int i = lo; i < hi; ++i) {
    sp += counts[i];
    si += (counts[i] + per_item - 1) / per_item;
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
    for (int s = 0; s < c; s += per_item) {
      if (ipos < max_items) {
        items[3 * ipos] = i;
        items[3 * ipos + 1] = pos + s;
        items[3 * ipos + 2] = min(per_item, c - s);
      }
      ++ipos;
    }
    pos += c;
  }
  if (tid == 1023) {
    offsets[n_buckets] = part_pairs[1023];
    *n_items = min(part_items[1023], max_items);
  }
}

__global__ void scatter_kernel(const int* __restrict__ node, int* __restrict__ cursors,
                               int* __restrict__ pairs, int n_tok, int topk, int m,
                               size_t n_slots) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots;
       i += (size_t)gridDim.x * blockDim.x) {
    const int x = node[i];
    if (x < 0 || x >= m) continue;
    const size_t bh = i / topk / n_tok;
    const int pos = atomicAdd(&cursors[bh * m + x], 1);
    pairs[pos] = (int)i;  // u * K + slot
  }
}

inline unsigned grid_for(size_t n, unsigned threads = 256, unsigned cap = 65536) {
  const size_t g = (n + threads - 1) / threads;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace
}  // namespace bucket
}  // namespace pisa
