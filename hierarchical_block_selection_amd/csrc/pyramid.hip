// Key pyramid: PISA reading page §4.1, eqs. (3) and (4).
//
// Level 1 row i is the mean of keys [iC, min((i+1)C, N)); level l+1 row i is
// the mean of the existing level-l rows {2i, 2i+1}.  HBM-bound: K is read once
// (N*d*sizeof(T) bytes per KV head) and R*d*4 bytes of summaries are written.
//
// Pass 1 (chunk kernel): one workgroup of 16 waves per (KV head, aligned
// chunk of 2^j = 32 leaves).  Each wave streams whole leaf blocks with 16-byte
// loads (a row is spread over d*sizeof(T)/16 lanes, several rows per load),
// reduces the rows across lanes, then the workgroup builds levels 2..j+1 of its
// chunk in LDS.  Pass 2 (top kernel): one workgroup per KV head builds levels
// j+2..L from level j+1 (M_1/32 rows), keeping every level after the first in
// LDS when it fits.
#include "pisa_common.h"
#include "pisa_launch.h"

namespace pisa {

constexpr int kPyrThreads = 1024;
constexpr int kPyrLeavesLog2 = 5;  // 32 leaf blocks per chunk workgroup
constexpr int kTopThreads = 256;
constexpr size_t kTopLds = 64 * 1024;

template <typename T, int D>
__global__ __launch_bounds__(kPyrThreads) void pyramid_chunk_kernel(
    const T* __restrict__ keys, float* __restrict__ pyr, int n_tok, int block, LevelTable lv) {
  constexpr int LPC = 1 << kPyrLeavesLog2;
  constexpr int VEC = Vec16<T>::n;
  constexpr int LPR = D / VEC;       // lanes per key row
  constexpr int RPI = kWave / LPR;   // key rows per load instruction
  __shared__ float buf[2][LPC * D];

  const int bh = blockIdx.y;
  const int leaf0 = blockIdx.x * LPC;
  const T* kb = keys + (size_t)bh * n_tok * D;
  float* pb = pyr + (size_t)bh * lv.rows * D;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int m1 = lv.size[0];

  // Level 1: one leaf block per wave iteration.
  for (int li = wave; li < LPC; li += kPyrThreads / kWave) {
    const int leaf = leaf0 + li;
    if (leaf >= m1) break;
    const int r0 = leaf * block, r1 = min(r0 + block, n_tok);
    const int sub = lane / LPR, col = (lane % LPR) * VEC;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll 8
    for (int r = r0 + sub; r < r1; r += RPI) {
      float v[VEC];
      load16(kb + (size_t)r * D + col, v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
    if (sub == 0) {
      const float inv = 1.f / float(r1 - r0);
      float* dst = pb + (size_t)(lv.off[0] + leaf) * D + col;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        float4 m = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
        *reinterpret_cast<float4*>(dst + e) = m;
        *reinterpret_cast<float4*>(&buf[0][li * D + col + e]) = m;
      }
    }
  }
  __syncthreads();

  // Levels 2..j+1 inside the chunk, ping-ponging between the two LDS buffers.
  const int top = min(lv.n, 1 + kPyrLeavesLog2);
  for (int l = 2; l <= top; ++l) {
    const float* src = buf[(l - 2) & 1];
    float* dst = buf[(l - 1) & 1];
    const int m_prev = lv.size[l - 2], m_cur = lv.size[l - 1];
    const int first = leaf0 >> (l - 1), first_prev = leaf0 >> (l - 2);
    const int here = min(LPC >> (l - 1), m_cur - first);
    for (int x = threadIdx.x; x < here * D; x += kPyrThreads) {
      const int node = x / D, col = x % D;
      const int g = first + node;
      const int c0 = 2 * g - first_prev;
      float v = src[c0 * D + col];
      if (2 * g + 1 < m_prev) v = 0.5f * (v + src[(c0 + 1) * D + col]);
      dst[node * D + col] = v;
      pb[(size_t)(lv.off[l - 1] + g) * D + col] = v;
    }
    __syncthreads();
  }
}

// Levels first_level..L.  The first of them is read from global memory; the
// rest ping-pong in LDS (dynamic, two buffers) when use_lds is set.
template <int D>
__global__ __launch_bounds__(kTopThreads) void pyramid_top_kernel(float* __restrict__ pyr,
                                                                   LevelTable lv, int first_level,
                                                                   int use_lds) {
  extern __shared__ float top_lds[];
  float* pb = pyr + (size_t)blockIdx.x * lv.rows * D;
  float* bufs[2] = {top_lds, top_lds + (size_t)lv.size[first_level - 1] * D};
  for (int l = first_level; l <= lv.n; ++l) {
    const int m_prev = lv.size[l - 2], m_cur = lv.size[l - 1];
    const bool from_lds = use_lds && l > first_level;
    const float* src = from_lds ? bufs[(l - first_level - 1) & 1] : pb + (size_t)lv.off[l - 2] * D;
    float* ldst = bufs[(l - first_level) & 1];
    float* dst = pb + (size_t)lv.off[l - 1] * D;
    for (int x = threadIdx.x; x < m_cur * D; x += kTopThreads) {
      const int node = x / D, col = x % D;
      float v = src[(size_t)(2 * node) * D + col];
      if (2 * node + 1 < m_prev) v = 0.5f * (v + src[(size_t)(2 * node + 1) * D + col]);
      dst[(size_t)node * D + col] = v;
      if (use_lds) ldst[(size_t)node * D + col] = v;
    }
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t launch_pyramid_t(const LaunchShape& s, const void* k, float* pyr,
                                   hipStream_t st) {
  const int chunks = (s.lv.size[0] + (1 << kPyrLeavesLog2) - 1) >> kPyrLeavesLog2;
  dim3 grid(chunks, s.batch * s.heads_kv);
  {
    prof::Scope ps("pyramid_chunk", st);
    hipLaunchKernelGGL((pyramid_chunk_kernel<T, D>), grid, dim3(kPyrThreads), 0, st,
                       static_cast<const T*>(k), pyr, s.seq_len, s.block, s.lv);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int first = 2 + kPyrLeavesLog2;
  if (s.lv.n >= first) {
    const size_t lds = (size_t)(s.lv.size[first - 1] + (s.lv.n > first ? s.lv.size[first] : 0)) *
                       D * sizeof(float);
    const bool use_lds = lds <= kTopLds;
    prof::Scope ps("pyramid_top", st);
    hipLaunchKernelGGL((pyramid_top_kernel<D>), dim3(s.batch * s.heads_kv), dim3(kTopThreads),
                       use_lds ? lds : 0, st, pyr, s.lv, first, use_lds ? 1 : 0);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_pyramid(const LaunchShape& s, const void* k, float* pyr, hipStream_t st) {
  if (s.bf16) {
    return s.head_dim == 128 ? launch_pyramid_t<bf16_t, 128>(s, k, pyr, st)
                             : launch_pyramid_t<bf16_t, 64>(s, k, pyr, st);
  }
  return s.head_dim == 128 ? launch_pyramid_t<float, 128>(s, k, pyr, st)
                           : launch_pyramid_t<float, 64>(s, k, pyr, st);
}

}  // namespace pisa
