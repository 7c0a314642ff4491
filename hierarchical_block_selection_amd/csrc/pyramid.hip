// Key pyramid: PISA reading page §4.1, eqs. (3) and (4).
//
// Level 1 row i is the mean of keys [iC, min((i+1)C, N)); level l+1 row i is
// the mean of the existing level-l rows {2i, 2i+1}.  HBM-bound: K is read once
// (N*d*sizeof(T) bytes per KV head) and R*d*4 bytes of summaries are written.
//
// Pass 1 (chunk kernel): one workgroup of 8 waves per (KV head, aligned
// chunk of 2^j = 16 leaves), two workgroups per CU.  Each wave streams whole
// leaf blocks with 16-byte loads (a row is spread over d*sizeof(T)/16 lanes,
// several rows per load), reduces the rows across lanes, then the workgroup
// builds levels 2..j+1 of its chunk in LDS.  Pass 2 (top kernel): one
// workgroup of 1024 threads per KV head builds levels j+2..L from level j+1
// (M_1/16 rows): the first of them with float4 loads, four outputs' worth
// requested per thread at once, the rest in LDS when they fit.
#include "pisa_common.h"
#include "pisa_launch.h"

namespace pisa {

constexpr int kPyrThreads = 512;
constexpr int kPyrLeavesLog2 = 4;  // 16 leaf blocks per chunk workgroup
constexpr int kTopThreads = 1024;
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

// Levels first_level..L.  The first of them is built from global memory
// with every thread's loads of a batch requested together (src and dst share
// the pyramid buffer, so a plain loop would wait on each load in turn); the
// rest ping-pong in LDS (dynamic, two buffers) when use_lds is set.
template <int D>
__global__ __launch_bounds__(kTopThreads) void pyramid_top_kernel(float* __restrict__ pyr,
                                                                   LevelTable lv, int first_level,
                                                                   int use_lds) {
  extern __shared__ float top_lds[];
  constexpr int D4 = D / 4;
  constexpr int NB = 4;  // float4 outputs per thread per batch
  float* pb = pyr + (size_t)blockIdx.x * lv.rows * D;
  float* bufs[2] = {top_lds, top_lds + (size_t)lv.size[first_level - 1] * D};
  {
    const int l = first_level;
    const int m_prev = lv.size[l - 2], m_cur = lv.size[l - 1];
    const float4* src = reinterpret_cast<const float4*>(pb + (size_t)lv.off[l - 2] * D);
    float4* dst = reinterpret_cast<float4*>(pb + (size_t)lv.off[l - 1] * D);
    float4* ldst = reinterpret_cast<float4*>(bufs[0]);
    const int total = m_cur * D4;
    for (int x0 = threadIdx.x; x0 < total; x0 += NB * kTopThreads) {
      float4 a[NB], b[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int x = min(x0 + k * kTopThreads, total - 1);
        const int node = x / D4, c4 = x % D4;
        a[k] = src[(size_t)(2 * node) * D4 + c4];
        b[k] = src[(size_t)min(2 * node + 1, m_prev - 1) * D4 + c4];
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int x = x0 + k * kTopThreads;
        if (x >= total) break;
        const int node = x / D4;
        float4 v = a[k];
        if (2 * node + 1 < m_prev) {
          v.x = 0.5f * (v.x + b[k].x);
          v.y = 0.5f * (v.y + b[k].y);
          v.z = 0.5f * (v.z + b[k].z);
          v.w = 0.5f * (v.w + b[k].w);
        }
        dst[x] = v;
        if (use_lds) ldst[x] = v;
      }
    }
    __syncthreads();
  }
  for (int l = first_level + 1; l <= lv.n; ++l) {
    const int m_prev = lv.size[l - 2], m_cur = lv.size[l - 1];
    const float* src = use_lds ? bufs[(l - first_level - 1) & 1] : pb + (size_t)lv.off[l - 2] * D;
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

// Pyramid cache upkeep for decode (PISA reading page §5.3, decode cache): the
// key of token t = cache_len - 1 has just been written to the cache; the
// nodes on t's path (leaf t / C and its ancestors) become those of the
// pyramid over exactly t + 1 tokens.  One wavefront per (sequence, KV head).
// The leaf mean uses the chunk kernel's lane mapping and summation order and
// every level the same (left + right) / 2, so the rows written are bit for
// bit those pisa_build_pyramid writes over t + 1 tokens; rows off the path
// are not touched.  The complete left siblings on the path are read into LDS
// before the levels are folded.
constexpr int kAppendWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(kAppendWaves * kWave) void pyramid_append_kernel(
    const int32_t* __restrict__ cache_len, const T* __restrict__ kc, float* __restrict__ pyr,
    int heads_kv, int capacity, int block, LevelTable lv, int n_units) {
  constexpr int VEC = Vec16<T>::n;
  constexpr int LPR = D / VEC;      // lanes per key row
  constexpr int RPI = kWave / LPR;  // key rows per load instruction
  __shared__ float sib_s[kAppendWaves][PISA_MAX_LEVELS][D];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int unit = blockIdx.x * kAppendWaves + wave;  // b * heads_kv + kvh
  if (unit >= n_units) return;
  const int n = cache_len[unit / heads_kv];
  if (n < 1 || n > capacity) return;
  const int t = n - 1, c = t / block;
  const int r0 = c * block, r1 = t + 1;
  const T* kb = kc + (size_t)unit * capacity * D;
  float* pb = pyr + (size_t)unit * lv.rows * D;
  // Left siblings of the path (node at level l - 1 odd): all lanes, to LDS.
  for (int l = 2; l <= lv.n; ++l) {
    const int node = c >> (l - 2);
    if (node & 1) {
      const float* src = pb + (size_t)(lv.off[l - 2] + node - 1) * D;
      for (int x = lane; x < D; x += kWave) sib_s[wave][l - 1][x] = src[x];
    }
  }
  // Leaf mean: rows r0 + sub, r0 + sub + RPI, ... added in order; 16 loads
  // are requested before the first is added.
  const int sub = lane / LPR, col = (lane % LPR) * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int rb = r0 + sub; rb < r1; rb += 16 * RPI) {
    uint4 raw[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      raw[k] = *reinterpret_cast<const uint4*>(kb + (size_t)min(rb + k * RPI, r1 - 1) * D + col);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (rb + k * RPI >= r1) break;
      float v[VEC];
      if constexpr (VEC == 8) {
        const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        v[0] = __uint_as_float(raw[k].x);
        v[1] = __uint_as_float(raw[k].y);
        v[2] = __uint_as_float(raw[k].z);
        v[3] = __uint_as_float(raw[k].w);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += v[e];
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  wave_lds_sync();
  if (sub != 0) return;  // lanes 0 .. LPR - 1 carry the path
  const float inv = 1.f / float(r1 - r0);
  float v[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) v[e] = acc[e] * inv;
  auto store = [&](int level_index, int node) {
    float* dst = pb + (size_t)(lv.off[level_index] + node) * D + col;
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
  };
  store(0, c);
  for (int l = 2; l <= lv.n; ++l) {
    const int node = c >> (l - 2);  // path node one level down (the last there)
    if (node & 1) {  // its left sibling exists: mean of both
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = 0.5f * (sib_s[wave][l - 1][col + e] + v[e]);
    }  // else it has no right sibling yet: the parent equals it
    store(l - 1, node >> 1);
  }
}

template <typename T, int D>
static hipError_t launch_append_t(const LaunchShape& s, const int32_t* cache_len, const void* kc,
                                  float* pyr, hipStream_t st) {
  const int units = s.batch * s.heads_kv;
  prof::Scope ps("pyramid_append", st);
  hipLaunchKernelGGL((pyramid_append_kernel<T, D>),
                     dim3((units + kAppendWaves - 1) / kAppendWaves), dim3(kAppendWaves * kWave),
                     0, st, cache_len, static_cast<const T*>(kc), pyr, s.heads_kv, s.seq_len,
                     s.block, s.lv, units);
  return hipGetLastError();
}

hipError_t launch_pyramid_append(const LaunchShape& s, const int32_t* cache_len, const void* kc,
                                 float* pyr, hipStream_t st) {
  if (s.bf16) {
    return s.head_dim == 128 ? launch_append_t<bf16_t, 128>(s, cache_len, kc, pyr, st)
                             : launch_append_t<bf16_t, 64>(s, cache_len, kc, pyr, st);
  }
  return s.head_dim == 128 ? launch_append_t<float, 128>(s, cache_len, kc, pyr, st)
                           : launch_append_t<float, 64>(s, cache_len, kc, pyr, st);
}

}  // namespace pisa
