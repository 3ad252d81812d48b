// Routing kernels: wavefront top-K + softmax with per-chunk expert histograms,
// the expert offset scan (+ grouped-GEMM tile list), the stable scatter into
// expert-sorted slots, and the deterministic gather-reduce combine.
//
// Top-K selection and the softmax over the selected logits follow the routed
// MoE of the pages (K of N experts per token: 6 of 128 in the Nemotron 3 Nano
// blog's granular MoE section, 22 of 512 in the Ultra release news); the gate
// function, the tie rule and the dropless policy are readings (see moe.h).
#include "common.h"

namespace moe {

// Orderable key: larger logit first, then lower expert id.  Invalid lanes are 0.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t e) {
  if (v == 0.0f) v = 0.0f;                                 // -0 ties with +0
  uint32_t u = __float_as_uint(v);
  u ^= (u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u ^= (u & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint32_t key_expert(uint64_t k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu);
}
// Zero `n` ints (the chunk histograms) with plain stores: safe inside captured graphs.
__global__ __launch_bounds__(256) void zero_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Wave-wide max of a 32-bit value: the same four DPP steps leave each lane
// with its row's max, then the four row maxima are combined as scalars.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1>(v);
  v = dpp_max_u32<0x4E>(v);
  v = dpp_max_u32<0x124>(v);
  v = dpp_max_u32<0x128>(v);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// a where the lane's bit of `lanes` is clear, b where it is set (one
// v_cndmask with a scalar lane mask; written out so that the per-round pop
// below stays a plain shift instead of an indexed select over all keys)
__device__ __forceinline__ uint32_t sel_lanes(uint32_t a, uint32_t b, uint64_t lanes) {
  uint32_t d;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(lanes));
  return d;
}

// Descending bitonic sorting network over a lane's NJ keys (NJ a power of 2).
template <int NJ>
__device__ __forceinline__ void sort_keys_desc(uint64_t (&k)[NJ]) {
#pragma unroll
  for (int size = 2; size <= NJ; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < NJ; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t a = k[i], b = k[j];
          const bool sw = ((i & size) == 0) ? a < b : a > b;
          k[i] = sw ? b : a;
          k[j] = sw ? a : b;
        }
      }
}

// One wavefront per token (4 per block).  Each lane holds the keys (value,
// then lower expert id first; see make_key) of experts lane, lane+64, ...,
// sorted descending, so its best remaining key is always key[0].  Each of the
// K rounds takes the wave-wide max of the lanes' best values, breaks a tie in
// value by the key's id half (a second max, only when several lanes hold the
// value), and pops the winning lane's key: the K largest keys in descending
// order.  The per-chunk expert histogram of chunk t / tc is kept with integer
// atomics (order-independent results).
template <int NJ>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int N,
                                                   int K, int tc, int* __restrict__ idx,
                                                   float* __restrict__ gate,
                                                   int* __restrict__ chunk_counts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // all NJ loads go out before any is used (lanes past N re-read the row's
  // last logit and get the invalid key 0, below every valid key)
  const float* row = logits + (int64_t)t * N;
  float lv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) lv[j] = row[min(j * 64 + lane, N - 1)];
#pragma unroll
  for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(lv[j]));  // keeps the loads together
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * 64 + lane;
    key[j] = e < N ? make_key(lv[j], (uint32_t)e) : 0ull;
  }
  sort_keys_desc<NJ>(key);
  uint32_t khi[NJ], klo[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    khi[j] = (uint32_t)(key[j] >> 32);
    klo[j] = (uint32_t)key[j];
  }
  uint64_t mine = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t hi = khi[0], lo = klo[0];
    const uint32_t mhi = wave_max_u32(hi);
    uint64_t at = __ballot(hi == mhi);             // lanes whose best value is the max
    uint32_t mlo;
    if (__popcll(at) == 1) {
      mlo = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((unsigned long long)at) - 1);
    } else {                                       // equal values: the larger id half wins
      mlo = wave_max_u32(hi == mhi ? lo : 0u);
      at = __ballot(hi == mhi && lo == mlo);
    }
    // pop the winning lane's best key (a one-bit lane mask)
    const uint64_t wm = 1ull << (__ffsll((unsigned long long)at) - 1);
#pragma unroll
    for (int j = 0; j + 1 < NJ; ++j) {
      khi[j] = sel_lanes(khi[j], khi[j + 1], wm);
      klo[j] = sel_lanes(klo[j], klo[j + 1], wm);
    }
    khi[NJ - 1] = sel_lanes(khi[NJ - 1], 0u, wm);
    klo[NJ - 1] = sel_lanes(klo[NJ - 1], 0u, wm);
    if (lane == k) mine = ((uint64_t)mhi << 32) | mlo;
  }
  const float v = key_value(mine);
  const float vmax = __shfl(v, 0, 64);
  float ex = lane < K ? expf(v - vmax) : 0.0f;
  float s = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane < K) {
    const uint32_t e = key_expert(mine);
    idx[(int64_t)t * K + lane] = (int)e;
    gate[(int64_t)t * K + lane] = ex / s;
    atomicAdd(&chunk_counts[(int64_t)(t / tc) * N + e], 1);
  }
}

hipError_t launch_topk(const float* logits, int T, int N, int K, int tc, int* idx, float* gate,
                       int* chunk_counts, hipStream_t s) {
  const int nchunks = (T + tc - 1) / tc;
  const int nz = nchunks * N;
  hipLaunchKernelGGL(zero_kernel, dim3((nz + 255) / 256), dim3(256), 0, s, chunk_counts, nz);
  dim3 g((T + 3) / 4), b(256);
  if (N <= 64) hipLaunchKernelGGL(topk_kernel<1>, g, b, 0, s, logits, T, N, K, tc, idx, gate, chunk_counts);
  else if (N <= 128) hipLaunchKernelGGL(topk_kernel<2>, g, b, 0, s, logits, T, N, K, tc, idx, gate, chunk_counts);
  else if (N <= 256) hipLaunchKernelGGL(topk_kernel<4>, g, b, 0, s, logits, T, N, K, tc, idx, gate, chunk_counts);
  else if (N <= 512) hipLaunchKernelGGL(topk_kernel<8>, g, b, 0, s, logits, T, N, K, tc, idx, gate, chunk_counts);
  else hipLaunchKernelGGL(topk_kernel<16>, g, b, 0, s, logits, T, N, K, tc, idx, gate, chunk_counts);
  return hipGetLastError();
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_excl_scan_1024(int v, int* total_out) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(x, off, 64);
    if (lane >= off) x += o;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  __syncthreads();
  *total_out = tot;
  return base + x - v;
}

// Per-expert exclusive prefix over many chunks, spread over ceil(N / 64)
// blocks: block b takes experts 64b .. 64b + 63 (one per lane) and its 16
// wavefronts split the chunks into 16 consecutive ranges.  Each wavefront sums
// its range, the ranges' sums are combined in LDS, then each wavefront re-reads
// its range (now L2-resident) and writes chunk_base.  counts[e] receives the
// expert's total.
__global__ __launch_bounds__(1024) void chunk_prefix_kernel(const int* __restrict__ chunk_counts,
                                                            int nchunks, int N,
                                                            int* __restrict__ chunk_base,
                                                            int* __restrict__ counts) {
  __shared__ int part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int ec = min(e, N - 1);                   // lanes past N read a valid column, write nothing
  const int per = (nchunks + 15) / 16;
  const int c0 = min(nchunks, w * per), c1 = min(nchunks, c0 + per);
  int sum = 0;
  for (int c = c0; c < c1; c += 16) {             // 16 independent loads in flight
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {              // rows past c1 re-read row c1 - 1, value unused
      const int x = chunk_counts[(int64_t)min(c + i, c1 - 1) * N + ec];
      v[i] = c + i < c1 ? x : 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += v[i];
  }
  part[w][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int u = 0; u < w; ++u) run += part[u][lane];
  for (int c = c0; c < c1; c += 16) {
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {              // rows past c1 re-read row c1 - 1, value unused
      const int x = chunk_counts[(int64_t)min(c + i, c1 - 1) * N + ec];
      v[i] = c + i < c1 ? x : 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (c + i < c1 && e < N) chunk_base[(int64_t)(c + i) * N + e] = run;
      run += v[i];
    }
  }
  if (w == 15 && e < N) counts[e] = run;          // the sum of all 16 ranges
}

// Single block: per-expert totals over chunks (chunk_base = exclusive prefix
// over chunks; or, with nchunks == 0, the totals already in counts), expert
// offsets, and the grouped-GEMM row-tile lists.
// With bms == 0 every expert's rows are cut into tiles of height bm
// (list 0).  With bms > 0 list 0 holds the full tiles of height bm and list 1
// one tile of height bms for each expert's remaining rows; a remainder of more
// than bms rows becomes one partial tile of list 0 instead.
// n_tiles[0..1] = list sizes.
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ chunk_counts,
                                                    int nchunks, int N, int bm, int bms,
                                                    int* __restrict__ chunk_base,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offs,
                                                    int4* __restrict__ tiles,
                                                    int4* __restrict__ tiles2,
                                                    int* __restrict__ n_tiles) {
  const int e = threadIdx.x;
  int total = 0;
  if (e < N && nchunks == 0) {
    total = counts[e];
  } else if (e < N) {
    int c = 0;
    for (; c + 32 <= nchunks; c += 32) {          // 32 independent loads in flight
      int v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = chunk_counts[(int64_t)(c + i) * N + e];
#pragma unroll
      for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(v[i]));
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        chunk_base[(int64_t)(c + i) * N + e] = total;
        total += v[i];
      }
    }
    for (; c < nchunks; ++c) {
      const int v = chunk_counts[(int64_t)c * N + e];
      chunk_base[(int64_t)c * N + e] = total;
      total += v;
    }
  }
  int all = 0;
  const int off = block_excl_scan_1024(total, &all);
  int nbig = bms > 0 ? total / bm : (total + bm - 1) / bm;
  int rem = bms > 0 ? total - nbig * bm : 0;
  if (bms > 0 && rem > bms) {                     // one partial tile of height bm: the expert's
    nbig += 1;                                    // weights are streamed once, not twice
    rem = 0;
  }
  const int nsmall = bms > 0 ? (rem + bms - 1) / bms : 0;
  int all_big = 0, all_small = 0;
  const int toff = block_excl_scan_1024(nbig, &all_big);
  const int soff = block_excl_scan_1024(nsmall, &all_small);
  if (e < N) {
    counts[e] = total;
    offs[e] = off;
    if (e == N - 1) offs[N] = off + total;
    for (int i = 0; i < nbig; ++i)
      tiles[toff + i] = make_int4(e, off + i * bm, min(off + total, off + (i + 1) * bm), 0);
    const int base = off + nbig * bm;
    for (int i = 0; i < nsmall; ++i)
      tiles2[soff + i] = make_int4(e, base + i * bms, min(off + total, base + (i + 1) * bms), 0);
  }
  if (e == 0) {
    n_tiles[0] = all_big;
    n_tiles[1] = all_small;
  }
}

hipError_t launch_scan(const int* chunk_counts, int nchunks, int N, int bm, int bms,
                       int* chunk_base, int* counts, int* offs, int4* tiles, int4* tiles2,
                       int* n_tiles, hipStream_t s) {
  if (N > 1024) return hipErrorInvalidValue;
  if (nchunks > 32) {             // many chunks: the per-expert prefix in parallel first
    hipLaunchKernelGGL(chunk_prefix_kernel, dim3((N + 63) / 64), dim3(1024), 0, s, chunk_counts,
                       nchunks, N, chunk_base, counts);
    nchunks = 0;
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, N, bm, bms,
                     chunk_base, counts, offs, tiles, tiles2, n_tiles);
  return hipGetLastError();
}

// One wavefront per chunk of tc tokens (tc * K <= kScatterMax).  The chunk's
// expert ids and its per-expert start slots are first staged in LDS with all
// loads in flight; then tokens are visited in order, lane k handling
// assignment (t, k).  A token's K experts are distinct, so the K lanes update
// K different LDS counters: within an expert the slots follow (t, k) order, a
// stable and deterministic scatter.
constexpr int kScatterMax = 2048;
__global__ __launch_bounds__(64) void scatter_kernel(const int* __restrict__ idx, int T, int K,
                                                     int N, int tc,
                                                     const int* __restrict__ chunk_base,
                                                     const int* __restrict__ offs,
                                                     int* __restrict__ slot_token,
                                                     int* __restrict__ tk_slot) {
  __shared__ int cnt[1024];
  __shared__ int sidx[kScatterMax];
  const int c = blockIdx.x, lane = threadIdx.x;
  const int t0 = c * tc, t1 = min(T, t0 + tc);
  const int n = (t1 - t0) * K;
  const int* src = idx + (int64_t)t0 * K;
  const int* cb = chunk_base + (int64_t)c * N;
  for (int i0 = 0; i0 < n; i0 += 8 * 64) {        // 8 loads per lane in flight
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[min(i0 + u * 64 + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * 64 + lane < n) sidx[i0 + u * 64 + lane] = v[u];
  }
  for (int i0 = 0; i0 < N; i0 += 8 * 64) {
    int a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + u * 64 + lane, N - 1);
      a[u] = offs[i];
      b[u] = cb[i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(a[u]), "+v"(b[u]));
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * 64 + lane < N) cnt[i0 + u * 64 + lane] = a[u] + b[u];
  }
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    if (lane < K) {
      const int e = sidx[(t - t0) * K + lane];
      const int slot = cnt[e];
      cnt[e] = slot + 1;
      slot_token[slot] = t;
      tk_slot[(int64_t)t * K + lane] = slot;
    }
  }
}

hipError_t launch_scatter(const int* idx, int T, int K, int N, int tc, const int* chunk_base,
                          const int* offs, int* slot_token, int* tk_slot, hipStream_t s) {
  const int nchunks = (T + tc - 1) / tc;
  if ((int64_t)tc * K > kScatterMax || N > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(64), 0, s, idx, T, K, N, tc,
                     chunk_base, offs, slot_token, tk_slot);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// out[t][c] = add[t][c] + sum_{k=0..K-1} gate[t][k] * O[tk_slot[t][k]][c], summed
// in fp32 in that fixed order (no atomics), then stored once.  8 columns per
// thread.
template <bool OF32, bool OUTF32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ O, int64_t ldo,
                                                      const int* __restrict__ tk_slot,
                                                      const float* __restrict__ gate, int K, int W,
                                                      const float* __restrict__ add,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x;
  const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (c0 >= W) return;
  float acc[8];
  if (add) {
    const float4* p = reinterpret_cast<const float4*>(add + (int64_t)t * W + c0);
    float4 a = p[0], b = p[1];
    acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
    acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  }
  const int* sl = tk_slot + (int64_t)t * K;
  const float* gl = gate + (int64_t)t * K;
  // groups of G gathered rows: their loads go out together, the sums still
  // run in k order; then the K % G rows left one at a time
  constexpr int G = 4;
  int k = 0;
  for (; k + G <= K; k += G) {
    float g[G];
    int64_t sr[G];
#pragma unroll
    for (int i = 0; i < G; ++i) { sr[i] = sl[k + i]; g[i] = gl[k + i]; }
    if (OF32) {
      float4 a[G], b[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float4* p = reinterpret_cast<const float4*>((const float*)O + sr[i] * ldo + c0);
        a[i] = p[0];
        b[i] = p[1];
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        acc[0] += g[i] * a[i].x; acc[1] += g[i] * a[i].y; acc[2] += g[i] * a[i].z; acc[3] += g[i] * a[i].w;
        acc[4] += g[i] * b[i].x; acc[5] += g[i] * b[i].y; acc[6] += g[i] * b[i].z; acc[7] += g[i] * b[i].w;
      }
    } else {
      uint4 v[G];
#pragma unroll
      for (int i = 0; i < G; ++i) v[i] = *reinterpret_cast<const uint4*>((const uint16_t*)O + sr[i] * ldo + c0);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        acc[0] += g[i] * bf2f(v[i].x & 0xFFFFu); acc[1] += g[i] * bf2f(v[i].x >> 16);
        acc[2] += g[i] * bf2f(v[i].y & 0xFFFFu); acc[3] += g[i] * bf2f(v[i].y >> 16);
        acc[4] += g[i] * bf2f(v[i].z & 0xFFFFu); acc[5] += g[i] * bf2f(v[i].z >> 16);
        acc[6] += g[i] * bf2f(v[i].w & 0xFFFFu); acc[7] += g[i] * bf2f(v[i].w >> 16);
      }
    }
  }
  for (; k < K; ++k) {
    const int64_t sr = sl[k];
    const float g = gl[k];
    if (OF32) {
      const float4* p = reinterpret_cast<const float4*>((const float*)O + sr * ldo + c0);
      float4 a = p[0], b = p[1];
      acc[0] += g * a.x; acc[1] += g * a.y; acc[2] += g * a.z; acc[3] += g * a.w;
      acc[4] += g * b.x; acc[5] += g * b.y; acc[6] += g * b.z; acc[7] += g * b.w;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>((const uint16_t*)O + sr * ldo + c0);
      acc[0] += g * bf2f(v.x & 0xFFFFu); acc[1] += g * bf2f(v.x >> 16);
      acc[2] += g * bf2f(v.y & 0xFFFFu); acc[3] += g * bf2f(v.y >> 16);
      acc[4] += g * bf2f(v.z & 0xFFFFu); acc[5] += g * bf2f(v.z >> 16);
      acc[6] += g * bf2f(v.w & 0xFFFFu); acc[7] += g * bf2f(v.w >> 16);
    }
  }
  if (OUTF32) {
    float4* p = reinterpret_cast<float4*>((float*)out + (int64_t)t * W + c0);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint4 v;
    v.x = pack_bf2(acc[0], acc[1]); v.y = pack_bf2(acc[2], acc[3]);
    v.z = pack_bf2(acc[4], acc[5]); v.w = pack_bf2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>((uint16_t*)out + (int64_t)t * W + c0) = v;
  }
}

hipError_t launch_combine(const void* O, bool o_f32, int64_t ldo, const int* tk_slot,
                          const float* gate, int T, int K, int W, const float* add, void* out,
                          bool out_f32, hipStream_t s) {
  // 8 columns per thread; blocks of up to 256 threads, none idle when W <= 2048
  const int nt = W / 8 > 192 ? 256 : ((W / 8 + 63) / 64) * 64;
  dim3 g(T, (W + nt * 8 - 1) / (nt * 8)), b(nt);
  if (o_f32 && out_f32) hipLaunchKernelGGL((combine_kernel<true, true>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  else if (o_f32) hipLaunchKernelGGL((combine_kernel<true, false>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  else if (out_f32) hipLaunchKernelGGL((combine_kernel<false, true>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  else hipLaunchKernelGGL((combine_kernel<false, false>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  return hipGetLastError();
}

}  // namespace moe
