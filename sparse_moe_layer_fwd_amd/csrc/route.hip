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
// One DPP step of a 64-bit max: combine with the value of another lane of the
// same row (quad permutations and row rotations have no memory round-trip).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, 0xF, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// Wave-wide max: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror 4, row_ror 8
// leave every lane with its 16-lane row's max; the four row maxima are then read
// as scalars.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1>(v);
  v = dpp_max_step<0x4E>(v);
  v = dpp_max_step<0x124>(v);
  v = dpp_max_step<0x128>(v);
  const uint64_t a = readlane64(v, 0), b = readlane64(v, 16);
  const uint64_t c = readlane64(v, 32), d = readlane64(v, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Zero `n` ints (the chunk histograms) with plain stores: safe inside captured graphs.
__global__ __launch_bounds__(256) void zero_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// One wavefront per token (4 per block).  Each lane holds the logits of experts
// lane, lane+64, ...; K rounds of a wave-wide max over packed (value, id) keys
// give the K largest in descending order.  The per-chunk expert histogram of
// chunk t / tc is kept with integer atomics (order-independent results).
template <int NJ>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int N,
                                                   int K, int tc, int* __restrict__ idx,
                                                   float* __restrict__ gate,
                                                   int* __restrict__ chunk_counts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * 64 + lane;
    key[j] = e < N ? make_key(logits[(int64_t)t * N + e], (uint32_t)e) : 0ull;
  }
  uint32_t taken = 0;
  uint64_t mine = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
    int bj = -1;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (!((taken >> j) & 1u) && key[j] > best) { best = key[j]; bj = j; }
    const uint64_t w = wave_max_u64(best);
    if (bj >= 0 && best == w) taken |= 1u << bj;
    if (lane == k) mine = w;
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

// Single block: per-expert totals over chunks (chunk_base = exclusive prefix
// over chunks), expert offsets, and the grouped-GEMM row-tile lists.  Experts
// with fewer than min_rows rows get no tiles (the skinny kernel takes them).
// With bms == 0 every other expert's rows are cut into tiles of height bm
// (list 0).  With bms > 0 list 0 holds only full tiles of height bm and list 1
// covers each expert's remaining rows with tiles of height bms.
// n_tiles[0..1] = list sizes.
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ chunk_counts,
                                                    int nchunks, int N, int bm, int bms, int min_rows,
                                                    int* __restrict__ chunk_base,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offs,
                                                    int4* __restrict__ tiles,
                                                    int4* __restrict__ tiles2,
                                                    int* __restrict__ n_tiles) {
  const int e = threadIdx.x;
  int total = 0;
  if (e < N) {
    int c = 0;
    for (; c + 8 <= nchunks; c += 8) {            // 8 independent loads in flight
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = chunk_counts[(int64_t)(c + i) * N + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
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
  const bool tiled = total >= min_rows;
  const int nbig = !tiled ? 0 : bms > 0 ? total / bm : (total + bm - 1) / bm;
  const int rem = bms > 0 && tiled ? total - nbig * bm : 0;
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

hipError_t launch_scan(const int* chunk_counts, int nchunks, int N, int bm, int bms, int min_rows,
                       int* chunk_base, int* counts, int* offs, int4* tiles, int4* tiles2,
                       int* n_tiles, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, N, bm, bms,
                     min_rows, chunk_base, counts, offs, tiles, tiles2, n_tiles);
  return hipGetLastError();
}

// One wavefront per chunk of tc tokens.  Tokens are visited in order; lane k
// handles assignment (t, k).  A token's K experts are distinct, so the K lanes
// update K different LDS counters: within an expert the slots follow (t, k)
// order, a stable and deterministic scatter.
__global__ __launch_bounds__(64) void scatter_kernel(const int* __restrict__ idx, int T, int K,
                                                     int N, int tc,
                                                     const int* __restrict__ chunk_base,
                                                     const int* __restrict__ offs,
                                                     int* __restrict__ slot_token,
                                                     int* __restrict__ tk_slot) {
  __shared__ int cnt[1024];
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int i = lane; i < N; i += 64) cnt[i] = offs[i] + chunk_base[(int64_t)c * N + i];
  __syncthreads();
  const int t1 = min(T, (c + 1) * tc);
  for (int t = c * tc; t < t1; ++t) {
    if (lane < K) {
      const int64_t a = (int64_t)t * K + lane;
      const int e = idx[a];
      const int slot = cnt[e];
      cnt[e] = slot + 1;
      slot_token[slot] = t;
      tk_slot[a] = slot;
    }
  }
}

hipError_t launch_scatter(const int* idx, int T, int K, int N, int tc, const int* chunk_base,
                          const int* offs, int* slot_token, int* tk_slot, hipStream_t s) {
  const int nchunks = (T + tc - 1) / tc;
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
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
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
  for (int k = 0; k < K; ++k) {
    const int64_t s = sl[k];
    const float g = gl[k];
    if (OF32) {
      const float4* p = reinterpret_cast<const float4*>((const float*)O + s * ldo + c0);
      float4 a = p[0], b = p[1];
      acc[0] += g * a.x; acc[1] += g * a.y; acc[2] += g * a.z; acc[3] += g * a.w;
      acc[4] += g * b.x; acc[5] += g * b.y; acc[6] += g * b.z; acc[7] += g * b.w;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>((const uint16_t*)O + s * ldo + c0);
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
  dim3 g(T, (W + 2047) / 2048), b(256);
  if (o_f32 && out_f32) hipLaunchKernelGGL((combine_kernel<true, true>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  else if (o_f32) hipLaunchKernelGGL((combine_kernel<true, false>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  else if (out_f32) hipLaunchKernelGGL((combine_kernel<false, true>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  else hipLaunchKernelGGL((combine_kernel<false, false>), g, b, 0, s, O, ldo, tk_slot, gate, K, W, add, out);
  return hipGetLastError();
}

}  // namespace moe
