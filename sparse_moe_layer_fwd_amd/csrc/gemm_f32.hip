// fp32 GEMM on CDNA4 fp32 MFMA (v_mfma_f32_16x16x4_f32): the router GEMV
// (logits = W_r z + b_r, kept in fp32 so that expert selection matches an exact
// reference) and every GEMM of an all-fp32 layer.  Dense or grouped over a
// device-side row-tile list, with an optional row gather on A.
//
// Tile 64x64x32, 256 threads = 4 wavefronts in a 2x2 grid, each 32x32 as 2x2
// MFMA 16x16 blocks.  Operands are staged in LDS (padded rows).
#include "common.h"

namespace moe {

template <bool ABF16, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 32;
  __shared__ float As[BM][BK + 1];
  __shared__ float Bs[BN][BK + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (p.N + BN - 1) / BN;
  const int nrt = p.tiles ? *p.n_tiles : (p.M + BM - 1) / BM;
  const int total = nrt * ntn;
  const int lr = tid >> 2, kq = (tid & 3) * 8;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int rt = item / ntn, nt = item - rt * ntn;
    int g = 0, r0, r1;
    if (p.tiles) {
      const int4 tl = p.tiles[rt];
      g = tl.x; r0 = tl.y; r1 = tl.z;
    } else {
      r0 = rt * BM; r1 = min(p.M, r0 + BM);
    }
    const int n0 = nt * BN;
    int ar = min(r0 + lr, r1 - 1);
    const int64_t arow = p.a_rows ? (int64_t)p.a_rows[ar] : (int64_t)ar;
    const int bn = min(n0 + lr, p.N - 1);
    const float* Bg = (const float*)p.B + (int64_t)g * p.b_gstride + (int64_t)bn * p.ldb;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // split-K (EPI_PARTIAL): slice blockIdx.y of gridDim.y covers K / gridDim.y
    const int kl = EPI == EPI_PARTIAL ? p.K / (int)gridDim.y : p.K;
    const int kb = EPI == EPI_PARTIAL ? (int)blockIdx.y * kl : 0;
    // this thread's 8 A and 8 B values of k-step k0, loaded one k-step ahead
    // (registers) so that their latency overlaps the MFMAs of the current one
    auto load = [&](int k0, float (&av)[8], float (&bv)[8]) {
      if (ABF16) {
        const uint4 v = *reinterpret_cast<const uint4*>((const uint16_t*)p.A + arow * p.lda + k0 + kq);
        av[0] = bf2f(v.x & 0xFFFFu); av[1] = bf2f(v.x >> 16);
        av[2] = bf2f(v.y & 0xFFFFu); av[3] = bf2f(v.y >> 16);
        av[4] = bf2f(v.z & 0xFFFFu); av[5] = bf2f(v.z >> 16);
        av[6] = bf2f(v.w & 0xFFFFu); av[7] = bf2f(v.w >> 16);
      } else {
        const float4* q = reinterpret_cast<const float4*>((const float*)p.A + arow * p.lda + k0 + kq);
        const float4 x0 = q[0], x1 = q[1];
        av[0] = x0.x; av[1] = x0.y; av[2] = x0.z; av[3] = x0.w;
        av[4] = x1.x; av[5] = x1.y; av[6] = x1.z; av[7] = x1.w;
      }
      const int seg = k0 / p.kseg, kin = k0 - seg * p.kseg;
      const float4* q = reinterpret_cast<const float4*>(Bg + (int64_t)seg * p.b_segstride + kin + kq);
      const float4 x0 = q[0], x1 = q[1];
      bv[0] = x0.x; bv[1] = x0.y; bv[2] = x0.z; bv[3] = x0.w;
      bv[4] = x1.x; bv[5] = x1.y; bv[6] = x1.z; bv[7] = x1.w;
    };
    float av[8], bv[8];
    load(kb, av, bv);
    for (int k0 = kb; k0 < kb + kl; k0 += BK) {
      __syncthreads();                                   // the previous k-step's reads are done
#pragma unroll
      for (int i = 0; i < 8; ++i) { As[lr][kq + i] = av[i]; Bs[lr][kq + i] = bv[i]; }
      __syncthreads();
      if (k0 + BK < kb + kl) load(k0 + BK, av, bv);
#pragma unroll
      for (int kk = 0; kk < BK; kk += 4) {
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = As[wm * 32 + i * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bs[wn * 32 + j * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
    // epilogue: D[i = 4*(lane/16) + r][j = lane%16] of each 16x16 block
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
          const int col = n0 + wn * 32 + j * 16 + (lane & 15);
          if (row >= r1 || col >= p.N) continue;
          float v = acc[i][j][r];
          float* C = (float*)p.C + (int64_t)row * p.ldc + col;
          if (EPI == EPI_PARTIAL) {
            C[(int64_t)blockIdx.y * p.M * p.ldc] = v;
          } else if (EPI == EPI_F32) {
            if (p.bias) v += p.bias[col];
            *C = v;
          } else if (EPI == EPI_SQRELU_F32) {
            v = fmaxf(v, 0.0f);
            *C = v * v;
          } else if (EPI == EPI_F32_ADD) {
            *C = v + p.add[(int64_t)row * p.ld_add + col];
          }
        }
  }
}

// Wide tiles for the large dense fp32 GEMMs (the router of a prefill batch):
// BM x 128 x 32 with BM = 64 or 128, 4 wavefronts in a 2x2 grid, each
// (BM/2) x 64 as v_mfma_f32_32x32x2_f32 blocks (4 times the MFMA work per
// fragment read of the 64x64 tile above).  Operands are double-buffered in
// LDS with one barrier per k-step; the next k-step's global loads (for
// 64-row tiles the next two) sit in registers while the current one is
// multiplied.  The sums run over k in
// ascending order within each MFMA chain, as in every other fp32 GEMM here.
template <bool ABF16, int BM>
__global__ __launch_bounds__(256) void gemm_f32_wide_kernel(GemmArgs p) {
  constexpr int BN = 128, BK = 32, LD = BK + 1, TI = BM / 64;
  __shared__ float As[2][BM * LD];
  __shared__ float Bs[2][BN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = p.N / BN;
  const int total = ((p.M + BM - 1) / BM) * ntn;
  const int nk = p.K / BK;
  const int lr = tid >> 3, kc = (tid & 7) * 4;     // rows lr + 32 q, k chunk kc .. kc + 3
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int rt = item / ntn, nt = item - rt * ntn;
    const int r0 = rt * BM, n0 = nt * BN;
    // BM = 64: two register sets, k-step ks + 2 is loaded while ks is
    // multiplied and ks + 1 (already in registers) waits to be stored, so each
    // load has two k-steps of MFMA work to land.  BM = 128 keeps one set (two
    // would take it past 256 registers, to one wavefront per SIMD).
    constexpr bool DEEP = BM == 64;
    f32x4 ra0[BM / 32], rb0[4], ra1[BM / 32], rb1[4];
    auto load = [&](f32x4 (&ra)[BM / 32], f32x4 (&rb)[4], int k0) {
#pragma unroll
      for (int q = 0; q < BM / 32; ++q) {
        const int64_t row = min(r0 + lr + 32 * q, p.M - 1);
        if (ABF16) {
          const uint2 v = *reinterpret_cast<const uint2*>((const uint16_t*)p.A + row * p.lda + k0 + kc);
          ra[q] = f32x4{bf2f(v.x & 0xFFFFu), bf2f(v.x >> 16), bf2f(v.y & 0xFFFFu), bf2f(v.y >> 16)};
        } else {
          ra[q] = *reinterpret_cast<const f32x4*>((const float*)p.A + row * p.lda + k0 + kc);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rb[q] = *reinterpret_cast<const f32x4*>((const float*)p.B + (int64_t)(n0 + lr + 32 * q) * p.ldb + k0 + kc);
    };
    auto store = [&](const f32x4 (&ra)[BM / 32], const f32x4 (&rb)[4], int buf) {
#pragma unroll
      for (int q = 0; q < BM / 32; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) As[buf][(lr + 32 * q) * LD + kc + i] = ra[q][i];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) Bs[buf][(lr + 32 * q) * LD + kc + i] = rb[q][i];
    };
    f32x16 acc[TI][2];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    auto compute = [&](int buf) {
      const float* Ab = As[buf] + (wm * (BM / 2) + (lane & 31)) * LD + (lane >> 5);
      const float* Bb = Bs[buf] + (wn * 64 + (lane & 31)) * LD + (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < BK; kk += 2) {
        float a[TI], b[2];
#pragma unroll
        for (int i = 0; i < TI; ++i) a[i] = Ab[i * 32 * LD + kk];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bb[j * 32 * LD + kk];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    };
    __syncthreads();                                     // the previous item's reads are done
    load(ra0, rb0, 0);
    store(ra0, rb0, 0);
    if (!DEEP) {
      __syncthreads();
      for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) load(ra0, rb0, (ks + 1) * BK);
        compute(buf);
        if (ks + 1 < nk) store(ra0, rb0, buf ^ 1);
        __syncthreads();
      }
    } else {
      if (nk > 1) load(ra0, rb0, BK);
      __syncthreads();
      // even k-steps use buffer 0 and find the next k-step in set 0; odd ones
      // use buffer 1 and set 1.  The steady state has no branches (so the
      // compiler's load waits stay per register set); the last 2-3 k-steps
      // take the guarded loop.
      int ks = 0;
      for (; ks + 3 < nk; ks += 2) {
        load(ra1, rb1, (ks + 2) * BK);
        __builtin_amdgcn_sched_barrier(0);             // the loads go out before the MFMAs
        compute(0);
        store(ra0, rb0, 1);
        __syncthreads();
        load(ra0, rb0, (ks + 3) * BK);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        store(ra1, rb1, 0);
        __syncthreads();
      }
      for (; ks < nk; ks += 2) {
        if (ks + 2 < nk) load(ra1, rb1, (ks + 2) * BK);
        compute(0);
        if (ks + 1 < nk) store(ra0, rb0, 1);
        __syncthreads();
        if (ks + 1 >= nk) break;
        if (ks + 3 < nk) load(ra0, rb0, (ks + 3) * BK);
        compute(1);
        if (ks + 2 < nk) store(ra1, rb1, 0);
        __syncthreads();
      }
    }
    // D[m][n] of each 32x32 block: n = lane % 32, m = 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        const float bias = p.bias ? p.bias[col] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < p.M) ((float*)p.C)[(int64_t)row * p.ldc + col] = acc[i][j][r] + bias;
        }
      }
  }
}

hipError_t launch_gemm_f32(const GemmArgs& a, bool a_is_bf16, int epi, int grid_cap, hipStream_t s) {
  if (!a.tiles && !a.a_rows && epi == EPI_F32 && a.N % 128 == 0 && a.K % 32 == 0 && a.kseg >= a.K &&
      a.lda % 4 == 0 && a.ldb % 4 == 0) {
    // grid_cap is two blocks per CU: 128-row tiles when they fill it, else 64-row
    const int64_t t128 = (int64_t)((a.M + 127) / 128) * (a.N / 128);
    const int64_t t64 = (int64_t)((a.M + 63) / 64) * (a.N / 128);
    if (t64 >= grid_cap) {
      const bool big = t128 >= grid_cap;
      const int64_t total = big ? t128 : t64;
      dim3 g((unsigned)(total < grid_cap ? total : grid_cap)), b(256);
      if (big && a_is_bf16) hipLaunchKernelGGL((gemm_f32_wide_kernel<true, 128>), g, b, 0, s, a);
      else if (big) hipLaunchKernelGGL((gemm_f32_wide_kernel<false, 128>), g, b, 0, s, a);
      else if (a_is_bf16) hipLaunchKernelGGL((gemm_f32_wide_kernel<true, 64>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm_f32_wide_kernel<false, 64>), g, b, 0, s, a);
      return hipGetLastError();
    }
  }
  const int ntn = (a.N + 63) / 64;
  const int nrt_max = a.tiles ? a.M : (a.M + 63) / 64;   // grouped: M carries the tile bound
  int64_t total = (int64_t)nrt_max * ntn;
  int grid = (int)(total < grid_cap ? total : grid_cap);
  if (grid < 1) grid = 1;
  dim3 g(grid), b(256);
#define MOE_F32_CASE(AB, E) \
  hipLaunchKernelGGL((gemm_f32_kernel<AB, E>), g, b, 0, s, a)
  switch (epi) {
    case EPI_F32: if (a_is_bf16) MOE_F32_CASE(true, EPI_F32); else MOE_F32_CASE(false, EPI_F32); break;
    case EPI_SQRELU_F32: if (a_is_bf16) MOE_F32_CASE(true, EPI_SQRELU_F32); else MOE_F32_CASE(false, EPI_SQRELU_F32); break;
    case EPI_F32_ADD: if (a_is_bf16) MOE_F32_CASE(true, EPI_F32_ADD); else MOE_F32_CASE(false, EPI_F32_ADD); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_F32_CASE
  return hipGetLastError();
}

// out[r][c] = epi( g * sum_{s=0..ks-1} P[s][r][c] ), summed in that fixed
// order; g = the weight scale b_gscale[0] times the activation scale *a_scale
// (FP8 dense GEMMs), 1 where absent.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int ks, int M,
                                                            int N, GemmArgs p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int row = (int)(i / N), col = (int)(i - (int64_t)row * N);
  // slices summed in order 0 .. ks-1, eight (then four) loads in flight at a time
  const int64_t MN = (int64_t)M * N;
  float v = 0.0f;
  int k = 0;
  for (; k + 8 <= ks; k += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = P[(int64_t)(k + j) * MN + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += t[j];
  }
  for (; k + 4 <= ks; k += 4) {
    float t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = P[(int64_t)(k + j) * MN + i];
#pragma unroll
    for (int j = 0; j < 4; ++j) v += t[j];
  }
  for (; k < ks; ++k) v += P[(int64_t)k * MN + i];
  v *= (p.b_gscale ? p.b_gscale[0] : 1.0f) * (p.a_scale ? *p.a_scale : 1.0f);
  const float rq = (EPI == EPI_Z8 || EPI == EPI_Q8 || EPI == EPI_SQRELU_Q8) ? 1.0f / *p.q_scale : 1.0f;
  if (EPI == EPI_F32) {
    if (p.bias) v += p.bias[col];
    ((float*)p.C)[(int64_t)row * p.ldc + col] = v;
  } else if (EPI == EPI_F32_ADD) {
    ((float*)p.C)[(int64_t)row * p.ldc + col] = v + p.add[(int64_t)row * p.ld_add + col];
  } else if (EPI == EPI_SQRELU_F32) {
    v = fmaxf(v, 0.0f);
    ((float*)p.C)[(int64_t)row * p.ldc + col] = v * v;
  } else if (EPI == EPI_Z) {
    ((float*)p.C)[(int64_t)row * p.ldc + col] = v;
    ((uint16_t*)p.C2)[(int64_t)row * p.ldc2 + col] = (uint16_t)f2bf(v);
  } else if (EPI == EPI_BF16) {
    ((uint16_t*)p.C)[(int64_t)row * p.ldc + col] = (uint16_t)f2bf(v);
  } else if (EPI == EPI_BF16_ADD) {
    ((uint16_t*)p.C)[(int64_t)row * p.ldc + col] = (uint16_t)f2bf(v + p.add[(int64_t)row * p.ld_add + col]);
  } else if (EPI == EPI_SQRELU_BF16) {
    v = fmaxf(v, 0.0f);
    ((uint16_t*)p.C)[(int64_t)row * p.ldc + col] = (uint16_t)f2bf(v * v);
  } else if (EPI == EPI_Z8) {
    ((float*)p.C)[(int64_t)row * p.ldc + col] = v;
    ((uint8_t*)p.C2)[(int64_t)row * p.ldc2 + col] = (uint8_t)q8(v, rq);
  } else if (EPI == EPI_Q8) {
    ((uint8_t*)p.C)[(int64_t)row * p.ldc + col] = (uint8_t)q8(v, rq);
  } else if (EPI == EPI_SQRELU_Q8) {
    v = fmaxf(v, 0.0f);
    ((uint8_t*)p.C)[(int64_t)row * p.ldc + col] = (uint8_t)q8(v * v, rq);
  }
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int epi, int ks, const float* P, hipStream_t s) {
  const int64_t n = (int64_t)a.M * a.N;
  dim3 g((unsigned)((n + 255) / 256)), b(256);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_F32>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_F32_ADD: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_F32_ADD>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_SQRELU_F32: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SQRELU_F32>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_Z: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_Z>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_BF16: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_BF16>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_BF16_ADD: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_BF16_ADD>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_SQRELU_BF16: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SQRELU_BF16>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_Z8: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_Z8>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_Q8: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_Q8>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    case EPI_SQRELU_Q8: hipLaunchKernelGGL(splitk_reduce_kernel<EPI_SQRELU_Q8>, g, b, 0, s, P, ks, a.M, a.N, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32_splitk(const GemmArgs& a, bool a_is_bf16, int epi, int ks, float* P,
                                  hipStream_t s) {
  if (a.tiles || ks < 2 || a.K % (32 * ks) != 0) return hipErrorInvalidValue;
  GemmArgs q = a;
  q.C = P; q.ldc = a.N; q.bias = nullptr;
  const int64_t tiles = (int64_t)((a.M + 63) / 64) * ((a.N + 63) / 64);
  dim3 g((unsigned)tiles, (unsigned)ks), b(256);
  if (a_is_bf16) hipLaunchKernelGGL((gemm_f32_kernel<true, EPI_PARTIAL>), g, b, 0, s, q);
  else hipLaunchKernelGGL((gemm_f32_kernel<false, EPI_PARTIAL>), g, b, 0, s, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(a, epi, ks, P, s);
}

}  // namespace moe
