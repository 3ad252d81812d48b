// bf16 GEMM on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation:
// the latent projections d -> l and l -> d, the shared experts, and the grouped
// expert GEMMs of the prefill path.
//
// Grouped mode walks a device-side list of row tiles (expert, row0, row1) made
// by the routing scan, so no host round-trip is needed for the data-dependent
// expert sizes.  The A tile can be gathered through a row map (the expert up
// GEMM reads latent rows straight from z by token id).  B is bf16 or NVFP4:
// NVFP4 codes (E2M1, 16-element E4M3 block scales, FP32 global scale: Korean
// Nemotron 3 summary, section 2.4 NVFP4 Training) are decoded exactly to bf16
// while staging into LDS (every e2m1*e4m3 product is a bf16 value); the global
// scale multiplies the fp32 accumulator in the epilogue.
//
// Tile BM x BN x 64, 256 threads = 4 wavefronts (2x2), each (BM/2) x (BN/2) in
// 32x32 MFMA blocks.  LDS is double-buffered: global loads of tile k+1 are in
// flight while tile k is multiplied.  Rows of 64 bf16 (8 chunks of 16 bytes)
// are stored with chunk index XOR (row & 7) so that a wavefront's 16-byte
// fragment reads spread over all banks.
#include "common.h"

namespace moe {

namespace {

__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t byte, float s) {
  const float lo = e2m1_to_f32(byte & 15u) * s;
  const float hi = e2m1_to_f32((byte >> 4) & 15u) * s;
  // exact products: the bf16 value is the upper half of the fp32 one
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// 16 packed codes (8 bytes in two words) of one block with scale s -> 16 bf16
__device__ __forceinline__ void dequant16(uint32_t w0, uint32_t w1, float s, uint4& o0, uint4& o1) {
  o0.x = fp4x2_to_bf16x2(w0 & 0xFFu, s);
  o0.y = fp4x2_to_bf16x2((w0 >> 8) & 0xFFu, s);
  o0.z = fp4x2_to_bf16x2((w0 >> 16) & 0xFFu, s);
  o0.w = fp4x2_to_bf16x2(w0 >> 24, s);
  o1.x = fp4x2_to_bf16x2(w1 & 0xFFu, s);
  o1.y = fp4x2_to_bf16x2((w1 >> 8) & 0xFFu, s);
  o1.z = fp4x2_to_bf16x2((w1 >> 16) & 0xFFu, s);
  o1.w = fp4x2_to_bf16x2(w1 >> 24, s);
}

__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

}  // namespace

template <int BM, int BN, bool FP4, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int A_CH = BM * 8 / 256;              // 16-byte A chunks per thread
  constexpr int B_CH = FP4 ? BN * 2 / 256 : BN * 8 / 256;
  constexpr int TM = BM / 64, TN = BN / 64;       // 32x32 blocks per wavefront
  __shared__ uint4 smem[2][(BM + BN) * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (p.N + BN - 1) / BN;
  const int nrt = p.tiles ? *p.n_tiles : (p.M + BM - 1) / BM;
  const int total = nrt * ntn;
  const int nk = p.K / 64;

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

    // per-thread global sources
    const uint16_t* asrc[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * 256, r = c >> 3, ch = c & 7;
      const int lr = min(r0 + r, r1 - 1);
      const int64_t pr = p.a_rows ? (int64_t)p.a_rows[lr] : (int64_t)lr;
      asrc[i] = (const uint16_t*)p.A + pr * p.lda + ch * 8;
    }
    const uint8_t* bsrc[B_CH];
    const uint8_t* ssrc[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * 256;
      if (FP4) {
        const int r = c >> 1, half = c & 1;
        const int n = min(n0 + r, p.N - 1);
        bsrc[i] = (const uint8_t*)p.B + (int64_t)g * p.b_gstride + (int64_t)n * p.ldb + half * 16;
        ssrc[i] = p.b_scale + (int64_t)g * p.s_gstride + (int64_t)n * p.lds_scale + half * 2;
      } else {
        const int r = c >> 3, ch = c & 7;
        const int n = min(n0 + r, p.N - 1);
        bsrc[i] = (const uint8_t*)((const uint16_t*)p.B + (int64_t)g * p.b_gstride +
                                   (int64_t)n * p.ldb + ch * 8);
        ssrc[i] = nullptr;
      }
    }

    uint4 ra[A_CH], rb[B_CH];
    uint32_t rs[B_CH];
    auto load = [&](int kt) {
      const int k0 = kt * 64;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const uint4*>(asrc[i] + k0);
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        if (FP4) {
          rb[i] = *reinterpret_cast<const uint4*>(bsrc[i] + k0 / 2);
          rs[i] = *reinterpret_cast<const uint16_t*>(ssrc[i] + k0 / 16);
        } else {
          const int seg = k0 / p.kseg, kin = k0 - seg * p.kseg;
          rb[i] = *reinterpret_cast<const uint4*>(
              (const uint16_t*)bsrc[i] + (int64_t)seg * p.b_segstride + kin);
        }
      }
    };
    auto store = [&](int buf) {
      uint4* As = smem[buf];
      uint4* Bs = smem[buf] + BM * 8;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const int c = tid + i * 256, r = c >> 3, ch = c & 7;
        As[swz(r, ch)] = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * 256;
        if (FP4) {
          const int r = c >> 1, half = c & 1;
          const float s0 = e4m3_to_f32(rs[i] & 0xFFu), s1 = e4m3_to_f32((rs[i] >> 8) & 0xFFu);
          uint4 o0, o1, o2, o3;
          dequant16(rb[i].x, rb[i].y, s0, o0, o1);
          dequant16(rb[i].z, rb[i].w, s1, o2, o3);
          Bs[swz(r, half * 4 + 0)] = o0;
          Bs[swz(r, half * 4 + 1)] = o1;
          Bs[swz(r, half * 4 + 2)] = o2;
          Bs[swz(r, half * 4 + 3)] = o3;
        } else {
          const int r = c >> 3, ch = c & 7;
          Bs[swz(r, ch)] = rb[i];
        }
      }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load(kt + 1);
      const uint4* As = smem[cur];
      const uint4* Bs = smem[cur] + BM * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = s * 2 + (lane >> 5);
        bf16x8 a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = wm * (BM / 2) + i * 32 + (lane & 31);
          a[i] = __builtin_bit_cast(bf16x8, As[swz(r, ch)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = wn * (BN / 2) + j * 32 + (lane & 31);
          b[j] = __builtin_bit_cast(bf16x8, Bs[swz(n, ch)]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }

    // epilogue: D[i = 8*(r/4) + 4*(lane/32) + r%4][j = lane%32] of each 32x32 block
    const float gs = (FP4 && p.b_gscale) ? p.b_gscale[g] : 1.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= r1) continue;
        float rsc = 1.0f;
        if (EPI == EPI_GATE_BF16) rsc = p.row_scale[row];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
          if (col >= p.N) continue;
          const float v = acc[i][j][r] * gs;
          const int64_t o = (int64_t)row * p.ldc + col;
          if (EPI == EPI_BF16) {
            ((uint16_t*)p.C)[o] = (uint16_t)f2bf(v);
          } else if (EPI == EPI_Z) {
            ((float*)p.C)[o] = v;
            ((uint16_t*)p.C2)[(int64_t)row * p.ldc2 + col] = (uint16_t)f2bf(v);
          } else if (EPI == EPI_SQRELU_BF16) {
            const float h = fmaxf(v, 0.0f);
            ((uint16_t*)p.C)[o] = (uint16_t)f2bf(h * h);
          } else if (EPI == EPI_GATE_BF16) {
            ((uint16_t*)p.C)[o] = (uint16_t)f2bf(rsc * v);
          } else if (EPI == EPI_F32) {
            ((float*)p.C)[o] = v;
          } else if (EPI == EPI_BF16_ADD) {
            ((uint16_t*)p.C)[o] = (uint16_t)f2bf(v + p.add[(int64_t)row * p.ld_add + col]);
          }
        }
      }
  }
}

hipError_t launch_gemm_bf16(const GemmArgs& a, bool b_nvfp4, int epi, int bm, int max_row_tiles,
                            int grid_cap, hipStream_t s) {
  constexpr int BN = 128;
  const int ntn = (a.N + BN - 1) / BN;
  const int nrt = a.tiles ? max_row_tiles : (a.M + bm - 1) / bm;
  const int64_t total = (int64_t)nrt * ntn;
  int grid = (int)(total < grid_cap ? total : grid_cap);
  if (grid < 1) grid = 1;
  dim3 g(grid), b(256);
  if (bm != 128) return hipErrorInvalidValue;
#define MOE_BF16_CASE(FP4, E) hipLaunchKernelGGL((gemm_bf16_kernel<128, BN, FP4, E>), g, b, 0, s, a)
  if (b_nvfp4) {
    switch (epi) {
      case EPI_SQRELU_BF16: MOE_BF16_CASE(true, EPI_SQRELU_BF16); break;
      case EPI_GATE_BF16: MOE_BF16_CASE(true, EPI_GATE_BF16); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      case EPI_BF16: MOE_BF16_CASE(false, EPI_BF16); break;
      case EPI_Z: MOE_BF16_CASE(false, EPI_Z); break;
      case EPI_SQRELU_BF16: MOE_BF16_CASE(false, EPI_SQRELU_BF16); break;
      case EPI_GATE_BF16: MOE_BF16_CASE(false, EPI_GATE_BF16); break;
      case EPI_F32: MOE_BF16_CASE(false, EPI_F32); break;
      case EPI_BF16_ADD: MOE_BF16_CASE(false, EPI_BF16_ADD); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_BF16_CASE
  return hipGetLastError();
}

}  // namespace moe
