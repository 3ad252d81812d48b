// Skinny grouped expert GEMM: experts with few rows, every expert of a batch
// of up to 128 tokens (batch decode).  Here
// the work is bound by streaming the expert's weights from HBM (the pages:
// latency-bound serving of tens to hundreds of tokens is dominated by expert
// weight traffic; Korean Nemotron 3 summary, section 2.2 LatentMoE), so the
// kernel keeps many bytes of each expert's weights in flight and reads every
// weight byte once per 64 rows.
//
// Grid: (column tiles of 64, experts).  A block owns 64 output columns of one
// expert; its 4 wavefronts split the reduction dimension in four and reduce
// through LDS at the end.  Per step a lane loads 16 contiguous elements of one
// weight row (16 bf16, 16 NVFP4 codes + their block scale, or 16 E4M3 codes)
// and the matching 16 activations of each row block (bf16, or E4M3 codes with
// FP8 weights), decodes codes exactly to bf16, and issues two
// v_mfma_f32_16x16x32_bf16 per (row block, column block).  Both operands use
// the same permutation of the reduction index inside a step, which leaves the
// dot products unchanged.
#include <string.h>

#include "common.h"

namespace moe {

// Rows [row0, row0 + cnt) (cnt <= 64) of expert e, columns [n0, n0 + 64).
// K range [kbeg, kbeg + klen) (klen a multiple of 256, of 512 when WIDE): each
// wavefront takes a quarter.  A lane takes 8 * NCH consecutive elements of its
// rows per step: 16, or 32 E4M3 codes when WIDE (FP8 only), so an FP8 step
// loads as many bytes per lane as a bf16 one.
// sc: the output scale, rq: the reciprocal quantisation scale (EPI_SQRELU_Q8).
template <int WT, int EPI, bool WIDE = false>
__device__ __forceinline__ void skinny_chunk(const SkinnyArgs& p, float (*red)[16][4][64], int e,
                                             int row0, int cnt, int n0, int kbeg, int klen,
                                             float sc = 1.0f, float rq = 1.0f) {
  constexpr bool FP4 = WT == WT_NVFP4, FP8 = WT == WT_FP8;
  static_assert(!WIDE || FP8, "32-element steps for FP8 codes");
  constexpr int NCH = WIDE ? 4 : 2;                      // 8-element chunks per lane and step
  constexpr int KS = 32 * NCH;                           // k per step (4 lane groups)
  constexpr int AEL = FP8 ? 1 : 2;                       // activation element bytes
  constexpr int MAXRB = 4;
  const int nrb = (cnt + 15) >> 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kq = klen >> 2;
  const int kw0 = kbeg + wave * kq;
  const int grp = lane >> 4;                             // which k slice of a step
  const char* arow[MAXRB];
#pragma unroll
  for (int rb = 0; rb < MAXRB; ++rb) {
    const int r = rb * 16 + (lane & 15);
    if (r < cnt) {
      const int lr = row0 + r;
      const int64_t pr = p.a_rows ? (int64_t)p.a_rows[lr] : (int64_t)lr;
      arow[rb] = (const char*)p.A + pr * p.lda * AEL;
    } else {
      arow[rb] = nullptr;
    }
  }
  const uint8_t* brow[4];
  const uint8_t* srow[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int n = min(n0 + cb * 16 + (lane & 15), p.N - 1);
    if (FP4) {                                           // k-tiled: row n of k-slab 0
      brow[cb] = (const uint8_t*)p.B + (int64_t)e * p.b_gstride + (int64_t)n * 32;
      srow[cb] = p.b_scale + (int64_t)e * p.s_gstride + (int64_t)n * 4;
    } else if (FP8) {
      brow[cb] = (const uint8_t*)p.B + (int64_t)e * p.b_gstride + (int64_t)n * p.ldb;
      srow[cb] = nullptr;
    } else {
      brow[cb] = (const uint8_t*)((const uint16_t*)p.B + (int64_t)e * p.b_gstride + (int64_t)n * p.ldb);
      srow[cb] = nullptr;
    }
  }

  f32x4 acc[MAXRB][4];
#pragma unroll
  for (int rb = 0; rb < MAXRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma nounroll
  for (int kb = kw0; kb < kw0 + kq; kb += KS) {
    const int k = kb + grp * 8 * NCH;
    uint4 b[4][NCH];
    uint4 braw[4][WIDE ? NCH / 2 : 1];                   // WIDE: E4M3 codes, decoded at their MFMAs
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (FP4) {
        // the step's 64 k are one k-slab: the lane's 16 codes (dwords 2 grp and
        // 2 grp + 1 of the row, stored at positions grp and 4 + grp) and their
        // scale, decoded by the hardware conversions to half their value (see
        // split_scale; the epilogue scale carries the factor 2)
        const int64_t slab = kb / 64;
        const uint8_t* bs = brow[cb] + slab * p.ldb + grp * 4;
        const uint2 c = make_uint2(*reinterpret_cast<const uint32_t*>(bs),
                                   *reinterpret_cast<const uint32_t*>(bs + 16));
        const Fp4Scale sc = split_scale(srow[cb][slab * p.lds_scale + grp]);
        b[cb][0] = fp4x8(c.x, sc);
        b[cb][1] = fp4x8(c.y, sc);
      } else if (FP8 && WIDE) {
#pragma unroll
        for (int h = 0; h < NCH / 2; ++h) braw[cb][h] = *reinterpret_cast<const uint4*>(brow[cb] + k + 16 * h);
      } else if (FP8) {
        const uint4 c = *reinterpret_cast<const uint4*>(brow[cb] + k);
        b[cb][0] = e4m3x8_bf(c.x, c.y);
        b[cb][1] = e4m3x8_bf(c.z, c.w);
      } else {
        const uint4* q = reinterpret_cast<const uint4*>((const uint16_t*)brow[cb] + k);
        b[cb][0] = q[0];
        b[cb][1] = q[1];
      }
    }
#pragma unroll
    for (int rb = 0; rb < MAXRB; ++rb) {
      if (rb < nrb) {
        uint4 a[NCH];
#pragma unroll
        for (int h = 0; h < NCH; ++h) a[h] = make_uint4(0, 0, 0, 0);
        if (arow[rb]) {
          const uint4* q = reinterpret_cast<const uint4*>(arow[rb] + k * AEL);
          if (FP8) {
#pragma unroll
            for (int h = 0; h < NCH / 2; ++h) {
              const uint4 c = q[h];
              a[2 * h] = e4m3x8_bf(c.x, c.y);
              a[2 * h + 1] = e4m3x8_bf(c.z, c.w);
            }
          } else {
            a[0] = q[0];
            a[1] = q[1];
          }
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int h = 0; h < NCH; ++h) {
            uint4 bh;
            if constexpr (WIDE) {
              const uint4 c = braw[cb][h / 2];
              bh = (h & 1) ? e4m3x8_bf(c.z, c.w) : e4m3x8_bf(c.x, c.y);
            } else {
              bh = b[cb][h];
            }
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[h]), __builtin_bit_cast(bf16x8, bh), acc[rb][cb], 0, 0, 0);
          }
      }
    }
  }

  __syncthreads();                                      // red[] free (previous chunk done)
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < MAXRB; ++rb)
      if (rb < nrb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wave - 1][rb * 4 + cb][i][lane] = acc[rb][cb][i];
  }
  __syncthreads();
  if (wave != 0) return;                                // the caller re-syncs every wavefront
#pragma unroll
  for (int rb = 0; rb < MAXRB; ++rb) {
    if (rb >= nrb) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + (lane >> 4) * 4 + i;     // D[i = 4*(lane/16) + r][j = lane%16]
      if (r >= cnt) continue;
      const int64_t orow = row0 + r;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int col = n0 + cb * 16 + (lane & 15);
        if (col >= p.N) continue;
        float v = acc[rb][cb][i] + red[0][rb * 4 + cb][i][lane] + red[1][rb * 4 + cb][i][lane] +
                  red[2][rb * 4 + cb][i][lane];
        if (EPI == EPI_PARTIAL) {                        // raw slice sum, K slice blockIdx.y
          p.P[(int64_t)blockIdx.y * p.p_slice + orow * p.N + col] = v;
          continue;
        }
        v *= sc;
        if (EPI == EPI_SQRELU_Q8) {
          const float h = fmaxf(v, 0.0f);
          ((uint8_t*)p.C)[orow * p.ldc + col] = (uint8_t)q8(h * h, rq);
          continue;
        }
        uint16_t* C = (uint16_t*)p.C + orow * p.ldc + col;
        if (EPI == EPI_SQRELU_BF16) {
          const float h = fmaxf(v, 0.0f);
          *C = (uint16_t)f2bf(h * h);
        } else {
          *C = (uint16_t)f2bf(v);
        }
      }
    }
  }
}

// Wavefronts per SIMD the register allocation must allow.  Left to itself the
// compiler gives these kernels 220-240 registers per lane (64 of them AGPRs),
// two wavefronts per SIMD; capped at 168 (no spills), three blocks share a CU.  That
// pays where a weight element costs decode work between its load and its MFMA
// (E4M3 and NVFP4 codes: FP8 decode expert GEMMs 0.381 -> 0.326 ms, NVFP4
// 0.629 -> 0.596 ms on the Ultra-like decode shape); bf16 weights stream
// slightly faster (1%) with the larger allocation.
template <int WT>
constexpr int skinny_waves() { return WT == WT_BF16 ? 1 : 3; }

// Grid (column tiles of 64, experts).  Each expert's rows are processed in
// chunks of up to 64 rows.
template <int WT, int EPI, bool WIDE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(skinny_waves<WT>())))
void skinny_kernel(SkinnyArgs p) {
  __shared__ float red[3][16][4][64];                    // partial sums of waves 1..3
  const int e = blockIdx.y;
  const int cnt = p.counts[e];
  if (cnt == 0) return;
  const int row0 = p.offs[e];
  // weight scale times activation scale (1 for bf16 operands), times 2 for
  // NVFP4 weights decoded as half their value; loaded here, ahead of the
  // weight stream, so the epilogue does not wait for them
  const float sc = (p.b_gscale ? p.b_gscale[e] : 1.0f) * (p.a_scale ? *p.a_scale : 1.0f) *
                   decode_factor<WT>();
  const float rq = EPI == EPI_SQRELU_Q8 ? 1.0f / *p.q_scale : 1.0f;
  for (int c0 = 0; c0 < cnt; c0 += 64) {
    skinny_chunk<WT, EPI, WIDE>(p, red, e, row0 + c0, min(64, cnt - c0), blockIdx.x * 64, 0, p.K, sc, rq);
    __syncthreads();
  }
}

// Dense split-K: grid (N / 64, ks, row chunks of 64).  Block (x, y, z) sums
// rows [64 z, 64 z + 64) x columns [64 x, 64 x + 64) over K slice y into the
// fp32 partials P[y].
// (three wavefronts per SIMD here for every operand type: the split-K
// projections measured 2-3% faster with them)
template <int WT, bool WIDE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void skinny_dense_kernel(SkinnyArgs p, int M) {
  __shared__ float red[3][16][4][64];
  const int kl = p.K / (int)gridDim.y;
  const int row0 = blockIdx.z * 64;
  skinny_chunk<WT, EPI_PARTIAL, WIDE>(p, red, 0, row0, min(64, M - row0), blockIdx.x * 64,
                                      (int)blockIdx.y * kl, kl);
}

hipError_t launch_skinny_splitk(const GemmArgs& a, bool fp8, int epi, int ks, float* P, hipStream_t s) {
  if (a.tiles || ks < 1 || a.K % (256 * ks) != 0 || a.N % 64 != 0 || a.kseg < a.K) return hipErrorInvalidValue;
  SkinnyArgs k;
  memset(&k, 0, sizeof(k));
  k.A = a.A; k.lda = a.lda; k.a_rows = nullptr;
  k.B = a.B; k.ldb = a.ldb; k.b_gstride = 0;
  k.N = a.N; k.K = a.K;
  k.P = P; k.p_slice = (int64_t)a.M * a.N;
  dim3 g(a.N / 64, ks, (a.M + 63) / 64), b(256);
  if (fp8 && (a.K / ks) % 512 == 0) hipLaunchKernelGGL((skinny_dense_kernel<WT_FP8, true>), g, b, 0, s, k, a.M);
  else if (fp8) hipLaunchKernelGGL((skinny_dense_kernel<WT_FP8, false>), g, b, 0, s, k, a.M);
  else hipLaunchKernelGGL((skinny_dense_kernel<WT_BF16, false>), g, b, 0, s, k, a.M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(a, epi, ks, P, s);
}

hipError_t launch_skinny(const SkinnyArgs& a, int wt, int epi, int n_experts, hipStream_t s) {
  dim3 g((a.N + 63) / 64, n_experts), b(256);
  if (wt == WT_NVFP4) {
    if (epi == EPI_SQRELU_BF16) hipLaunchKernelGGL((skinny_kernel<WT_NVFP4, EPI_SQRELU_BF16>), g, b, 0, s, a);
    else if (epi == EPI_BF16) hipLaunchKernelGGL((skinny_kernel<WT_NVFP4, EPI_BF16>), g, b, 0, s, a);
    else return hipErrorInvalidValue;
  } else if (wt == WT_FP8) {
    const bool wide = a.K % 512 == 0;    // 32 codes per lane and step
    if (epi == EPI_SQRELU_Q8 && wide) hipLaunchKernelGGL((skinny_kernel<WT_FP8, EPI_SQRELU_Q8, true>), g, b, 0, s, a);
    else if (epi == EPI_SQRELU_Q8) hipLaunchKernelGGL((skinny_kernel<WT_FP8, EPI_SQRELU_Q8, false>), g, b, 0, s, a);
    else if (epi == EPI_BF16 && wide) hipLaunchKernelGGL((skinny_kernel<WT_FP8, EPI_BF16, true>), g, b, 0, s, a);
    else if (epi == EPI_BF16) hipLaunchKernelGGL((skinny_kernel<WT_FP8, EPI_BF16, false>), g, b, 0, s, a);
    else return hipErrorInvalidValue;
  } else if (wt == WT_BF16) {
    if (epi == EPI_SQRELU_BF16) hipLaunchKernelGGL((skinny_kernel<WT_BF16, EPI_SQRELU_BF16>), g, b, 0, s, a);
    else if (epi == EPI_BF16) hipLaunchKernelGGL((skinny_kernel<WT_BF16, EPI_BF16>), g, b, 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
