// Internal declarations shared by the HIP sources of libmoe.so (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// ------------------------------------------------------------------ conversions
// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// two fp32 -> packed bf16x2 (lo in low half)
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// NVFP4 element: E2M1 code (4 bits) -> fp32, from the format's fields.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t mag = c & 7u;
  uint32_t bits;
  if (mag < 2u) bits = mag ? 0x3F000000u : 0u;            // 0, 0.5 (subnormal)
  else bits = (((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22);
  return __uint_as_float(bits | ((c & 8u) << 28));
}
// NVFP4 block scale: E4M3 byte -> fp32 (bias 7; exponent field 0 is subnormal).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (b & 0x80u) ? -v : v;
}

// ------------------------------------------------------------------ kernel params
enum Epi : int {
  EPI_BF16 = 0,        // C(bf16) = g*acc                             (expert down, dense)
  EPI_Z = 1,           // C(f32) = acc and C2(bf16) = acc             (latent z32 / z16)
  EPI_SQRELU_BF16 = 2, // C(bf16) = max(g*acc,0)^2                    (expert up)
  EPI_F32 = 4,         // C(f32) = acc (+ bias[col])                  (router, shared down)
  EPI_BF16_ADD = 5,    // C(bf16) = acc + add[r][c] (fp32)            (up-proj + shared)
  EPI_SQRELU_F32 = 6,  // C(f32) = max(acc,0)^2
  EPI_F32_ADD = 8,     // C(f32) = acc + add[r][c]
  EPI_PARTIAL = 9      // C(f32)[slice blockIdx.y] = acc over that slice of K (split-K)
};
// g: the NVFP4 per-expert global scale (1 for bf16 weights).  Gates are not
// applied by any GEMM: the combine step multiplies each expert output by its
// gate while summing a token's K outputs.

// A tile row source.  Logical row r of the GEMM reads physical row
// a_rows ? a_rows[r] : r of A.
struct GemmArgs {
  const void* A; int64_t lda; const int* a_rows;
  const void* B; int64_t ldb; int64_t b_gstride;     // element units (bf16/f32) or bytes (fp4 codes)
  int32_t kseg; int64_t b_segstride;                  // k split into segments of kseg (shared W2)
  const uint8_t* b_scale; int64_t lds_scale; int64_t s_gstride;  // NVFP4 scales
  const float* b_gscale;                              // NVFP4 per-group global scale
  int32_t M, N, K;
  const int4* tiles; const int* n_tiles;              // grouped: (group, row0, row1, -)
  const int4* tiles2;                                 // grouped: second (remainder) list
  void* C; int64_t ldc; void* C2; int64_t ldc2;
  const float* bias;                                  // per column
  const float* add; int64_t ld_add;                   // fp32 addend
};

struct SkinnyArgs {
  const uint16_t* A; int64_t lda; const int* a_rows;
  const void* B; int64_t ldb; int64_t b_gstride;
  const uint8_t* b_scale; int64_t lds_scale; int64_t s_gstride;
  const float* b_gscale;
  int32_t N, K;
  const int* counts; const int* offs;
  int32_t max_rows;                                   // experts with >= max_rows rows are skipped
  uint16_t* C; int64_t ldc;
  float* P; int64_t p_slice;                          // split-K partials: slice s at P + s * p_slice
};

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_gemm_f32(const GemmArgs& a, bool a_is_bf16, int epi, int grid_cap, hipStream_t s);
// Dense GEMM with K split into ks slices (ks > 1): partial sums into P
// (ks * M * N floats), then a fixed-order sum over the slices and epilogue epi.
// Every dimension of the fp32 kernel: K % (32 * ks) == 0.
hipError_t launch_gemm_f32_splitk(const GemmArgs& a, bool a_is_bf16, int epi, int ks, float* P,
                                  hipStream_t s);
// bf16 dense GEMM with M <= 64 on the skinny kernel, K split into ks slices
// (K % (256 * ks) == 0, N % 64 == 0), then the same sum and epilogue.
hipError_t launch_skinny_splitk(const GemmArgs& a, int epi, int ks, float* P, hipStream_t s);
// out = epi( sum over the ks slices of P ), one thread per output element
hipError_t launch_splitk_reduce(const GemmArgs& a, int epi, int ks, const float* P, hipStream_t s);
// num_cu: compute units of the device (the persistent grid is sized from it)
hipError_t launch_gemm_bf16(const GemmArgs& a, bool b_nvfp4, int epi, int bm, int bn, int bms,
                            int64_t max_items, int num_cu, hipStream_t s);
hipError_t launch_skinny(const SkinnyArgs& a, bool b_nvfp4, int epi, int n_experts, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int N, int K, int tc, int* idx, float* gate,
                       int* chunk_counts, hipStream_t s);
hipError_t launch_scan(const int* chunk_counts, int nchunks, int N, int bm, int bms, int min_rows,
                       int* chunk_base, int* counts, int* offs, int4* tiles, int4* tiles2,
                       int* n_tiles, hipStream_t s);
hipError_t launch_scatter(const int* idx, int T, int K, int N, int tc, const int* chunk_base,
                          const int* offs, int* slot_token, int* tk_slot, hipStream_t s);
hipError_t launch_combine(const void* O, bool o_f32, int64_t ldo, const int* tk_slot,
                          const float* gate, int T, int K, int W, const float* add, void* out,
                          bool out_f32, hipStream_t s);

}  // namespace moe
