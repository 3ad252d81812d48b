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

// NVFP4 decode.  A block scale s (E4M3) is converted exactly to fp32 by the
// hardware (v_cvt_scalef32_f32_fp8, unit scale).  The gfx950 conversion
// v_cvt_scalef32_pk_f32_fp4 turns one byte (two E2M1 codes, low nibble first)
// into two fp32 values multiplied by the power of two of its scale operand
// (only the operand's exponent is used); given |s| it applies
// 2^floor(log2|s|), and one fp32 multiply by frexp_mant(s) = s / 2^(floor+1)
// (in [0.5, 1) with s's sign, 0 when s = 0) completes the product.  The result
// is w / 2 for the element's true value w = e2m1 * s: exact, since every
// e2m1 * e4m3 product has at most 6 significant bits; the factor 2 is folded
// into the epilogue's fp32 scale.  The pair is packed to bf16 by taking the
// high halves (exact values, so truncation is exact).
struct Fp4Scale {
  float pow2, frac;
};
// byte 0 of `sbyte` is the E4M3 scale
__device__ __forceinline__ Fp4Scale split_scale(uint32_t sbyte) {
  const float s = __builtin_amdgcn_cvt_scalef32_f32_fp8((int)sbyte, 1.0f, 0);
  Fp4Scale r;
  r.pow2 = __builtin_fabsf(s);
  r.frac = __builtin_amdgcn_frexp_mantf(s);
  return r;
}
template <int BYTE>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, const Fp4Scale& sc) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc.pow2, BYTE);
  const float lo = v.x * sc.frac, hi = v.y * sc.frac;
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
// 8 codes (one dword) -> 8 bf16 (one uint4), each half its true value
__device__ __forceinline__ uint4 fp4x8(uint32_t w, const Fp4Scale& sc) {
  return make_uint4(fp4_pair<0>(w, sc), fp4_pair<1>(w, sc), fp4_pair<2>(w, sc), fp4_pair<3>(w, sc));
}

// OCP FP8 E4M3 quantisation: code = RNE_e4m3(clamp(v * r, -448, 448)), r the
// fp32 reciprocal of the per-tensor scale.  The hardware conversion rounds to
// nearest even; the clamp makes the saturation explicit (the format has no
// infinities and 448 is its largest finite value).
__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
// four values -> four codes in one dword (first value in the low byte)
__device__ __forceinline__ uint32_t q8x4(float a, float b, float c, float d, float r) {
  int q = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a * r), sat448(b * r), 0, false);
  q = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c * r), sat448(d * r), q, true);
  return (uint32_t)q;
}
__device__ __forceinline__ uint32_t q8(float v, float r) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(v * r), 0.0f, 0, false) & 0xFFu;
}
// E4M3 -> bf16, exact (every E4M3 value is a bf16 value): codes 2w, 2w+1 of
// the 16-bit word `HI` of w -> bf16x2 (lower code in the low half)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// 8 codes (two dwords) -> 8 bf16 (one uint4)
__device__ __forceinline__ uint4 e4m3x8_bf(uint32_t lo, uint32_t hi) {
  return make_uint4(e4m3x2_bf<false>(lo), e4m3x2_bf<true>(lo), e4m3x2_bf<false>(hi), e4m3x2_bf<true>(hi));
}

// ------------------------------------------------------------------ kernel params
// Weight (B operand) storage of a GEMM.  FP8: A and B are both E4M3 codes.
enum WType : int { WT_BF16 = 0, WT_NVFP4 = 1, WT_FP8 = 2 };
// the epilogue factor that undoes the halving of decoded NVFP4 weights
template <int WT>
constexpr float decode_factor() { return WT == WT_NVFP4 ? 2.0f : 1.0f; }

enum Epi : int {
  EPI_BF16 = 0,        // C(bf16) = g*acc                             (expert down, dense)
  EPI_Z = 1,           // C(f32) = acc and C2(bf16) = acc             (latent z32 / z16)
  EPI_SQRELU_BF16 = 2, // C(bf16) = max(g*acc,0)^2                    (expert up)
  EPI_F32 = 4,         // C(f32) = acc (+ bias[col])                  (router, shared down)
  EPI_BF16_ADD = 5,    // C(bf16) = acc + add[r][c] (fp32)            (up-proj + shared)
  EPI_SQRELU_F32 = 6,  // C(f32) = max(acc,0)^2
  EPI_F32_ADD = 8,     // C(f32) = acc + add[r][c]
  EPI_PARTIAL = 9,     // C(f32)[slice blockIdx.y] = acc over that slice of K (split-K)
  EPI_Z8 = 10,         // C(f32) = acc and C2(e4m3) = q(acc)          (latent z32 / z8)
  EPI_Q8 = 11,         // C(e4m3) = q(acc)                            (latent z8 only)
  EPI_SQRELU_Q8 = 12   // C(e4m3) = q(max(g*acc,0)^2)                 (FP8 expert up)
};
// g: the weight scale times the activation scale: the NVFP4 per-expert global
// scale or the FP8 per-matrix weight scale (b_gscale[group]), times the FP8
// per-tensor scale of the A operand (*a_scale); 1 where absent.  q(v): E4M3
// code of v / *q_scale.  Gates are not applied by any GEMM: the combine step
// multiplies each expert output by its gate while summing a token's K outputs.

// A tile row source.  Logical row r of the GEMM reads physical row
// a_rows ? a_rows[r] : r of A.
struct GemmArgs {
  const void* A; int64_t lda; const int* a_rows;
  const void* B; int64_t ldb; int64_t b_gstride;     // element units (bf16/f32) or bytes (fp4 codes)
  int32_t kseg; int64_t b_segstride;                  // k split into segments of kseg (shared W2)
  const uint8_t* b_scale; int64_t lds_scale; int64_t s_gstride;  // NVFP4 scales
  // NVFP4 weights are k-tiled (codes [K/64][N][32 B], scales [K/64][N][4 B]
  // per group): ldb and lds_scale are the byte strides of one 64-deep k-slab
  const float* b_gscale;                              // NVFP4 / FP8 per-group weight scale
  const float* a_scale;                               // FP8 A: per-tensor scale (device scalar)
  const float* q_scale;                               // FP8 outputs: per-tensor scale
  int32_t M, N, K;
  const int4* tiles; const int* n_tiles;              // grouped: (group, row0, row1, -)
  const int4* tiles2;                                 // grouped: second (remainder) list
  int32_t lists;                                      // grouped: bit 0 list 0, bit 1 list 1
  void* C; int64_t ldc; void* C2; int64_t ldc2;
  const float* bias;                                  // per column
  const float* add; int64_t ld_add;                   // fp32 addend
};

struct SkinnyArgs {
  const void* A; int64_t lda; const int* a_rows;      // bf16, or E4M3 codes with FP8 weights
  const void* B; int64_t ldb; int64_t b_gstride;      // NVFP4: k-tiled as in GemmArgs
  const uint8_t* b_scale; int64_t lds_scale; int64_t s_gstride;
  const float* b_gscale;
  const float* a_scale; const float* q_scale;
  int32_t N, K;
  const int* counts; const int* offs;
  void* C; int64_t ldc;
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
// bf16 or FP8 (fp8: A and B E4M3 codes) dense GEMM of a small batch on the
// skinny kernel over ceil(M / 64) chunks of 64 rows, K split into ks slices
// (K % (256 * ks) == 0, N % 64 == 0), then the same sum and epilogue.  The
// dispatcher sends M <= 64 here, and M <= 256 when the output has fewer than
// num_cu / 8 tiles of 128 x 128.
hipError_t launch_skinny_splitk(const GemmArgs& a, bool fp8, int epi, int ks, float* P, hipStream_t s);
// out = epi( sum over the ks slices of P ), one thread per output element
hipError_t launch_splitk_reduce(const GemmArgs& a, int epi, int ks, const float* P, hipStream_t s);
// num_cu: compute units of the device (the persistent grid is sized from it)
// wt: WT_BF16, WT_NVFP4 (B only) or WT_FP8 (A and B; every size, stride and
// leading dimension in elements = bytes, all even)
hipError_t launch_gemm_bf16(const GemmArgs& a, int wt, int epi, int bm, int bn, int bms,
                            int64_t max_items, int num_cu, hipStream_t s);
// list 1 (the remainder tiles, height 128) of a grouped NVFP4 GEMM alone, on
// 4-wavefront 128 x 256 tiles, two blocks per CU; epi EPI_SQRELU_BF16 or EPI_BF16
hipError_t launch_gemm_fp4_rem(const GemmArgs& a, int epi, int64_t max_items, int num_cu, hipStream_t s);
hipError_t launch_skinny(const SkinnyArgs& a, int wt, int epi, int n_experts, hipStream_t s);
// out[i] = E4M3 code of in[i] / *scale (in bf16), n % 16 == 0
hipError_t launch_quant_fp8(const uint16_t* in, int64_t n, const float* scale, uint8_t* out,
                            hipStream_t s);
// NVFP4 row-major codes/scales -> the k-tiled layout (quant.hip)
hipError_t launch_nvfp4_tile(const uint8_t* codes, const uint8_t* scales, uint8_t* codes_t,
                             uint8_t* scales_t, int64_t n_mats, int rows, int k, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int N, int K, int tc, int* idx, float* gate,
                       int* chunk_counts, hipStream_t s);
hipError_t launch_scan(const int* chunk_counts, int nchunks, int N, int bm, int bms,
                       int* chunk_base, int* counts, int* offs, int4* tiles, int4* tiles2,
                       int* n_tiles, hipStream_t s);
hipError_t launch_scatter(const int* idx, int T, int K, int N, int tc, const int* chunk_base,
                          const int* offs, int* slot_token, int* tk_slot, hipStream_t s);
hipError_t launch_combine(const void* O, bool o_f32, int64_t ldo, const int* tk_slot,
                          const float* gate, int T, int K, int W, const float* add, void* out,
                          bool out_f32, hipStream_t s);

}  // namespace moe
