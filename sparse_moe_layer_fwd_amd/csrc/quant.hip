// Activation quantisation to OCP FP8 E4M3 with a per-tensor scale: the input
// of an FP8 GEMM that no other kernel produces (x for FP8 shared experts, and
// for FP8 routed experts of a layer without latent projection).  FP8
// post-training quantisation of weights and activations: Nemotron 3 Nano blog,
// FP8 quantisation section.  HBM-bound: each thread reads 32 bytes of bf16 and
// writes 16 codes.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint4* __restrict__ in, int64_t n16,
                                                        const float* __restrict__ scale,
                                                        uint4* __restrict__ out) {
  const float r = 1.0f / *scale;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const uint4 a = in[2 * i], b = in[2 * i + 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = q8x4(bf2f(w[2 * j] & 0xFFFFu), bf2f(w[2 * j] >> 16), bf2f(w[2 * j + 1] & 0xFFFFu),
                  bf2f(w[2 * j + 1] >> 16), r);
    out[i] = make_uint4(q[0], q[1], q[2], q[3]);
  }
}

hipError_t launch_quant_fp8(const uint16_t* in, int64_t n, const float* scale, uint8_t* out,
                            hipStream_t s) {
  if (n < 0 || n % 16 != 0) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const int64_t n16 = n / 16;
  const int64_t blocks = (n16 + 255) / 256;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid), dim3(256), 0, s, (const uint4*)in, n16, scale,
                     (uint4*)out);
  return hipGetLastError();
}

// NVFP4 weights from row-major codes [mats][rows][k/2] and scales
// [mats][rows][k/16] to the k-tiled layout the expert GEMMs stream: for each
// matrix, 64-deep k-slab t holds every row's 32 code bytes (elements 64t ..
// 64t + 63) in row order, and every row's 4 scale bytes (blocks 4t .. 4t + 3)
// likewise.  Within a row's 32 bytes the dwords (8 codes each) go in the
// order 0, 2, 4, 6, 1, 3, 5, 7: half h then holds the codes of k 16i + 8h ..
// + 7 for i = 0..3, which one lane half of a GEMM wavefront consumes.  A pure
// permutation of bytes; thread i moves one (matrix, slab, row), consecutive
// threads consecutive rows of one slab.
__global__ __launch_bounds__(256) void nvfp4_tile_kernel(const uint4* __restrict__ codes,
                                                         const uint32_t* __restrict__ scales,
                                                         uint4* __restrict__ codes_t,
                                                         uint32_t* __restrict__ scales_t,
                                                         int64_t total, int rows, int slabs) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i % rows, ms = i / rows;           // ms = matrix * slabs + slab
    const int64_t e = ms / slabs, t = ms - e * slabs;
    const int64_t src = (e * rows + r) * slabs + t;      // 32-byte unit of the row-major codes
    const uint4 a = codes[2 * src], b = codes[2 * src + 1];   // dwords 0-3, 4-7
    codes_t[2 * i] = make_uint4(a.x, a.z, b.x, b.z);
    codes_t[2 * i + 1] = make_uint4(a.y, a.w, b.y, b.w);
    scales_t[i] = scales[src];
  }
}

hipError_t launch_nvfp4_tile(const uint8_t* codes, const uint8_t* scales, uint8_t* codes_t,
                             uint8_t* scales_t, int64_t n_mats, int rows, int k, hipStream_t s) {
  if (n_mats < 0 || rows < 1 || k < 64 || k % 64 != 0) return hipErrorInvalidValue;
  const int64_t total = n_mats * rows * (int64_t)(k / 64);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(nvfp4_tile_kernel, dim3(grid), dim3(256), 0, s, (const uint4*)codes,
                     (const uint32_t*)scales, (uint4*)codes_t, (uint32_t*)scales_t, total, rows, k / 64);
  return hipGetLastError();
}

}  // namespace moe
