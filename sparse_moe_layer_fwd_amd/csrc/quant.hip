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

}  // namespace moe
