/*
 * moe.h - C ABI of the MI355X LatentMoE layer forward library (libmoe.so).
 *
 * The layer (sources cited by page title and section):
 *   - LatentMoE: each token is projected from the hidden size d to a latent
 *     size l < d (d/l about 4), routed to K of N experts whose FFNs run in the
 *     latent space, combined, and projected back to d.  Per-expert weight
 *     traffic and routed payload shrink by d/l.  ("NVIDIA Nemotron 3: Efficient
 *     and Open Intelligence" Korean summary, section 2.2 LatentMoE; notes.yuuk.io
 *     Nemotron 3 note, method 2 LatentMoE.)
 *   - Standard MoE with always-on shared experts (l = d, no projection):
 *     Nemotron 3 Nano blog, granular MoE section (128 experts, 6 active, 2 shared).
 *   - NVFP4 expert weights: E2M1 elements, one E4M3 scale per 16-element block,
 *     one FP32 global scale (Korean summary, section 2.4 NVFP4 Training); the
 *     Ultra release ships NVFP4 routed experts (Ultra release news, quantization).
 *   - FP8 (OCP E4M3) weights and activations: FP8 post-training quantisation of
 *     weights and activations (Nemotron 3 Nano blog, FP8 quantisation section);
 *     FP8 shared experts beside NVFP4 routed ones (Ultra release news).
 * Readings taken where the pages are silent: the router is one linear layer
 * (fp32, optional bias) on the latent, or on x at d when router_on_x is set (the
 * Korean summary's LatentMoE section keeps routing and the shared experts at
 * full width); gates are the softmax over the K selected
 * logits; the expert FFN is W2 * sqrelu(W1 * z) with sqrelu(h) = max(h,0)^2 and
 * no biases; equal logits select the lower expert id; routing is dropless.
 *
 * Conventions
 *   - Row-major everywhere; weights are [out][in] (reduction dim contiguous).
 *   - All tensor pointers are DEVICE pointers, owned by the caller, 16-byte
 *     aligned.  The library never allocates or frees device memory.  Weights
 *     must outlive the handle.
 *   - Work is enqueued on the caller's HIP stream (a hipStream_t passed as
 *     void*, NULL = the null stream).  Calls return right after enqueueing; no
 *     call synchronises the host.  Faults during execution surface at the
 *     caller's next synchronisation, as the HIP runtime reports them.
 *   - Errors are integer status codes; every argument check runs on the host
 *     before any launch, so a failing call enqueues nothing.
 *   - A handle is immutable after moe_init and may be used from several host
 *     threads; concurrent calls need distinct workspaces.  It belongs to the
 *     device that was current at moe_init: moe_route / moe_forward return
 *     MOE_ERR_INVALID_ARG when another device is current.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_handle* moe_handle_t;

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, K > N, T > max_tokens, misalignment */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but not implemented shape / dtype combination */
  MOE_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than moe_workspace_size() */
  MOE_ERR_NO_DEVICE = 4,     /* no HIP device visible */
  MOE_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_NVFP4 = 2, MOE_FP8 = 3 };

typedef struct {
  int32_t d;               /* hidden size                                   */
  int32_t latent;          /* latent size l (== d when has_latent_proj = 0) */
  int32_t n_experts;       /* N routed experts, 1..1024                     */
  int32_t top_k;           /* K active experts per token, 1..min(N, 64)     */
  int32_t ffn;             /* m, routed expert FFN width                    */
  int32_t n_shared;        /* S always-on shared experts (at d), may be 0   */
  int32_t shared_ffn;      /* shared expert FFN width                       */
  int32_t max_tokens;      /* largest T any call will pass                  */
  int32_t has_latent_proj; /* 1: LatentMoE; 0: standard MoE, latent == d    */
  int32_t act_dtype;       /* MOE_F32 or MOE_BF16: x, projections, y        */
  int32_t expert_dtype;    /* MOE_F32 (with act F32), MOE_BF16, MOE_NVFP4 or
                              MOE_FP8 (the last three with act BF16)          */
  int32_t router_on_x;     /* 0: the router reads the latent z (W_r [N][l]);
                              1: it reads x at d (W_r [N][d]), the router
                              placement of the Korean Nemotron 3 summary,
                              section 2.2 LatentMoE                           */
  int32_t shared_fp8;      /* 0: shared expert weights in the act dtype;
                              1: FP8 E4M3 (act BF16, n_shared > 0)            */
} moe_config_t;

typedef struct {
  const void* w_down;      /* [l][d] act dtype; NULL unless has_latent_proj          */
  const float* w_router;   /* [N][l] fp32 ([N][d] when router_on_x)                  */
  const float* b_router;   /* [N] fp32 added to the logits before top-K, or NULL     */
  const void* w1;          /* [N][m][l]; NVFP4: codes uint8, k-tiled [N][l/64][m][32];
                              FP8: E4M3 codes uint8 [N][m][l]                  */
  const void* w2;          /* [N][l][m]; NVFP4: codes uint8, k-tiled [N][m/64][l][32];
                              FP8: E4M3 codes uint8 [N][l][m]                  */
  const uint8_t* w1_scale; /* NVFP4 only: E4M3 bytes, k-tiled [N][l/64][m][4], else NULL */
  const uint8_t* w2_scale; /* NVFP4 only: E4M3 bytes, k-tiled [N][m/64][l][4], else NULL */
  const float* w1_gscale;  /* NVFP4: [N] fp32 global scales; FP8: [N] fp32 per-matrix
                              weight scales; else NULL                          */
  const float* w2_gscale;  /* as w1_gscale, for W2                                  */
  const void* w_up;        /* [d][l] act dtype; NULL unless has_latent_proj          */
  const void* ws1;         /* [S][shared_ffn][d] act dtype (E4M3 codes if shared_fp8),
                              NULL if S == 0                                    */
  const void* ws2;         /* [S][d][shared_ffn] act dtype (E4M3 codes if shared_fp8),
                              NULL if S == 0                                    */
  const float* act_scale;  /* FP8 experts: [2] fp32, the per-tensor scales of the
                              expert inputs z (W1's) and h (W2's); else NULL   */
  const float* ws1_scale;  /* shared_fp8: [1] fp32 weight scale of all of ws1     */
  const float* ws2_scale;  /* shared_fp8: [1] fp32 weight scale of all of ws2     */
  const float* shared_act_scale; /* shared_fp8: [2] fp32 per-tensor scales of x and
                              of the shared hidden activations; else NULL     */
} moe_weights_t;
/* NVFP4 packing: w = e2m1(code) * e4m3(scale) * gscale[expert], one E4M3
 * scale per block of 16 elements along the reduction dimension.  The weights
 * are k-tiled: a matrix of R rows (output features) and reduction length Kr
 * is stored as Kr/64 slabs; slab t holds, for each row r in order, 32 code
 * bytes and, in the scale array, 4 scale bytes (byte b: block 4t+b, elements
 * 64t+16b .. 64t+16b+15).  Code bytes 16h+4i .. 16h+4i+3 (h = 0, 1; i =
 * 0..3) hold elements 64t+16i+8h .. 64t+16i+8h+7, two per byte, the lower
 * element in the low nibble.  moe_nvfp4_tile converts row-major codes (byte j
 * of a row: elements 2j, low nibble, and 2j+1) and scales to this layout.
 * FP8 (OCP E4M3: bias 7, no infinities, 448 the largest finite value, S.1111.111
 * NaN): a weight is e4m3(code) * its matrix scale.  An FP8 GEMM input v with
 * per-tensor scale a is quantised as code = RNE_e4m3(clamp(fp32(v) * r, -448,
 * 448)), r = 1/a as a correctly rounded fp32, and stands for a * e4m3(code).
 * The S shared experts form one FFN of width S * shared_ffn, hence one scale
 * per shared weight tensor.  Scale pointers are device pointers, 4-byte aligned. */

/* Create a handle for one layer.  Host only: validates the configuration and
 * weight pointers, binds the caller-owned weights, reads the current device's
 * compute-unit count.  No device work.
 * Shape rules: d, l, m, shared_ffn multiples of 64; N <= 1024; K <= min(N, 64);
 * act F32 requires expert F32; act BF16 requires expert BF16, NVFP4 or FP8.
 * FP8 experts: l and m multiples of 128 and at least 256.  shared_fp8: d and
 * shared_ffn multiples of 128, d and n_shared * shared_ffn at least 256.
 * Every activation matrix of a call (up to max_tokens * top_k rows) and every
 * weight matrix must be smaller than 4 GiB (the GEMMs use 32-bit byte offsets).
 * Outside these rules the call returns MOE_ERR_UNSUPPORTED.
 * Returns MOE_ERR_NO_DEVICE when no HIP device is visible. */
int moe_init(const moe_config_t* cfg, const moe_weights_t* w, moe_handle_t* out);

/* Bytes of device workspace a call with T tokens needs (T <= max_tokens). */
int moe_workspace_size(moe_handle_t h, int32_t T, size_t* bytes);

/* Routing only: down-projection (if latent), router GEMV, top-K + softmax and
 * the per-expert histogram.  Writes idx [T][K] int32 (per token in descending
 * logit order, equal logits -> lower id), gate [T][K] fp32 (softmax over the
 * K selected logits, gate[t][k] pairs with idx[t][k]) and counts [N] int32.
 * x is [T][d] in the act dtype.  T == 0 returns MOE_OK and enqueues nothing. */
int moe_route(moe_handle_t h, const void* x, int32_t T, int32_t* idx, float* gate,
              int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/* The whole layer: y [T][d] (act dtype) = LatentMoE(x).  idx/gate/counts are
 * optional outputs (each may be NULL) with the same meaning and exactly the
 * same values as moe_route's.  Deterministic: the same inputs give bitwise
 * the same outputs (no floating-point atomics; fixed summation orders). */
int moe_forward(moe_handle_t h, const void* x, int32_t T, void* y, int32_t* idx, float* gate,
                int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the whole
 * layer exactly as moe_forward (same kernels, bitwise the same outputs), with
 * the workspace taken from the library's own device array of
 * MOE_SCRATCH_BYTES bytes instead of a caller buffer.  Each GPU the library
 * runs on holds one such array from the first moe_init on that device until the
 * process ends; the call allocates and frees nothing and records no stage
 * timer events.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (each call initialises what it reads), so calls that overlap
 * on one GPU (several streams, host threads or handles) race: serialise them.
 * Returns MOE_ERR_WORKSPACE when moe_workspace_size(h, T) exceeds
 * MOE_SCRATCH_BYTES (decode batches fit: e.g. T = 128 at d = 8192, l = m =
 * 2048, 512 experts, top-22 needs about 33 MB), else as moe_forward. */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(moe_handle_t h, const void* x, int32_t T, void* y, int32_t* idx, float* gate,
                        int32_t* counts, void* stream);

/* Quantise n bf16 values (device, 16-byte aligned) to OCP FP8 E4M3 codes
 * (device, 16-byte aligned) with the per-tensor scale *scale (device fp32):
 * the FP8 input rule above.  For callers preparing FP8 weights or activations.
 * n must be a multiple of 16; n == 0 enqueues nothing.  Enqueued on `stream`. */
int moe_quantize_fp8(const void* in, int64_t n, const float* scale, uint8_t* out, void* stream);

/* Convert NVFP4 weights of n_mats matrices of `rows` rows and reduction length
 * k from row-major codes [n_mats][rows][k/2] and scales [n_mats][rows][k/16]
 * (device) to the k-tiled layout above (device, caller-allocated, same sizes).
 * A byte permutation run once when weights are loaded (NVFP4 format: E2M1
 * elements, E4M3 block scales of 16; Korean Nemotron 3 summary, section 2.4
 * NVFP4 Training).  k must be a multiple of 64 and rows >= 1; all four
 * pointers 16-byte aligned, the outputs overlapping neither input nor each
 * other (MOE_ERR_INVALID_ARG otherwise).  n_mats == 0 enqueues nothing.
 * Enqueued on `stream`. */
int moe_nvfp4_tile(const uint8_t* codes, const uint8_t* scales, uint8_t* codes_tiled,
                   uint8_t* scales_tiled, int64_t n_mats, int32_t rows, int32_t k, void* stream);

/* Release a handle (host memory only).  NULL is accepted. */
int moe_destroy(moe_handle_t h);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* ---- stage timing (benchmarks; off by default) ----
 * Stages of one call, in launch order (QUANT, numbered last, runs before
 * EXPERT_UP).  EXPERT_UP and EXPERT_DOWN are the two
 * grouped expert GEMMs; SHARED covers both shared-expert GEMMs (and the FP8
 * quantisation of their input); QUANT is the FP8 quantisation of x for FP8
 * routed experts of a layer without latent projection.  EXPERT_UP_REM and
 * EXPERT_DOWN_REM are recorded only in the phase-split mode below. */
enum moe_stage {
  MOE_STAGE_DOWN_PROJ = 0, MOE_STAGE_ROUTER, MOE_STAGE_TOPK, MOE_STAGE_SCAN,
  MOE_STAGE_SCATTER, MOE_STAGE_EXPERT_UP, MOE_STAGE_EXPERT_DOWN, MOE_STAGE_SHARED,
  MOE_STAGE_COMBINE, MOE_STAGE_UP_PROJ, MOE_STAGE_QUANT, MOE_STAGE_EXPERT_UP_REM,
  MOE_STAGE_EXPERT_DOWN_REM, MOE_NUM_STAGES
};

/* enable = 1: later moe_route / moe_forward calls record a HIP event pair
 * around each stage on the caller's stream (process-wide setting; the events
 * are host-side objects, no device memory is allocated).  enable = 2 also
 * splits each tiled grouped expert GEMM into two launches of the same kernel,
 * the full row tiles (timed as EXPERT_UP / EXPERT_DOWN) and then the
 * remainder tiles of each expert's last rows (EXPERT_UP_REM /
 * EXPERT_DOWN_REM): a measurement mode with the same results, a few percent
 * slower than the single launch.  enable = 0 stops recording.  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG for another value, or MOE_ERR_HIP if an event cannot be
 * created. */
int moe_profile_enable(int enable);

/* Waits for every recorded event, then writes per stage the number of
 * recorded launches (launches[MOE_NUM_STAGES]) and their summed durations in
 * milliseconds (ms[MOE_NUM_STAGES]), and clears the record.  Either pointer
 * may be NULL. */
int moe_profile_read(int32_t* launches, double* ms);

/* Static name of a stage ("expert_up", ...), or "unknown". */
const char* moe_stage_name(int stage);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
