// Host side of libmoe.so: argument validation, the workspace layout, and the
// launch sequence of the LatentMoE layer forward on the caller's stream.
//
// Dataflow (Korean Nemotron 3 summary, section 2.2 LatentMoE; notes.yuuk.io
// Nemotron 3 note, method 2): x --(W_d, d->l)--> z --router--> top-K, gates
// --> expert FFNs in l (grouped GEMMs over expert-sorted rows) --> gate-weighted
// combine --(W_u, l->d)--> y.  A standard MoE (l = d) skips both projections;
// shared experts run on x at d and are added to y (Nemotron 3 Nano blog,
// granular MoE section).  No call synchronises the host; data-dependent
// per-expert sizes stay on the device (tile list, counts, offsets).
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/moe.h"
#include "common.h"

using namespace moe;

struct moe_handle {
  moe_config_t c;
  moe_weights_t w;
  int device;
  int num_cu;
  void* scratch;     // this device's copy of `scratch` (device address)
};

// Workspace of moe_forward_noalloc: a file-scope device array, one copy per GPU
// (allocated when the library's code object is loaded on that device and held
// until the process ends).  Host code never uses its name as an address: the
// name is a host-side stand-in; each device's address comes from
// hipGetSymbolAddress, taken once per device at moe_init.
static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

namespace {

constexpr int kTokensPerChunk = 32;   // routing chunk: one histogram row / one scatter wavefront
constexpr int kF32BM = 64;            // fp32 GEMM row-tile height
constexpr int kSmallBM = 64;          // grouped bf16 GEMM: height of each expert's remainder tiles
constexpr int kSmallBM256 = 128;      // ... when the full tiles are 256 rows high
constexpr int kSkinnyMaxT = 128;      // batches up to this many tokens -> skinny path
// split-K partial buffer: floats per CU (two blocks of 64 x 64 outputs)
constexpr size_t kPartialPerCu = 2 * 64 * 64;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// ---- optional stage timing: a HIP event pair around each stage ----
// moe_forward_noalloc records no stage events (event creation is a host-side
// allocation the no-allocation entry point avoids)
thread_local bool tls_no_stage_events = false;
struct Prof {
  std::mutex mu;
  bool on = false;
  bool split = false;        // grouped expert GEMMs as two launches, one per tile list
  struct Rec { int stage; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  int64_t launches[MOE_NUM_STAGES] = {};
  double ms[MOE_NUM_STAGES] = {};
};
Prof& prof() {
  static Prof* p = new Prof;   // never destroyed: safe at process exit
  return *p;
}
hipEvent_t prof_event() {
  Prof& P = prof();
  if (!P.pool.empty()) {
    hipEvent_t e = P.pool.back();
    P.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
// The phase-split timing mode (moe_profile_enable(2)) is on.
bool prof_split() {
  if (tls_no_stage_events) return false;
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  return P.on && P.split;
}
// Records the start of a stage; returns the index of its record or -1.
int prof_begin(int stage, hipStream_t s) {
  if (tls_no_stage_events) return -1;
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (!P.on) return -1;
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b || hipEventRecord(a, s) != hipSuccess) {   // no record for this stage
    if (a) P.pool.push_back(a);
    if (b) P.pool.push_back(b);
    return -1;
  }
  P.pending.push_back({stage, a, b});
  return (int)P.pending.size() - 1;
}
void prof_end(int rec, hipStream_t s) {
  if (rec < 0) return;
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  // a failed end record surfaces as a failed elapsed-time query in moe_profile_read
  if (rec < (int)P.pending.size()) (void)hipEventRecord(P.pending[rec].b, s);
}
struct StageScope {
  int rec;
  hipStream_t s;
  StageScope(int stage, hipStream_t st) : rec(prof_begin(stage, st)), s(st) {}
  ~StageScope() { prof_end(rec, s); }
  void end() {   // ends the stage before the scope does
    prof_end(rec, s);
    rec = -1;
  }
};
size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// Device address of `scratch` on device `dev` (the current device), looked up
// once per device.
constexpr int kMaxDevices = 64;
struct ScratchTable {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
ScratchTable& scratch_table() {
  static ScratchTable* t = new ScratchTable;   // never destroyed: safe at process exit
  return *t;
}
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchTable& T = scratch_table();
  std::lock_guard<std::mutex> g(T.mu);
  if (!T.ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    T.ptr[dev] = p;
  }
  *out = T.ptr[dev];
  return hipSuccess;
}

struct Plan {
  size_t z32, z16, z8, logits, idx, gate, ccount, cbase, counts, offs, tiles, tiles2, ntiles;
  size_t slot_token, tk_slot, H, O, u, x8, Hs, ys, partial, total;
  int nchunks, bm, bms, max_tiles, max_tiles2;
  bool f32, skinny;
  bool fp8;        // FP8 routed experts: E4M3 latent rows z8 and hidden rows H
  bool sfp8;       // FP8 shared experts: E4M3 x8 and hidden rows Hs
};

bool use_f32(const moe_config_t& c) { return c.act_dtype == MOE_F32; }

// weight storage of the routed experts' GEMMs
int expert_wt(const moe_config_t& c) {
  return c.expert_dtype == MOE_NVFP4 ? WT_NVFP4 : c.expert_dtype == MOE_FP8 ? WT_FP8 : WT_BF16;
}

bool use_skinny(const moe_config_t& c, int T) {
  return !use_f32(c) && T <= kSkinnyMaxT && c.latent % 256 == 0 && c.ffn % 256 == 0;
}

Plan make_plan(const moe_config_t& c, int T, int num_cu) {
  Plan p;
  memset(&p, 0, sizeof(p));
  const size_t Tz = (size_t)T, N = (size_t)c.n_experts, K = (size_t)c.top_k;
  const size_t L = (size_t)c.latent, M = (size_t)c.ffn, D = (size_t)c.d;
  p.f32 = use_f32(c);
  p.skinny = use_skinny(c, T);
  p.fp8 = c.expert_dtype == MOE_FP8;
  p.sfp8 = c.n_shared > 0 && c.shared_fp8;
  const size_t es = p.f32 ? 4 : 2;
  const size_t esh = p.fp8 ? 1 : es;                 // expert hidden rows H
  const size_t ess = p.sfp8 ? 1 : es;                // shared hidden rows Hs
  p.nchunks = (T + kTokensPerChunk - 1) / kTokensPerChunk;
  if (p.f32) {
    p.bm = kF32BM;
    p.bms = 0;
    p.max_tiles = (int)(N + (Tz * K + p.bm - 1) / p.bm);
    p.max_tiles2 = 0;
  } else if (Tz * K >= 64 * N) {
    // prefill with at least 64 rows per expert on average: full 256-row
    // tiles, each expert's remaining rows in one 128-row tile or, past 128
    // rows, in one partial 256-row tile.  (Sending the cold experts to the
    // skinny kernel instead, with a 64- or 256-row cutoff, measured no faster
    // on MI355X.)  Every expert adds at most one partial tile to list 0.
    p.bm = 256;
    p.bms = kSmallBM256;
    p.max_tiles = (int)((Tz * K) / p.bm + N);
    p.max_tiles2 = (int)std::min<size_t>(N * (size_t)(p.bm / p.bms), N + (Tz * K + p.bms - 1) / p.bms);
  } else {
    // smaller batches: full 128-row tiles plus one 64-row tile or one
    // partial 128-row tile for each expert's remainder
    p.bm = 128;
    p.bms = kSmallBM;
    p.max_tiles = (int)((Tz * K) / p.bm + N);
    p.max_tiles2 = (int)std::min<size_t>(N * (size_t)(p.bm / p.bms), N + (Tz * K + p.bms - 1) / p.bms);
  }
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up256(bytes); return at; };
  // z32 feeds the router (unless it reads x); z16 or z8 the experts
  p.z32 = take(c.has_latent_proj && (p.f32 || !c.router_on_x) ? Tz * L * 4 : 0);
  p.z16 = take(c.has_latent_proj && !p.f32 && !p.fp8 ? Tz * L * 2 : 0);
  p.z8 = take(p.fp8 ? Tz * L : 0);
  p.logits = take(Tz * N * 4);
  p.idx = take(Tz * K * 4);
  p.gate = take(Tz * K * 4);
  p.ccount = take((size_t)p.nchunks * N * 4);
  p.cbase = take((size_t)p.nchunks * N * 4);
  p.counts = take(N * 4);
  p.offs = take((N + 1) * 4);
  p.tiles = take((size_t)p.max_tiles * 16);
  p.tiles2 = take((size_t)p.max_tiles2 * 16);
  p.ntiles = take(8);
  // 64 bytes past the end: the tiled GEMM reads a tile's row indices in
  // aligned groups of up to 16 with scalar loads and discards those past the tile
  p.slot_token = take(Tz * K * 4 + 64);
  p.tk_slot = take(Tz * K * 4);
  p.H = take(Tz * K * M * esh);
  p.O = take(Tz * K * L * es);
  p.u = take(c.has_latent_proj ? Tz * L * es : 0);
  p.x8 = take(p.sfp8 ? Tz * D : 0);
  p.Hs = take(c.n_shared ? Tz * (size_t)c.n_shared * c.shared_ffn * ess : 0);
  p.ys = take(c.n_shared ? Tz * D * 4 : 0);
  // split-K partial sums of the dense GEMMs whose output tiles cannot fill the
  // device (small batches); the split factors keep them within this bound
  p.partial = take(kPartialPerCu * (size_t)num_cu * 4);
  p.total = o;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>((char*)ws + off); }

// Dense bf16 GEMM tile shape: the largest tile that still gives every CU work.
void dense_shape(int M, int N, int num_cu, int* bm, int* bn) {
  auto tiles = [&](int a, int b) { return (int64_t)((M + a - 1) / a) * ((N + b - 1) / b); };
  if (tiles(256, 256) >= num_cu) { *bm = 256; *bn = 256; }
  else if (tiles(256, 128) >= num_cu) { *bm = 256; *bn = 128; }
  else { *bm = 128; *bn = 128; }
}

// K-split factor for an output of `tiles` tiles: the largest power of two
// that keeps tiles * ks within two blocks per CU, with K divisible by
// kstep * ks and slices of at least min_slice.  1 when the tiles alone fill
// the device.  tiles * ks <= 2 * num_cu bounds the partial sums.
int split_factor(int64_t tiles, int K, int kstep, int min_slice, int num_cu) {
  if (tiles >= num_cu) return 1;
  int ks = 1;
  while (tiles * ks * 2 <= 2 * (int64_t)num_cu && K % (kstep * ks * 2) == 0 && K / (ks * 2) >= min_slice)
    ks *= 2;
  return ks;
}

// Dense bf16 GEMM.  Small batches (M <= 64, or M <= 256 when the output has
// fewer than num_cu / 8 tiles of 128 x 128) run on the skinny kernel with K
// split across blocks (weights streamed by every CU); larger ones on the
// largest tile that still gives every CU work.
// fp8: A and B are E4M3 codes (the shared experts of an FP8 layer).
hipError_t dense_bf16(const GemmArgs& a, int epi, int num_cu, float* P, hipStream_t s,
                      bool fp8 = false) {
  const int64_t t128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
  if ((a.M <= 64 || (a.M <= 256 && t128 * 8 < num_cu)) && a.N % 64 == 0 && a.K % 256 == 0 &&
      a.kseg >= a.K) {
    const int ks = split_factor((int64_t)(a.N / 64) * ((a.M + 63) / 64), a.K, 256, 256, num_cu);
    if ((size_t)ks * a.M * a.N <= kPartialPerCu * (size_t)num_cu)   // always, unless N is huge
      return launch_skinny_splitk(a, fp8, epi, ks, P, s);
  }
  int bm, bn;
  dense_shape(a.M, a.N, num_cu, &bm, &bn);
  return launch_gemm_bf16(a, fp8 ? WT_FP8 : WT_BF16, epi, bm, bn, 0, 0, num_cu, s);
}

// Dense fp32 GEMM (the router, and every dense GEMM of an all-fp32 layer),
// K split across blocks when its 64 x 64 output tiles cannot fill the device.
hipError_t dense_f32(const GemmArgs& a, bool a_bf16, int epi, int num_cu, float* P, hipStream_t s) {
  const int64_t tiles = (int64_t)((a.M + 63) / 64) * ((a.N + 63) / 64);
  const int ks = a.kseg >= a.K ? split_factor(tiles, a.K, 32, 64, num_cu) : 1;
  if (ks > 1) return launch_gemm_f32_splitk(a, a_bf16, epi, ks, P, s);
  return launch_gemm_f32(a, a_bf16, epi, num_cu * 2, s);
}

GemmArgs gemm_args() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.kseg = 1 << 30;
  a.lists = 3;
  return a;
}

int check_call(moe_handle_t h, const void* x, int32_t T, void* ws, size_t ws_bytes) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (T < 0 || T > h->c.max_tokens) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  int dev = -1;                            // the handle's weights live on its device
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev != h->device) return MOE_ERR_INVALID_ARG;
  if (!x || !aligned16(x)) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(h->c, T, h->num_cu);
  if (!ws || ws_bytes < p.total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

#define MOE_TRY(expr)                       \
  do {                                      \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// Down-projection + router + top-K + bookkeeping.  Shared by route and forward.
int enqueue_routing(moe_handle_t h, const void* x, int T, void* ws, const Plan& p, hipStream_t s) {
  const moe_config_t& c = h->c;
  const moe_weights_t& w = h->w;
  if (c.has_latent_proj) {
    StageScope sc(MOE_STAGE_DOWN_PROJ, s);
    GemmArgs a = gemm_args();
    a.A = x; a.lda = c.d;
    a.B = w.w_down; a.ldb = c.d;
    a.M = T; a.N = c.latent; a.K = c.d;
    a.C = at<void>(ws, p.z32); a.ldc = c.latent;
    if (p.f32) {
      MOE_TRY(dense_f32(a, false, EPI_F32, h->num_cu, at<float>(ws, p.partial), s));
    } else if (p.fp8) {
      // the experts read E4M3 latent rows quantised with their input scale
      a.q_scale = w.act_scale;
      if (c.router_on_x) {
        a.C = at<void>(ws, p.z8);
        MOE_TRY(dense_bf16(a, EPI_Q8, h->num_cu, at<float>(ws, p.partial), s));
      } else {
        a.C2 = at<void>(ws, p.z8); a.ldc2 = c.latent;
        MOE_TRY(dense_bf16(a, EPI_Z8, h->num_cu, at<float>(ws, p.partial), s));
      }
    } else if (c.router_on_x) {
      // the router reads x, so only the experts' bf16 latent rows are needed
      a.C = at<void>(ws, p.z16);
      MOE_TRY(dense_bf16(a, EPI_BF16, h->num_cu, at<float>(ws, p.partial), s));
    } else {
      a.C2 = at<void>(ws, p.z16); a.ldc2 = c.latent;
      MOE_TRY(dense_bf16(a, EPI_Z, h->num_cu, at<float>(ws, p.partial), s));
    }
  }
  {
    StageScope sc(MOE_STAGE_ROUTER, s);
    GemmArgs a = gemm_args();
    // the router's input: the fp32 latent z32, or x at d (also when there is
    // no latent projection)
    const bool on_x = c.router_on_x || !c.has_latent_proj;
    const int kr = on_x ? c.d : c.latent;
    a.A = on_x ? x : (const void*)at<float>(ws, p.z32);
    a.lda = kr;
    a.B = w.w_router; a.ldb = kr;
    a.M = T; a.N = c.n_experts; a.K = kr;
    a.C = at<float>(ws, p.logits); a.ldc = c.n_experts;
    a.bias = w.b_router;
    const bool a_bf16 = on_x && c.act_dtype == MOE_BF16;
    MOE_TRY(dense_f32(a, a_bf16, EPI_F32, h->num_cu, at<float>(ws, p.partial), s));
  }
  {
    StageScope sc(MOE_STAGE_TOPK, s);
    MOE_TRY(launch_topk(at<float>(ws, p.logits), T, c.n_experts, c.top_k, kTokensPerChunk,
                        at<int>(ws, p.idx), at<float>(ws, p.gate), at<int>(ws, p.ccount), s));
  }
  StageScope sc(MOE_STAGE_SCAN, s);
  MOE_TRY(launch_scan(at<int>(ws, p.ccount), p.nchunks, c.n_experts, p.bm, p.bms,
                      at<int>(ws, p.cbase), at<int>(ws, p.counts), at<int>(ws, p.offs),
                      at<int4>(ws, p.tiles), at<int4>(ws, p.tiles2), at<int>(ws, p.ntiles), s));
  return MOE_OK;
}

int copy_out(moe_handle_t h, int T, const void* ws, const Plan& p, int32_t* idx, float* gate,
             int32_t* counts, hipStream_t s) {
  const size_t tk = (size_t)T * h->c.top_k;
  if (idx) MOE_TRY(hipMemcpyAsync(idx, (const char*)ws + p.idx, tk * 4, hipMemcpyDeviceToDevice, s));
  if (gate) MOE_TRY(hipMemcpyAsync(gate, (const char*)ws + p.gate, tk * 4, hipMemcpyDeviceToDevice, s));
  if (counts)
    MOE_TRY(hipMemcpyAsync(counts, (const char*)ws + p.counts, (size_t)h->c.n_experts * 4,
                           hipMemcpyDeviceToDevice, s));
  return MOE_OK;
}

// One grouped expert GEMM (up: sqrelu epilogue; down: plain, gates are applied by
// the combine).  FP8: the up GEMM writes E4M3 hidden rows quantised with the
// down GEMM's input scale.
int enqueue_expert_gemm(moe_handle_t h, const Plan& p, void* ws, bool up, const void* A,
                        const int* a_rows, void* C, hipStream_t s) {
  const moe_config_t& c = h->c;
  const moe_weights_t& w = h->w;
  const int64_t rows = up ? c.ffn : c.latent;     // output columns
  const int64_t kdim = up ? c.latent : c.ffn;     // reduction
  const int wt = expert_wt(c);
  const bool fp4 = wt == WT_NVFP4, fp8 = wt == WT_FP8;
  const void* B = up ? w.w1 : w.w2;
  const uint8_t* S = up ? w.w1_scale : w.w2_scale;
  const float* G = (fp4 || fp8) ? (up ? w.w1_gscale : w.w2_gscale) : nullptr;
  const float* as = fp8 ? w.act_scale + (up ? 0 : 1) : nullptr;   // scale of this GEMM's input
  const float* qs = fp8 && up ? w.act_scale + 1 : nullptr;        // scale of its E4M3 output
  const int cap = h->num_cu * 2;
  StageScope sc(up ? MOE_STAGE_EXPERT_UP : MOE_STAGE_EXPERT_DOWN, s);
  SkinnyArgs sk;
  memset(&sk, 0, sizeof(sk));
  sk.A = (const uint16_t*)A; sk.lda = kdim; sk.a_rows = a_rows;
  sk.B = B;
  // NVFP4 (k-tiled): ldb and lds_scale are the byte strides of one 64-deep k-slab
  sk.ldb = fp4 ? rows * 32 : kdim;
  sk.b_gstride = fp4 ? rows * kdim / 2 : rows * kdim;
  sk.b_scale = S; sk.lds_scale = rows * 4; sk.s_gstride = rows * kdim / 16;
  sk.b_gscale = G; sk.a_scale = as; sk.q_scale = qs;
  sk.N = (int)rows; sk.K = (int)kdim;
  sk.counts = at<int>(ws, p.counts); sk.offs = at<int>(ws, p.offs);
  sk.C = C; sk.ldc = rows;
  const int epi = up ? (fp8 ? EPI_SQRELU_Q8 : EPI_SQRELU_BF16) : EPI_BF16;
  if (p.skinny) {
    MOE_TRY(launch_skinny(sk, wt, epi, c.n_experts, s));
    return MOE_OK;
  }
  GemmArgs a = gemm_args();
  a.A = A; a.lda = kdim; a.a_rows = a_rows;
  a.B = B;
  a.ldb = fp4 ? rows * 32 : kdim;
  a.b_gstride = fp4 ? rows * kdim / 2 : rows * kdim;
  a.b_scale = S; a.lds_scale = rows * 4; a.s_gstride = rows * kdim / 16;
  a.b_gscale = G; a.a_scale = as; a.q_scale = qs;
  a.N = (int)rows; a.K = (int)kdim;
  a.tiles = at<int4>(ws, p.tiles); a.n_tiles = at<int>(ws, p.ntiles);
  a.tiles2 = at<int4>(ws, p.tiles2);
  a.C = C; a.ldc = rows;
  if (p.f32) {
    a.M = p.max_tiles;   // grouped: upper bound on row tiles (grid sizing)
    MOE_TRY(launch_gemm_f32(a, false, up ? EPI_SQRELU_F32 : EPI_F32, cap, s));
    return MOE_OK;
  }
  const int bn = p.bm == 256 ? 256 : 128;
  const int64_t ntn = (rows + bn - 1) / bn;
  const int64_t items = (int64_t)(p.max_tiles + p.max_tiles2) * ntn;
  // NVFP4 weights on the 256-row plan: the remainder tiles get a launch of
  // their own (two blocks per CU), after the full row tiles
  const bool fp4_rem = wt == WT_NVFP4 && p.bm == 256 && p.bms == 128;
  if (p.bms > 0 && (prof_split() || fp4_rem)) {
    // phase-split timing also runs the two lists as two launches, timed apart
    // (for other weights both on the grouped kernel; same results either way)
    a.lists = 1;
    MOE_TRY(launch_gemm_bf16(a, wt, epi, p.bm, bn, p.bms, items, h->num_cu, s));
    a.lists = 2;
    const int64_t items2 = (int64_t)p.max_tiles2 * ntn;
    if (prof_split()) {
      sc.end();
      StageScope rem(up ? MOE_STAGE_EXPERT_UP_REM : MOE_STAGE_EXPERT_DOWN_REM, s);
      if (fp4_rem) MOE_TRY(launch_gemm_fp4_rem(a, epi, items2, h->num_cu, s));
      else MOE_TRY(launch_gemm_bf16(a, wt, epi, p.bm, bn, p.bms, items, h->num_cu, s));
    } else {
      MOE_TRY(launch_gemm_fp4_rem(a, epi, items2, h->num_cu, s));
    }
    return MOE_OK;
  }
  MOE_TRY(launch_gemm_bf16(a, wt, epi, p.bm, bn, p.bms, items, h->num_cu, s));
  return MOE_OK;
}

int forward_impl(moe_handle_t h, const void* x, int32_t T, void* y, int32_t* idx, float* gate,
                 int32_t* counts, void* ws, size_t ws_bytes, void* stream);

}  // namespace

extern "C" {

const char* moe_status_string(int st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported shape or dtype combination";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_NO_DEVICE: return "MOE_ERR_NO_DEVICE: no HIP device visible";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime call or kernel launch failed";
    default: return "unknown moe status";
  }
}

int moe_init(const moe_config_t* cfg, const moe_weights_t* w, moe_handle_t* out) {
  if (!cfg || !w || !out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  const moe_config_t& c = *cfg;
  if (c.d <= 0 || c.latent <= 0 || c.ffn <= 0 || c.max_tokens <= 0) return MOE_ERR_INVALID_ARG;
  if (c.n_experts < 1 || c.top_k < 1 || c.top_k > c.n_experts) return MOE_ERR_INVALID_ARG;
  if (c.n_shared < 0 || (c.n_shared > 0 && c.shared_ffn <= 0)) return MOE_ERR_INVALID_ARG;
  if (c.has_latent_proj != 0 && c.has_latent_proj != 1) return MOE_ERR_INVALID_ARG;
  if (c.router_on_x != 0 && c.router_on_x != 1) return MOE_ERR_INVALID_ARG;
  if (!c.has_latent_proj && c.latent != c.d) return MOE_ERR_INVALID_ARG;
  if ((int64_t)c.max_tokens * c.top_k > (1 << 30)) return MOE_ERR_INVALID_ARG;
  if (c.act_dtype != MOE_F32 && c.act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c.expert_dtype != MOE_F32 && c.expert_dtype != MOE_BF16 && c.expert_dtype != MOE_NVFP4 &&
      c.expert_dtype != MOE_FP8)
    return MOE_ERR_INVALID_ARG;
  if (c.shared_fp8 != 0 && c.shared_fp8 != 1) return MOE_ERR_INVALID_ARG;
  if (c.shared_fp8 && c.n_shared == 0) return MOE_ERR_INVALID_ARG;
  if (c.n_experts > 1024 || c.top_k > 64) return MOE_ERR_UNSUPPORTED;
  if (c.d % 64 || c.latent % 64 || c.ffn % 64 || (c.n_shared && c.shared_ffn % 64))
    return MOE_ERR_UNSUPPORTED;
  if ((c.act_dtype == MOE_F32) != (c.expert_dtype == MOE_F32)) return MOE_ERR_UNSUPPORTED;
  // FP8 GEMMs run whole 128-code k-tiles, at least two of them
  if (c.expert_dtype == MOE_FP8 && (c.latent % 128 || c.ffn % 128 || c.latent < 256 || c.ffn < 256))
    return MOE_ERR_UNSUPPORTED;
  if (c.shared_fp8 && (c.act_dtype != MOE_BF16 || c.d % 128 || c.shared_ffn % 128 || c.d < 256 ||
                       c.n_shared * c.shared_ffn < 256))
    return MOE_ERR_UNSUPPORTED;
  // the tiled GEMMs address each operand with 32-bit byte offsets from a
  // uniform base: every activation matrix (up to max_tokens * top_k rows) and
  // every weight matrix must stay below 4 GiB
  {
    const int64_t lim = (int64_t)1 << 32, es = c.act_dtype == MOE_F32 ? 4 : 2;
    const int64_t T = c.max_tokens, TK = (int64_t)c.max_tokens * c.top_k;
    const int64_t sw = (int64_t)c.n_shared * c.shared_ffn;
    const int64_t wide = std::max<int64_t>(std::max<int64_t>(c.d, c.latent), std::max<int64_t>(c.ffn, sw));
    if (TK * std::max(c.ffn, c.latent) * es >= lim || T * wide * es >= lim ||
        (int64_t)c.d * std::max<int64_t>(c.latent, sw) * es >= lim ||
        (int64_t)c.ffn * c.latent * es >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  // weights
  if (!w->w_router || !aligned16(w->w_router) || !w->w1 || !aligned16(w->w1) || !w->w2 ||
      !aligned16(w->w2))
    return MOE_ERR_INVALID_ARG;
  if (w->b_router && !aligned16(w->b_router)) return MOE_ERR_INVALID_ARG;
  if (c.has_latent_proj) {
    if (!w->w_down || !aligned16(w->w_down) || !w->w_up || !aligned16(w->w_up))
      return MOE_ERR_INVALID_ARG;
  }
  if (c.expert_dtype == MOE_NVFP4) {
    if (!w->w1_scale || !w->w2_scale || !w->w1_gscale || !w->w2_gscale ||
        !aligned16(w->w1_scale) || !aligned16(w->w2_scale))
      return MOE_ERR_INVALID_ARG;
  }
  if (c.expert_dtype == MOE_FP8) {
    if (!w->w1_gscale || !w->w2_gscale || !w->act_scale || !aligned4(w->w1_gscale) ||
        !aligned4(w->w2_gscale) || !aligned4(w->act_scale))
      return MOE_ERR_INVALID_ARG;
  }
  if (c.n_shared) {
    if (!w->ws1 || !aligned16(w->ws1) || !w->ws2 || !aligned16(w->ws2)) return MOE_ERR_INVALID_ARG;
  }
  if (c.shared_fp8) {
    if (!w->ws1_scale || !w->ws2_scale || !w->shared_act_scale || !aligned4(w->ws1_scale) ||
        !aligned4(w->ws2_scale) || !aligned4(w->shared_act_scale))
      return MOE_ERR_INVALID_ARG;
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return MOE_ERR_NO_DEVICE;
  }
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  void* sp = nullptr;
  if (scratch_address(dev, &sp) != hipSuccess) return MOE_ERR_HIP;
  moe_handle* h = new (std::nothrow) moe_handle;
  if (!h) return MOE_ERR_INVALID_ARG;
  h->c = c;
  h->w = *w;
  h->device = dev;
  h->num_cu = ncu > 0 ? ncu : 256;
  h->scratch = sp;
  *out = h;
  return MOE_OK;
}

int moe_workspace_size(moe_handle_t h, int32_t T, size_t* bytes) {
  if (!h || !bytes || T < 0 || T > h->c.max_tokens) return MOE_ERR_INVALID_ARG;
  *bytes = T == 0 ? 0 : make_plan(h->c, T, h->num_cu).total;
  return MOE_OK;
}

int moe_profile_enable(int enable) {
  if (enable < 0 || enable > 2) return MOE_ERR_INVALID_ARG;
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.on = enable != 0;
  P.split = enable == 2;
  return MOE_OK;
}

int moe_profile_read(int32_t* launches, double* ms) {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  int st = MOE_OK;
  for (auto& r : P.pending) {
    float t = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      st = MOE_ERR_HIP;
    } else {
      P.launches[r.stage] += 1;
      P.ms[r.stage] += t;
    }
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.pending.clear();
  for (int i = 0; i < MOE_NUM_STAGES; ++i) {
    if (launches) launches[i] = (int32_t)P.launches[i];
    if (ms) ms[i] = P.ms[i];
    P.launches[i] = 0;
    P.ms[i] = 0.0;
  }
  return st;
}

const char* moe_stage_name(int stage) {
  static const char* names[MOE_NUM_STAGES] = {"down_proj", "router", "topk", "scan", "scatter",
                                              "expert_up", "expert_down", "shared", "combine",
                                              "up_proj", "quant_x", "expert_up_rem", "expert_down_rem"};
  return (stage >= 0 && stage < MOE_NUM_STAGES) ? names[stage] : "unknown";
}

int moe_quantize_fp8(const void* in, int64_t n, const float* scale, uint8_t* out, void* stream) {
  if (n < 0 || n % 16 != 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!in || !out || !scale || !aligned16(in) || !aligned16(out) || !aligned4(scale))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_quant_fp8((const uint16_t*)in, n, scale, out, (hipStream_t)stream));
  return MOE_OK;
}

int moe_nvfp4_tile(const uint8_t* codes, const uint8_t* scales, uint8_t* codes_tiled,
                   uint8_t* scales_tiled, int64_t n_mats, int32_t rows, int32_t k, void* stream) {
  if (n_mats < 0 || rows < 1 || k < 64 || k % 64 != 0) return MOE_ERR_INVALID_ARG;
  if (n_mats == 0) return MOE_OK;
  if (!codes || !scales || !codes_tiled || !scales_tiled || !aligned16(codes) || !aligned16(scales) ||
      !aligned16(codes_tiled) || !aligned16(scales_tiled))
    return MOE_ERR_INVALID_ARG;
  // the outputs must not overlap the inputs
  const uintptr_t cb = (uintptr_t)n_mats * rows * (k / 2), sb = (uintptr_t)n_mats * rows * (k / 16);
  auto overlap = [](const void* a, uintptr_t an, const void* b, uintptr_t bn) {
    return (uintptr_t)a < (uintptr_t)b + bn && (uintptr_t)b < (uintptr_t)a + an;
  };
  if (overlap(codes, cb, codes_tiled, cb) || overlap(codes, cb, scales_tiled, sb) ||
      overlap(scales, sb, codes_tiled, cb) || overlap(scales, sb, scales_tiled, sb) ||
      overlap(codes_tiled, cb, scales_tiled, sb))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_nvfp4_tile(codes, scales, codes_tiled, scales_tiled, n_mats, rows, k,
                            (hipStream_t)stream));
  return MOE_OK;
}

int moe_destroy(moe_handle_t h) {
  delete h;
  return MOE_OK;
}

int moe_route(moe_handle_t h, const void* x, int32_t T, int32_t* idx, float* gate,
              int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  int st = check_call(h, x, T, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!idx || !gate || !counts || !aligned16(idx) || !aligned16(gate) || !aligned16(counts))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const Plan p = make_plan(h->c, T, h->num_cu);
  st = enqueue_routing(h, x, T, ws, p, s);
  if (st != MOE_OK) return st;
  return copy_out(h, T, ws, p, idx, gate, counts, s);
}

int moe_forward(moe_handle_t h, const void* x, int32_t T, void* y, int32_t* idx, float* gate,
                int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(h, x, T, y, idx, gate, counts, ws, ws_bytes, stream);
}

int moe_forward_noalloc(moe_handle_t h, const void* x, int32_t T, void* y, int32_t* idx,
                        float* gate, int32_t* counts, void* stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (T < 0 || T > h->c.max_tokens) return MOE_ERR_INVALID_ARG;
  if (T > 0 && make_plan(h->c, T, h->num_cu).total > MOE_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  tls_no_stage_events = true;
  const int st = forward_impl(h, x, T, y, idx, gate, counts, h->scratch, MOE_SCRATCH_BYTES, stream);
  tls_no_stage_events = false;
  return st;
}

}  // extern "C"

namespace {

int forward_impl(moe_handle_t h, const void* x, int32_t T, void* y, int32_t* idx, float* gate,
                 int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  int st = check_call(h, x, T, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!y || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if ((idx && !aligned16(idx)) || (gate && !aligned16(gate)) || (counts && !aligned16(counts)))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const moe_config_t& c = h->c;
  const moe_weights_t& w = h->w;
  const Plan p = make_plan(c, T, h->num_cu);
  st = enqueue_routing(h, x, T, ws, p, s);
  if (st != MOE_OK) return st;
  {
    StageScope sc(MOE_STAGE_SCATTER, s);
    MOE_TRY(launch_scatter(at<int>(ws, p.idx), T, c.top_k, c.n_experts, kTokensPerChunk,
                           at<int>(ws, p.cbase), at<int>(ws, p.offs), at<int>(ws, p.slot_token),
                           at<int>(ws, p.tk_slot), s));
  }
  // expert FFNs over expert-sorted rows
  if (p.fp8 && !c.has_latent_proj) {
    // no projection writes the experts' E4M3 input rows: quantise x
    StageScope sc(MOE_STAGE_QUANT, s);
    MOE_TRY(launch_quant_fp8((const uint16_t*)x, (int64_t)T * c.d, w.act_scale, at<uint8_t>(ws, p.z8), s));
  }
  const void* zsrc = p.fp8 ? (const void*)at<uint8_t>(ws, p.z8)
                     : c.has_latent_proj ? (p.f32 ? (const void*)at<float>(ws, p.z32)
                                                  : (const void*)at<uint16_t>(ws, p.z16))
                                         : x;
  st = enqueue_expert_gemm(h, p, ws, true, zsrc, at<int>(ws, p.slot_token), at<void>(ws, p.H), s);
  if (st != MOE_OK) return st;
  st = enqueue_expert_gemm(h, p, ws, false, at<void>(ws, p.H), nullptr, at<void>(ws, p.O), s);
  if (st != MOE_OK) return st;
  // shared experts at d: Hs = sqrelu(x Ws1^T), ys = Hs Ws2^T (fp32)
  const float* ys = nullptr;
  if (c.n_shared) {
    StageScope sc(MOE_STAGE_SHARED, s);
    const int sm = c.n_shared * c.shared_ffn;
    if (p.sfp8)
      MOE_TRY(launch_quant_fp8((const uint16_t*)x, (int64_t)T * c.d, w.shared_act_scale,
                               at<uint8_t>(ws, p.x8), s));
    GemmArgs a = gemm_args();
    a.A = p.sfp8 ? (const void*)at<uint8_t>(ws, p.x8) : x; a.lda = c.d;
    a.B = w.ws1; a.ldb = c.d;
    a.M = T; a.N = sm; a.K = c.d;
    a.C = at<void>(ws, p.Hs); a.ldc = sm;
    if (p.sfp8) { a.b_gscale = w.ws1_scale; a.a_scale = w.shared_act_scale; a.q_scale = w.shared_act_scale + 1; }
    if (p.f32) MOE_TRY(dense_f32(a, false, EPI_SQRELU_F32, h->num_cu, at<float>(ws, p.partial), s));
    else MOE_TRY(dense_bf16(a, p.sfp8 ? EPI_SQRELU_Q8 : EPI_SQRELU_BF16, h->num_cu,
                            at<float>(ws, p.partial), s, p.sfp8));
    GemmArgs b = gemm_args();
    b.A = at<void>(ws, p.Hs); b.lda = sm;
    b.B = w.ws2; b.ldb = c.shared_ffn;
    b.kseg = c.shared_ffn; b.b_segstride = (int64_t)c.d * c.shared_ffn;
    b.M = T; b.N = c.d; b.K = sm;
    b.C = at<float>(ws, p.ys); b.ldc = c.d;
    if (p.sfp8) { b.b_gscale = w.ws2_scale; b.a_scale = w.shared_act_scale + 1; }
    if (p.f32) MOE_TRY(dense_f32(b, false, EPI_F32, h->num_cu, at<float>(ws, p.partial), s));
    else MOE_TRY(dense_bf16(b, EPI_F32, h->num_cu, at<float>(ws, p.partial), s, p.sfp8));
    ys = at<float>(ws, p.ys);
  }
  if (c.has_latent_proj) {
    {
      StageScope sc(MOE_STAGE_COMBINE, s);
      MOE_TRY(launch_combine(at<void>(ws, p.O), p.f32, c.latent, at<int>(ws, p.tk_slot),
                             at<float>(ws, p.gate), T, c.top_k, c.latent, nullptr, at<void>(ws, p.u),
                             p.f32, s));
    }
    StageScope sc(MOE_STAGE_UP_PROJ, s);
    GemmArgs a = gemm_args();
    a.A = at<void>(ws, p.u); a.lda = c.latent;
    a.B = w.w_up; a.ldb = c.latent;
    a.M = T; a.N = c.d; a.K = c.latent;
    a.C = y; a.ldc = c.d;
    a.add = ys; a.ld_add = c.d;
    if (p.f32) MOE_TRY(dense_f32(a, false, ys ? EPI_F32_ADD : EPI_F32, h->num_cu, at<float>(ws, p.partial), s));
    else MOE_TRY(dense_bf16(a, ys ? EPI_BF16_ADD : EPI_BF16, h->num_cu, at<float>(ws, p.partial), s));
  } else {
    StageScope sc(MOE_STAGE_COMBINE, s);
    MOE_TRY(launch_combine(at<void>(ws, p.O), p.f32, c.latent, at<int>(ws, p.tk_slot),
                           at<float>(ws, p.gate), T, c.top_k, c.d, ys, y, p.f32, s));
  }
  return copy_out(h, T, ws, p, idx, gate, counts, s);
}

}  // namespace
