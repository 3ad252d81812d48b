// bf16 GEMM on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation:
// the latent projections d -> l and l -> d, the shared experts, and the grouped
// expert GEMMs of the prefill path.
//
// C[r][n] = epilogue( sum_k A[row(r)][k] * B_g[n][k] ).  Grouped mode walks a
// device-side list of row tiles (expert g, row0, row1) made by the routing
// scan, so the data-dependent expert sizes never need a host round-trip.  The A
// rows can be gathered through a row map (the expert up GEMM reads latent rows
// straight from z by token id).  B is bf16 or NVFP4: NVFP4 codes (E2M1 values,
// 16-element E4M3 block scales, FP32 global scale; Korean Nemotron 3 summary,
// section 2.4 NVFP4 Training) are staged raw in LDS and decoded exactly to bf16
// (as half their value) in registers by each wavefront right before its MFMAs
// (every e2m1*e4m3 product is a bf16 value); twice the global scale multiplies
// the fp32 accumulator in the epilogue.  Or both operands are FP8 E4M3 codes (FP8 post-training
// quantisation of weights and activations, Nemotron 3 Nano blog, FP8
// quantisation section; FP8 shared experts, Ultra release news): the loads and
// LDS layout are those of a bf16 GEMM over K/2 (two codes per 16-bit slot),
// two 16-wide bf16 substeps form one 64-deep step of
// v_mfma_f32_32x32x64_f8f6f4 (each lane's 32 bytes: its 16 bytes of both
// substeps; A and B take the same k for each lane and byte, so the dot
// product is unchanged), and the per-tensor scales multiply the accumulator.
// FP8 outputs (the activations of the next FP8 GEMM) are quantised in the
// epilogue.
//
// Data movement: operands go global -> LDS with gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16*lane)
// through a ring of NST stages, so NST-1 k-tiles are in flight while one is
// multiplied and no VGPRs are spent on staging.  The grouped 8-wavefront
// bf16 / FP8 kernels split the ring by operand instead: 2 A stages and 3 B
// (weight) stages in the same LDS, the weights loaded one k-tile further ahead.  The ring runs continuously
// over each persistent block's sequence of output tiles.  Each wavefront waits for its
// own loads with an explicit vmcnt, then a bare s_barrier publishes the stage.
// LDS rows hold BK bf16 as 16-byte chunks; chunk c of row r sits at c ^ f(r),
// which spreads the fragment reads of 8 or 16 consecutive rows over distinct
// bank groups.  The swizzle is applied on the global side (which chunk a lane
// fetches) because the LDS side of a direct load is fixed by the lane id.
//
// Tile BM x BN, WGM x WGN wavefronts, each owning (BM/WGM) x (BN/WGN) in 32x32
// MFMA blocks.  The MFMA computes C^T (weights as the A operand, activations as
// the B operand) so each lane holds 4 consecutive output columns of one row;
// bf16 outputs are transposed through LDS before they are stored.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

// Direct-to-LDS loads (M0 = the wavefront's LDS destination, each lane's
// bytes at M0 + lane * size).  They are written as inline asm so that the
// compiler's waitcnt insertion does not see them: with an LDS-DMA of its own in
// flight it waits for every outstanding fragment read (lgkmcnt(0)) at each MFMA
// step instead of only the ones that step needs.  Their completion is tracked
// by the explicit vmcnt waits below.  The asm has no register outputs.  M0 is
// a reserved register: the compiler sets it right before each instruction of
// its own that reads it (none in these kernels), hence the clobber, and the
// warning that clobbering a reserved register draws is silenced here.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// a wavefront-uniform pointer, kept in scalar registers for the asm's "s" operand
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const char* base, uint32_t off, void* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
// 4-byte direct load (sub-dword LDS-DMA forms are not used: their LDS placement
// is not the 2- or 1-byte lane stride the packed layouts here would need)
template <int BYTES>
__device__ __forceinline__ void dma_small(const char* base, uint32_t off, void* lds_wave_base) {
  static_assert(BYTES == 4, "dword LDS-DMA only");
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// barrier without the compiler's implied vmcnt(0): LDS-DMA completion is
// tracked by the explicit vmcnt waits above
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }
// barrier after this wavefront's own LDS writes
__device__ __forceinline__ void bar_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// chunk swizzle for rows of CPR 16-byte chunks (conflict-free for 32 or 64 banks)
template <int CPR>
__device__ __forceinline__ int swz_chunk(int row, int c) {
  if (CPR == 8) return c ^ ((row & 7) ^ ((row >> 3) & 1));
  return c ^ (((row >> 1) & 3) ^ ((row >> 3) & 1));
}

// NVFP4 codes of a 64-deep k-slab in a stage: row r's 32 bytes as two
// 16-byte halves (the k-tiled layout puts the codes of k 16i + 8h .. + 7, i =
// 0..3, in half h); half h sits in slot h ^ fp4_slot_swz(r), so that the
// 16-byte fragment reads of 8 (or 16) consecutive rows fall in distinct banks.
__device__ __forceinline__ int fp4_slot_swz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

}  // namespace

template <int BM, int BN, int BK, int WGM, int WGN, int NST, int WT>
struct TileCfg {
  static constexpr bool FP4 = WT == WT_NVFP4, IS_FP4 = FP4, IS_FP8 = WT == WT_FP8;
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per bf16 row
  static constexpr int KSUB = BK / 16;                         // 16-deep MFMA substeps per k-tile
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int BQ_BYTES = BN * 32;                     // NVFP4 codes: the whole 64-deep slab
  static constexpr int BS_BYTES = BN * 4;                      // NVFP4 scales: one aligned dword per row
  static constexpr int B_BYTES = FP4 ? BQ_BYTES + BS_BYTES : BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int EPB = 32 * WGM * BN * 2;                // epilogue staging: one 32-row block per wave row
  static constexpr int LDS = NST * STAGE + EPB;
  static constexpr int A_TOT = BM * CPR / 64;                  // 1 KB DMA blocks per k-tile
  static constexpr int B_TOT = FP4 ? BQ_BYTES / 1024 : BN * CPR / 64;
  static constexpr int S_TOT = FP4 ? BS_BYTES / 256 : 0;       // dword-per-lane DMA blocks
  static constexpr int A_PW = (A_TOT + NW - 1) / NW;           // per wavefront
  static constexpr int B_PW = (B_TOT + NW - 1) / NW;
  static constexpr int S_PW = (S_TOT + NW - 1) / NW;
  static constexpr int S_PW1 = S_PW > 0 ? S_PW : 1;
  static constexpr int S_TOT1 = S_TOT > 0 ? S_TOT : 1;
  static constexpr int LOADS = A_PW + B_PW + S_PW;             // vm ops per wave per k-tile
  static constexpr int WM = BM / WGM, WN = BN / WGN;           // wavefront tile
  static constexpr int TM = WM / 32, TN = WN / 32;             // 32x32 MFMA blocks per wavefront
  static_assert(A_TOT >= 1 && B_TOT >= 1 && (!FP4 || S_TOT >= 1), "tile too small");
  static_assert(LOADS * (NST - 1) < 64, "vmcnt range");
  static_assert(STAGE % 16 == 0, "stage alignment");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(!IS_FP8 || BK % 32 == 0, "FP8: whole 64-code steps per k-tile");
  static_assert(!FP4 || BK == 64 || BK == 32, "NVFP4: k-tiles of 32 or 64 in 64-deep weight slabs");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Load through the scalar unit; the address must be wavefront-uniform.  Scalar
// loads count on lgkmcnt, so waiting for them never drains the direct-to-LDS
// loads in flight (vmcnt), as a vector load of the tile list, the row indices
// or the global scale would.
template <class T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Wait until at most `pd` k-tiles of LOADS vector-memory ops each (the newest
// ones) plus EXTRA further ops issued after them (an epilogue's stores) are
// still in flight; pd is wavefront-uniform and <= MAXPD.  Any other ops issued
// after those loads also count, which only makes it wait longer.
template <int LOADS, int MAXPD, int EXTRA = 0>
__device__ __forceinline__ void wait_tiles(int pd) {
  static_assert(MAXPD * LOADS + EXTRA < 64, "vmcnt range");
  if constexpr (MAXPD >= 5) {
    if (pd >= 5) { wait_vm<5 * LOADS + EXTRA>(); return; }
  }
  if constexpr (MAXPD >= 4) {
    if (pd >= 4) { wait_vm<4 * LOADS + EXTRA>(); return; }
  }
  if constexpr (MAXPD >= 3) {
    if (pd >= 3) { wait_vm<3 * LOADS + EXTRA>(); return; }
  }
  if constexpr (MAXPD >= 2) {
    if (pd >= 2) { wait_vm<2 * LOADS + EXTRA>(); return; }
  }
  if constexpr (MAXPD >= 1) {
    if (pd >= 1) { wait_vm<LOADS + EXTRA>(); return; }
  }
  wait_vm<EXTRA>();
}

// Wait for k-tile `need` of a stream that has issued `issued` k-tiles, the
// last epilogue's STORES stores going out after k-tile `st_tile`.
template <int LOADS, int MAXPD, int STORES>
__device__ __forceinline__ void wait_tile(int need, int issued, int st_tile) {
  if (STORES > 0 && need <= st_tile) wait_tiles<LOADS, MAXPD, STORES>(issued - 1 - need);
  else wait_tiles<LOADS, MAXPD, 0>(issued - 1 - need);
}

// Global sources of one output tile: rows [r0, r1) of group g, columns
// [n0, n0 + BN), as tile-uniform bases plus this lane's 32-bit offsets.
template <class C>
struct TileSrc {
  int g, r0, r1, n0;
  const char* A;
  const char* B;
  const char* S;
  uint32_t aoff[C::A_PW], boff[C::B_PW], soff[C::S_PW1];
};

// Row tile `rt`, column tile `nt` of a list (or of the dense row blocks).
template <int BM, int BN>
__device__ __forceinline__ void item_coords(const GemmArgs& p, const int4* list, int nrt, int ntn,
                                            int it, int& g, int& r0, int& r1, int& n0) {
  int rt = it / ntn, nt = it - rt * ntn;
  if (!list && ntn > 8) {
    // dense and wide: walk bands of 4 row tiles column by column, so the 32
    // consecutive items of one XCD reuse 4 A and 8 B strips from its L2
    const int band = it / (4 * ntn), in = it - band * 4 * ntn;
    const int rows = min(4, nrt - band * 4);
    rt = band * 4 + in % rows;
    nt = in / rows;
  }
  if (list) {
    g = sload(&list[rt].x); r0 = sload(&list[rt].y); r1 = sload(&list[rt].z);
  } else {
    g = 0; r0 = rt * BM; r1 = min(p.M, r0 + BM);
  }
  n0 = nt * BN;
}

template <int BM, int BN, int BK, int WGM, int WGN, int NST, int WT>
__device__ __forceinline__ void make_src(const GemmArgs& p, int g, int r0, int r1, int n0,
                                         TileSrc<TileCfg<BM, BN, BK, WGM, WGN, NST, WT>>& s) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT>;
  constexpr bool FP4 = C::FP4;
  constexpr int CPR = C::CPR, NW = C::NW;
  constexpr int RPB = 64 / CPR;                    // A rows per 1 KB DMA block
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  s.g = g; s.r0 = r0; s.r1 = r1; s.n0 = n0;
  s.A = (const char*)p.A;
#pragma unroll
  for (int j = 0; j < C::A_PW; ++j) {
    const int blk = (wave + j * NW) % C::A_TOT;
    const int q = blk * 64 + lane;                 // LDS chunk index in the A region
    const int row = q / CPR, pos = q % CPR;        // row = blk * RPB + lane / CPR
    uint32_t pr;
    if (p.a_rows) {
      // the block's RPB row indices through the scalar unit (the index array
      // is padded, so reading up to RPB - 1 entries past r1 stays in bounds),
      // then each lane picks its own; rows past the end re-read the last row
      const int rb = r0 + blk * RPB;
      const int last = sload(p.a_rows + (r1 - 1));
      int pick = last;
      if (rb < r1) {
        int v[RPB];
#pragma unroll
        for (int u = 0; u < RPB; ++u) v[u] = sload(p.a_rows + rb + u);
        const int sub = lane / CPR;
        pick = v[0];
#pragma unroll
        for (int u = 1; u < RPB; ++u) pick = sub == u ? v[u] : pick;
        if (rb + sub >= r1) pick = last;
      }
      pr = (uint32_t)pick;
    } else {
      pr = (uint32_t)min(r0 + row, r1 - 1);        // rows past the end re-read the last row
    }
    s.aoff[j] = (pr * (uint32_t)p.lda + swz_chunk<CPR>(row, pos) * 8) * 2;   // bytes
  }
  s.B = FP4 ? (const char*)p.B + (int64_t)g * p.b_gstride
            : (const char*)p.B + (int64_t)g * p.b_gstride * 2;
  s.S = FP4 ? (const char*)p.b_scale + (int64_t)g * p.s_gstride : nullptr;
#pragma unroll
  for (int j = 0; j < C::B_PW; ++j) {
    const int blk = (wave + j * NW) % C::B_TOT;
    if (FP4) {
      // k-tiled codes: a 64-deep k-slab holds every row's 32 bytes in row
      // order; a DMA block is 32 rows x 32 bytes (two lanes per row, halves
      // swizzled).  A 32-deep k-tile loads its whole slab too.  Offsets are
      // relative to the slab.
      const int q = blk * 64 + lane, row = q >> 1;
      const uint32_t n = (uint32_t)min(n0 + row, p.N - 1);
      s.boff[j] = n * 32u + (uint32_t)(((q & 1) ^ fp4_slot_swz(row)) * 16);
    } else {
      const int q = blk * 64 + lane, row = q / CPR, pos = q % CPR;
      const uint32_t n = (uint32_t)min(n0 + row, p.N - 1);
      s.boff[j] = (n * (uint32_t)p.ldb + swz_chunk<CPR>(row, pos) * 8) * 2;   // bytes
    }
  }
#pragma unroll
  for (int j = 0; j < C::S_PW1; ++j) {
    const int blk = (wave + j * NW) % C::S_TOT1;
    const uint32_t n = (uint32_t)min(n0 + blk * 64 + lane, p.N - 1);
    s.soff[j] = n * 4u;                            // bytes in the k-slab: the row's dword holds
                                                   // the slab's four block scales
  }
}

// Direct-to-LDS loads of k-tile kt of a tile into one stage: the A part
// (PARTS bit 0) and the B part (bit 1).
template <int BM, int BN, int BK, int WGM, int WGN, int NST, int WT, int PARTS = 3>
__device__ __forceinline__ void issue_tile(const GemmArgs& p,
                                           const TileSrc<TileCfg<BM, BN, BK, WGM, WGN, NST, WT>>& s,
                                           int kt, char* stage) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT>;
  constexpr bool FP4 = C::FP4;
  constexpr int NW = C::NW;
  const int wave = threadIdx.x >> 6;
  const uint32_t k0 = (uint32_t)kt * BK;
  if constexpr (PARTS & 1) {
#pragma unroll
    for (int j = 0; j < C::A_PW; ++j) {
      const int blk = (wave + j * NW) % C::A_TOT;
      dma16(s.A + k0 * 2, s.aoff[j], stage + blk * 1024);
    }
  }
  if constexpr (!(PARTS & 2)) {
    return;
  } else if (FP4) {
    const uint32_t slab = k0 / 64;
    const char* Bk = s.B + slab * (uint32_t)p.ldb;
#pragma unroll
    for (int j = 0; j < C::B_PW; ++j) {
      const int blk = (wave + j * NW) % C::B_TOT;
      dma16(Bk, s.boff[j], stage + C::A_BYTES + blk * 1024);
    }
#pragma unroll
    for (int j = 0; j < C::S_PW; ++j) {
      const int blk = (wave + j * NW) % C::S_TOT1;
      dma_small<4>(s.S + slab * (uint32_t)p.lds_scale, s.soff[j], stage + C::A_BYTES + C::BQ_BYTES + blk * 256);
    }
  } else {
    const char* Bk = s.B + k0 * 2;
    if (p.kseg < p.K) {                    // B stored as k segments (shared experts' W2)
      const int seg = (int)(k0 / (uint32_t)p.kseg);
      Bk = s.B + ((int64_t)seg * p.b_segstride + (k0 - (uint32_t)seg * p.kseg)) * 2;
    }
#pragma unroll
    for (int j = 0; j < C::B_PW; ++j) {
      const int blk = (wave + j * NW) % C::B_TOT;
      dma16(Bk, s.boff[j], stage + C::A_BYTES + blk * 1024);
    }
  }
}

// Epilogue.  acc[j][i][r] = C[row][col] with row = i-block row (lane & 31),
// col = j-block column 8*(r/4) + 4*(lane/32) + r%4: 4 consecutive columns per r/4.
// bf16 and E4M3 outputs go through LDS (`stage`, EPB bytes): a lane's own
// values cover 8 (bf16) or 4 (E4M3) bytes of each of 32 rows per store, so they
// are transposed one i-block (32 rows per wavefront row) at a time and written
// back as whole 16-byte units, each wavefront store covering complete rows of
// the tile.  Contains barriers: every wavefront of the block calls it.
template <int EPI>
struct EpiKind {
  static constexpr bool STAGED = EPI == EPI_BF16 || EPI == EPI_SQRELU_BF16 || EPI == EPI_Q8 ||
                                 EPI == EPI_SQRELU_Q8;
  static constexpr int ELEM = (EPI == EPI_Q8 || EPI == EPI_SQRELU_Q8) ? 1 : 2;   // staged output bytes
  static constexpr bool SQRELU = EPI == EPI_SQRELU_BF16 || EPI == EPI_SQRELU_Q8;
  static constexpr bool Q8 = EPI == EPI_Q8 || EPI == EPI_SQRELU_Q8 || EPI == EPI_Z8;
};

template <int BM, int BN, int BK, int WGM, int WGN, int NST, int WT, int EPI>
__device__ __forceinline__ void epilogue_tile(
    const GemmArgs& p, int g, int r0, int r1, int n0, char* stage,
    f32x16 (&acc)[TileCfg<BM, BN, BK, WGM, WGN, NST, WT>::TN][TileCfg<BM, BN, BK, WGM, WGN, NST, WT>::TM]) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT>;
  using K = EpiKind<EPI>;
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  // weight scale times activation scale (1 for bf16 operands)
  const float sc = (p.b_gscale ? sload(p.b_gscale + g) : 1.0f) * (p.a_scale ? sload(p.a_scale) : 1.0f) *
                   decode_factor<WT>();
  const float rq = K::Q8 ? 1.0f / sload(p.q_scale) : 1.0f;
  if constexpr (K::STAGED) {
    constexpr int EL = K::ELEM;
    constexpr int RB = BN * EL;                    // staged row bytes
    constexpr int U = RB / 16;                     // 16-byte units per staged row
    constexpr int ROWS = 32 * WGM;                 // staged rows per i-block
    constexpr int PER = ROWS * U / C::NT;          // units stored per thread
    static_assert(ROWS * U % C::NT == 0, "epilogue units");
    const int lr = wm * 32 + (lane & 31);          // this lane's staged row
    // stores through a buffer resource over the tile's rows: lanes past the
    // tile's last row or column get an out-of-range offset and are dropped by
    // the hardware, so every thread issues all PER stores per i-block (the
    // k-loop waits count them)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (char*)p.C + (int64_t)r0 * p.ldc * EL, 0, (r1 - r0) * (int)p.ldc * EL, 0x00020000);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v0 = acc[j][i][4 * q + 0] * sc, v1 = acc[j][i][4 * q + 1] * sc;
          float v2 = acc[j][i][4 * q + 2] * sc, v3 = acc[j][i][4 * q + 3] * sc;
          if (K::SQRELU) {
            v0 = fmaxf(v0, 0.f); v1 = fmaxf(v1, 0.f); v2 = fmaxf(v2, 0.f); v3 = fmaxf(v3, 0.f);
            v0 *= v0; v1 *= v1; v2 *= v2; v3 *= v3;
          }
          const int lc = wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
          const int cb = lc * EL;                  // byte column in the staged row
          const int u = (cb >> 4) ^ (lr & (U - 1));
          char* dst = stage + lr * RB + u * 16 + (cb & 15);
          if constexpr (EL == 2) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
          } else {
            *reinterpret_cast<uint32_t*>(dst) = q8x4(v0, v1, v2, v3, rq);
          }
        }
      }
      bar_lds();                                   // i-block staged by every wavefront
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int gidx = threadIdx.x + k * C::NT;
        const int row = gidx / U, un = gidx % U;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + row * RB + (un ^ (row & (U - 1))) * 16);
        const int lrow = (row >> 5) * WM + i * 32 + (row & 31);   // row within the tile
        const int col = n0 + un * (16 / EL);
        const int off = (r0 + lrow < r1 && col < p.N) ? (lrow * (int)p.ldc + col) * EL : 0x7FFFFFF0;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, 0);
      }
      bar_lds();                                   // staging free for the next i-block
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + wm * WM + i * 32 + (lane & 31);
      if (row >= r1) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
          if (col >= p.N) continue;
          float v0 = acc[j][i][4 * q + 0], v1 = acc[j][i][4 * q + 1];
          float v2 = acc[j][i][4 * q + 2], v3 = acc[j][i][4 * q + 3];
          const int64_t o = (int64_t)row * p.ldc + col;
          if (EPI == EPI_F32) {
            v0 *= sc; v1 *= sc; v2 *= sc; v3 *= sc;
            *reinterpret_cast<float4*>((float*)p.C + o) = make_float4(v0, v1, v2, v3);
          } else if (EPI == EPI_Z) {
            *reinterpret_cast<float4*>((float*)p.C + o) = make_float4(v0, v1, v2, v3);
            *reinterpret_cast<uint2*>((uint16_t*)p.C2 + (int64_t)row * p.ldc2 + col) =
                make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
          } else if (EPI == EPI_Z8) {
            *reinterpret_cast<float4*>((float*)p.C + o) = make_float4(v0, v1, v2, v3);
            *reinterpret_cast<uint32_t*>((uint8_t*)p.C2 + (int64_t)row * p.ldc2 + col) =
                q8x4(v0, v1, v2, v3, rq);
          } else if (EPI == EPI_BF16_ADD) {
            const float4 ad = *reinterpret_cast<const float4*>(p.add + (int64_t)row * p.ld_add + col);
            v0 += ad.x; v1 += ad.y; v2 += ad.z; v3 += ad.w;
            *reinterpret_cast<uint2*>((uint16_t*)p.C + o) =
                make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
          }
        }
      }
    }
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
// two 16-byte LDS chunks -> one 8-dword MFMA operand
__device__ __forceinline__ i32x8 lds_pair(const uint4* base, int c0, int c1) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + c0);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + c1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// NVFP4 pipeline.  Substep s of a k-tile covers k 16s .. 16s + 15, lane half
// h its 8 k from 16s + 8h (A chunk 2s + h), as in the bf16 kernels.  In the
// k-tiled layout those codes of every substep are one 16-byte half of the
// row's slab, so a lane reads its codes once per k-tile (BK/4 bytes), and its
// block scales as one dword.
template <class C>
struct Fp4A {
  bf16x8 a[C::TM];
};
template <class C>
struct Fp4B {
  uint32_t q[C::TN][C::KSUB];   // raw codes: dword s feeds substep s
  uint32_t sc[C::TN];           // the row's block scales (E4M3) of the slab
};

// A fragments of substep s of the k-tile in `stage`.
template <int BM, int BN, int BK, int WGM, int WGN, int NST>
__device__ __forceinline__ void read_fp4_a(const char* stage, int s,
                                           Fp4A<TileCfg<BM, BN, BK, WGM, WGN, NST, WT_NVFP4>>& f) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT_NVFP4>;
  constexpr int CPR = C::CPR, WM = C::WM;
  const uint4* As = reinterpret_cast<const uint4*>(stage);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN;
  const int ch = s * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * WM + i * 32 + (lane & 31);
    f.a[i] = __builtin_bit_cast(bf16x8, As[row * CPR + swz_chunk<CPR>(row, ch)]);
  }
}

// Raw B fragments (codes and scales) of the k-tile in `stage`; odd: a 32-deep
// k-tile in the slab's second half.
template <int BM, int BN, int BK, int WGM, int WGN, int NST>
__device__ __forceinline__ void read_fp4_b(const char* stage, int odd,
                                           Fp4B<TileCfg<BM, BN, BK, WGM, WGN, NST, WT_NVFP4>>& f) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT_NVFP4>;
  constexpr int WN = C::WN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % WGN, h = lane >> 5;
  const uint8_t* Q = reinterpret_cast<const uint8_t*>(stage + C::A_BYTES);
  const uint8_t* Sc = Q + C::BQ_BYTES;
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int n = wn * WN + j * 32 + (lane & 31);
    const uint8_t* half = Q + n * 32 + ((h ^ fp4_slot_swz(n)) << 4);
    if constexpr (BK == 64) {
      const uint4 v = *reinterpret_cast<const uint4*>(half);
      f.q[j][0] = v.x; f.q[j][1] = v.y; f.q[j][2] = v.z; f.q[j][3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(half + 8 * odd);
      f.q[j][0] = v.x; f.q[j][1] = v.y;
    }
    f.sc[j] = *reinterpret_cast<const uint32_t*>(Sc + n * 4);
  }
}

// The decoded (exact) bf16 B fragments of substep s; kbyte: position of the
// k-tile's first block scale in the scale dword.
template <class C>
__device__ __forceinline__ void decode_fp4_b(const Fp4B<C>& f, int s, int kbyte, bf16x8 (&b)[C::TN]) {
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
    b[j] = __builtin_bit_cast(bf16x8, fp4x8(f.q[j][s], split_scale(f.sc[j] >> (8 * (kbyte + s)))));
}

// acc += A fragments x decoded B fragments (the MFMA computes C^T: weights as
// its A operand).
template <class C>
__device__ __forceinline__ void mma_fp4(const Fp4A<C>& f, const bf16x8 (&b)[C::TN], f32x16 (&acc)[C::TN][C::TM]) {
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], f.a[i], acc[j][i], 0, 0, 0);
}

// Scheduling constraint for one substep: alternate NR LDS reads (the next
// substep's fragments) with this substep's MFMAs, so each read's latency hides
// behind MFMAs instead of stalling the wavefront before the first of them.
template <class C, int NR>
__device__ __forceinline__ void interleave_reads_mfma() {
  constexpr int NM = C::TM * C::TN;
  constexpr int P = NR < NM ? NR : NM;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
  }
  if constexpr (NR > P) __builtin_amdgcn_sched_group_barrier(0x100, NR - P, 0);
  if constexpr (NM > P) __builtin_amdgcn_sched_group_barrier(0x008, NM - P, 0);
}

// One block's share of one tile list (items first, first + step, ... of the
// nrt x ntn items) with NVFP4 weights (bf16 and FP8 operands run
// gemm_stream_lean: the same ring, waits and barriers with a leaner fragment
// pipeline, which NVFP4's raw B fragments do not fit).  The direct-to-LDS ring runs continuously
// across the block's items: the last k-iterations of one item already load the
// first k-tiles of the next, so its epilogue overlaps those loads and the
// pipeline never drains between items.  LDS reads are software-pipelined: the
// fragments of substep s + 1 are read while the MFMAs of substep s run (two
// register sets), and the one barrier per k-tile sits before the tile's last
// substep: after it the wavefront reads the next tile's first fragments and
// refills the stage it has just finished with, while the last MFMAs of the
// tile execute.  All NST stages hold k-tiles; requires K / BK >= NST.  The
// waits leave the previous epilogue's stores in flight until a k-tile issued
// after them is needed.  NVFP4 stages hold the raw codes and scales; each
// wavefront decodes the B fragments it multiplies (those of its wavefront
// column; with a 1 x 8 wavefront grid each element is decoded by one
// wavefront), so the decode runs on the VALU beside the other wavefront's
// MFMAs.
template <int BM, int BN, int BK, int WGM, int WGN, int NST, int EPI>
__device__ __forceinline__ void gemm_stream_fp4(const GemmArgs& p, char* smem, const int4* list,
                                                int nrt, int first, int step) {
  constexpr int WT = WT_NVFP4;
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT>;
  constexpr int TM = C::TM, TN = C::TN, S = BK / 16;
  static_assert(S % 2 == 0, "substep 0 of every k-tile uses the first register set");
  const int ntn = (p.N + BN - 1) / BN;
  const int total = nrt * ntn;
  if (first >= total) return;
  const int nk = p.K / BK;

  wait_vm<0>();   // only this stream's loads are in flight from here on
  TileSrc<C> cur, nxt;
  int it = first;
  {
    int g, r0, r1, n0;
    item_coords<BM, BN>(p, list, nrt, ntn, it, g, r0, r1, n0);
    make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, g, r0, r1, n0, cur);
  }
#pragma unroll
  for (int s = 0; s < NST; ++s) issue_tile<BM, BN, BK, WGM, WGN, NST, WT>(p, cur, s, smem + s * C::STAGE);
  int issued = NST;          // k-tiles of this stream issued so far
  wait_tiles<C::LOADS, NST - 1>(issued - 1);
  bar();
  Fp4A<C> f0, f1;          // A fragments of alternate substeps
  Fp4B<C> fb;              // raw B fragments of the current k-tile
  // the scale dword of each row holds k-tile kt's first block scale at this
  // byte (a slab's 4 blocks hold two 32-deep k-tiles)
  auto kbyte = [](int kt) { return (kt * (BK / 16)) & 3; };
  read_fp4_a<BM, BN, BK, WGM, WGN, NST>(smem, 0, f0);
  read_fp4_b<BM, BN, BK, WGM, WGN, NST>(smem, 0, fb);
  int gt = 0;                // k-tiles of this stream consumed so far
  // stores per thread of one staged epilogue (all issued, see epilogue_tile)
  constexpr int ST = EpiKind<EPI>::STAGED ? TM * (32 * WGM * (BN * EpiKind<EPI>::ELEM / 16)) / C::NT : 0;
  int st_tile = -1;          // last k-tile issued before the latest epilogue's stores

  for (;;) {
    const int itn = it + step;
    const bool has_next = itn < total;
    int ng = 0, nr0 = 0, nr1 = 0, nn0 = 0;
    if (has_next) item_coords<BM, BN>(p, list, nrt, ntn, itn, ng, nr0, nr1, nn0);
    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

    for (int kt = 0; kt < nk; ++kt) {
      const int sg = gt % NST;
      const char* st = smem + sg * C::STAGE;
#pragma unroll
      for (int s = 0; s + 1 < S; ++s) {
        bf16x8 b[TN];
        decode_fp4_b<C>(fb, s, kbyte(kt), b);
        if (s % 2 == 0) {
          read_fp4_a<BM, BN, BK, WGM, WGN, NST>(st, s + 1, f1);
          mma_fp4<C>(f0, b, acc);
        } else {
          read_fp4_a<BM, BN, BK, WGM, WGN, NST>(st, s + 1, f0);
          mma_fp4<C>(f1, b, acc);
        }
        interleave_reads_mfma<C, TM>();
      }
      // refill stage sg with the k-tile NST ahead.  With 8 wavefronts the
      // weight codes and scales go out right after the barrier and the A rows
      // after the last substep (measured 3-4% faster than the reverse order on
      // the Ultra-like NVFP4 prefill, everything after the barrier 2-3% slower,
      // the A rows spread over the next k-tile's first substeps 1.5-2.5% slower)
      constexpr int FIRST = C::NW == 8 ? 2 : 3;
      const int j = kt + NST;
      char* fs = smem + sg * C::STAGE;
      int refill = 0;                    // 1: k-tile j of this item, 2: k-tile j - nk of the next
      const char* nst = smem + ((gt + 1) % NST) * C::STAGE;
      if (kt + 1 < nk || has_next) {
        // k-tile gt + 1 landed (own loads), own reads of stage sg complete;
        // after the barrier the same holds for every wavefront
        wait_tile<C::LOADS, NST - 2, ST>(gt + 1, issued, st_tile);
        bar_lds();
        if (j < nk) {
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, FIRST>(p, cur, j, fs);
          refill = 1;
          ++issued;
        } else if (has_next) {
          if (j == nk) make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, ng, nr0, nr1, nn0, nxt);
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, FIRST>(p, nxt, j - nk, fs);
          refill = 2;
          ++issued;
        }
        if (FIRST == 3) refill = 0;
        read_fp4_a<BM, BN, BK, WGM, WGN, NST>(nst, 0, f0);
      }
      // one call site for the last substep: duplicating it in both branches
      // doubles the live accumulators and spills them.  Its B fragments are
      // decoded first, then the next k-tile's raw ones read into the same
      // registers (in the stream's last k-tile a harmless read of a stale stage)
      {
        bf16x8 b[TN];
        decode_fp4_b<C>(fb, S - 1, kbyte(kt), b);
        read_fp4_b<BM, BN, BK, WGM, WGN, NST>(nst, kt + 1 < nk ? (kt + 1) & 1 : 0, fb);
        mma_fp4<C>(f1, b, acc);
      }
      interleave_reads_mfma<C, TM + 2 * TN>();
      // the A part of the refill: k-tile j of this item or j - nk of the next
      if (refill == 1) issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, cur, j, fs);
      else if (refill == 2) issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, nxt, j - nk, fs);
      ++gt;
    }
    st_tile = issued - 1;
    epilogue_tile<BM, BN, BK, WGM, WGN, NST, WT, EPI>(p, cur.g, cur.r0, cur.r1, cur.n0,
                                                       smem + NST * C::STAGE, acc);
    if (!has_next) break;
    cur = nxt;
    it = itn;
  }
  bar_lds();   // every wave is done with the LDS before the caller reuses it
}

// Operands of step s for MFMA row block i (A) or column block j (B) of this
// wavefront: swizzled LDS chunks as in the direct-to-LDS ring; one 16-byte chunk per lane for bf16 (16-wide
// step), two for FP8 (64-code step).
template <class C>
using LeanOp = typename std::conditional<C::IS_FP8, i32x8, bf16x8>::type;
template <class C>
__device__ __forceinline__ LeanOp<C> lean_read(const uint4* rows, int r, int s) {
  constexpr int CPR = C::CPR;
  const int h = (threadIdx.x & 63) >> 5;
  if constexpr (C::IS_FP8) {
    const int c0 = s * 4 + h;
    return lds_pair(rows + r * CPR, swz_chunk<CPR>(r, c0), swz_chunk<CPR>(r, c0 + 2));
  } else {
    return __builtin_bit_cast(bf16x8, rows[r * CPR + swz_chunk<CPR>(r, s * 2 + h)]);
  }
}
template <class C, int WGN>
__device__ __forceinline__ LeanOp<C> lean_a(const char* stage, int s, int i) {
  const int wm = (threadIdx.x >> 6) / WGN;
  return lean_read<C>(reinterpret_cast<const uint4*>(stage), wm * C::WM + i * 32 + (threadIdx.x & 31), s);
}
template <class C, int WGN>
__device__ __forceinline__ LeanOp<C> lean_b(const char* stage, int s, int j) {
  const int wn = (threadIdx.x >> 6) % WGN;
  return lean_read<C>(reinterpret_cast<const uint4*>(stage + C::A_BYTES), wn * C::WN + j * 32 + (threadIdx.x & 31), s);
}
template <class C>
__device__ __forceinline__ f32x16 lean_mfma(const LeanOp<C>& b, const LeanOp<C>& a, const f32x16& c) {
  if constexpr (C::IS_FP8)   // E4M3 x E4M3 (format selectors 0), no block scales: the unscaled MFMA
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
}

// Scheduling order of one step: per row block I, its TN MFMAs, then its reads
// (A block I and the B blocks j = I mod TM; R ds_read_b128 per operand).
template <class C, int I, int R>
__device__ __forceinline__ void sched_lean_rows() {
  if constexpr (I < C::TM) {
    constexpr int NB = (C::TN - I + C::TM - 1) / C::TM;
    __builtin_amdgcn_sched_group_barrier(0x008, C::TN, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R * (1 + NB), 0);
    sched_lean_rows<C, I + 1, R>();
  }
}

// One step: the MFMAs of (fa, fb) and, interleaved with them, the reads of the
// step after it (step sn of `next`): each A fragment is re-read into its own
// registers right after its last MFMA (row blocks outermost), B into the other
// buffer fbn.  One A set plus two B sets keep the 8-wavefront 256x256 tile
// within 256 registers per lane.
template <class C, int WGN>
__device__ __forceinline__ void lean_step(f32x16 (&acc)[C::TN][C::TM], LeanOp<C> (&fa)[C::TM],
                                          const LeanOp<C> (&fb)[C::TN], LeanOp<C> (&fbn)[C::TN],
                                          const char* next, int sn) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j][i] = lean_mfma<C>(fb[j], fa[i], acc[j][i]);
    fa[i] = lean_a<C, WGN>(next, sn, i);
#pragma unroll
    for (int j = i; j < C::TN; j += C::TM) fbn[j] = lean_b<C, WGN>(next, sn, j);
  }
  sched_lean_rows<C, 0, C::IS_FP8 ? 2 : 1>();
}

// lean_step with the A and B operands in separate stages (b_stage - A_BYTES is
// passed as the B side's "stage" so that lean_b's offset lands in b_stage)
template <class C, int WGN>
__device__ __forceinline__ void lean_step_ab(f32x16 (&acc)[C::TN][C::TM], LeanOp<C> (&fa)[C::TM],
                                             const LeanOp<C> (&fb)[C::TN], LeanOp<C> (&fbn)[C::TN],
                                             const char* anext, const char* bnext, int sn) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j][i] = lean_mfma<C>(fb[j], fa[i], acc[j][i]);
    fa[i] = lean_a<C, WGN>(anext, sn, i);
#pragma unroll
    for (int j = i; j < C::TN; j += C::TM) fbn[j] = lean_b<C, WGN>(bnext - C::A_BYTES, sn, j);
  }
  sched_lean_rows<C, 0, C::IS_FP8 ? 2 : 1>();
}

// 8-wavefront bf16 / FP8 tiles: the same continuous fragment pipeline with
// separate rings for the operands, 2 A stages and 3 B stages (the weights,
// whose loads cost the most, are issued a k-tile earlier).  Per k-tile: after
// the wait for k-tile gt + 1 and the barrier, A k-tile gt + 2 refills the A
// stage just consumed; after the tile's last step B k-tile gt + 3 refills its
// B stage.  Each wait then leaves exactly the newest B group (and, after an
// item's epilogue, its stores) in flight.  The epilogue stages its rows in the
// B stage just consumed and issues that stage's refill after it.
template <int BM, int BN, int BK, int WGM, int WGN, int NST, int WT, int EPI>
__device__ __forceinline__ void gemm_stream_ab(const GemmArgs& p, char* smem, const int4* list,
                                               int nrt, int first, int step) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT>;
  using Op = LeanOp<C>;
  constexpr int TM = C::TM, TN = C::TN, S = C::IS_FP8 ? BK / 32 : BK / 16;
  constexpr int NA = 2, NB = 3;
  static_assert(!C::IS_FP4 && C::NW == 8, "8-wavefront bf16 / FP8 tiles");
  static_assert(S % 2 == 0, "step 0 of every k-tile reads the first B set");
  static_assert(EpiKind<EPI>::STAGED ? 32 * WGM * BN * EpiKind<EPI>::ELEM <= C::B_BYTES : true,
                "epilogue staging fits a B stage");
  static_assert(C::A_PW + C::B_PW < 64 && 2 * C::B_PW + C::A_PW < 64, "vmcnt range");
  const int ntn = (p.N + BN - 1) / BN;
  const int total = nrt * ntn;
  if (first >= total) return;
  const int nk = p.K / BK;                           // >= NB: the kernel takes this path only then
  char* const abase = smem;
  char* const bbase = smem + NA * C::A_BYTES;
  auto astage = [&](int t) { return abase + (t % NA) * C::A_BYTES; };
  auto bstage = [&](int t) { return bbase + (t % NB) * C::B_BYTES; };   // the B data itself
  constexpr int ST = EpiKind<EPI>::STAGED ? TM * (32 * WGM * (BN * EpiKind<EPI>::ELEM / 16)) / C::NT : 0;
  static_assert(C::B_PW + ST < 64, "vmcnt range");

  wait_vm<0>();
  TileSrc<C> cur, nxt;
  int it = first;
  {
    int g, r0, r1, n0;
    item_coords<BM, BN>(p, list, nrt, ntn, it, g, r0, r1, n0);
    make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, g, r0, r1, n0, cur);
  }
  // prologue, in this order: A0 B0 B1 A1 B2
  issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, cur, 0, astage(0));
  issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 2>(p, cur, 0, bstage(0) - C::A_BYTES);
  issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 2>(p, cur, 1, bstage(1) - C::A_BYTES);
  issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, cur, 1, astage(1));
  issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 2>(p, cur, 2, bstage(2) - C::A_BYTES);
  wait_vm<2 * C::B_PW + C::A_PW>();                  // A0 and B0 landed
  bar();
  Op fa[TM], fb0[TN], fb1[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[i] = lean_a<C, WGN>(astage(0), 0, i);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb0[j] = lean_b<C, WGN>(bstage(0) - C::A_BYTES, 0, j);
  int gt = 0;
  // in flight after the newest A group: 1 = one B group, 2 = one B group and
  // an epilogue's stores
  int after_a = 1;

  for (;;) {
    const int itn = it + step;
    const bool has_next = itn < total;
    int ng = 0, nr0 = 0, nr1 = 0, nn0 = 0;
    if (has_next) item_coords<BM, BN>(p, list, nrt, ntn, itn, ng, nr0, nr1, nn0);
    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;
    bool made_nxt = false;
    int bdelay = -1;                                 // B k-tile (of nxt) left for after the epilogue

    for (int kt = 0; kt < nk; ++kt) {
      const char* as = astage(gt);
      const char* bs = bstage(gt);
#pragma unroll
      for (int s = 0; s + 1 < S; ++s) {              // steps 0 .. S-2 read steps 1 .. S-1
        if (s % 2 == 0) lean_step_ab<C, WGN>(acc, fa, fb0, fb1, as, bs, s + 1);
        else lean_step_ab<C, WGN>(acc, fa, fb1, fb0, as, bs, s + 1);
      }
      const bool more = kt + 1 < nk || has_next;     // a k-tile gt + 1 exists
      if (more) {
        // A and B of k-tile gt + 1 landed (own loads), own reads of this
        // tile's stages complete; after the barrier the same holds for all
        if (after_a == 2) wait_vm<C::B_PW + ST>();
        else if (after_a == 1) wait_vm<C::B_PW>();
        else wait_vm<0>();
        bar_lds();
        // A k-tile gt + 2 into the A stage just consumed
        const int ja = kt + NA;
        if (ja < nk) {
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, cur, ja, astage(gt));
        } else if (has_next) {
          if (!made_nxt) { make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, ng, nr0, nr1, nn0, nxt); made_nxt = true; }
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, nxt, ja - nk, astage(gt));
        }
      }
      // the last step reads step 0 of k-tile gt + 1 (stale stages after the
      // last k-tile of the last item: read, not used)
      lean_step_ab<C, WGN>(acc, fa, fb1, fb0, astage(gt + 1), bstage(gt + 1), 0);
      // B k-tile gt + 3 into the B stage just consumed; an item's last k-tile
      // keeps that stage for the epilogue and issues the load after it
      const int jb = kt + NB;
      after_a = 0;
      if (more) {
        if (jb < nk) {
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 2>(p, cur, jb, bstage(gt) - C::A_BYTES);
          after_a = 1;
        } else if (has_next) {
          if (!made_nxt) { make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, ng, nr0, nr1, nn0, nxt); made_nxt = true; }
          if (kt + 1 < nk) {
            issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 2>(p, nxt, jb - nk, bstage(gt) - C::A_BYTES);
            after_a = 1;
          } else {
            bdelay = jb - nk;
          }
        }
      }
      ++gt;
    }
    // epilogue in the B stage of the item's last k-tile (gt - 1), free since
    // that k-tile's barrier (the last item's last k-tile has none: add it)
    if (!has_next) bar_lds();
    char* est = bstage(gt - 1);
    epilogue_tile<BM, BN, BK, WGM, WGN, NST, WT, EPI>(p, cur.g, cur.r0, cur.r1, cur.n0, est, acc);
    if (!has_next) break;
    if (bdelay >= 0) {
      issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 2>(p, nxt, bdelay, est - C::A_BYTES);
      after_a = 2;
    }
    cur = nxt;
    it = itn;
  }
  bar_lds();
}

// gemm_stream_fp4's ring with the register-lean fragment pipeline of lean_step, for bf16
// and FP8 operands (S steps per k-tile): the same continuous ring, waits and
// barrier placement.
template <int BM, int BN, int BK, int WGM, int WGN, int NST, int WT, int EPI>
__device__ __forceinline__ void gemm_stream_lean(const GemmArgs& p, char* smem, const int4* list,
                                                 int nrt, int first, int step) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, WT>;
  using Op = LeanOp<C>;
  constexpr int TM = C::TM, TN = C::TN, S = C::IS_FP8 ? BK / 32 : BK / 16;
  static_assert(!C::IS_FP4, "NVFP4 uses gemm_stream_fp4");
  static_assert(S % 2 == 0, "step 0 of every k-tile reads the first B set");
  const int ntn = (p.N + BN - 1) / BN;
  const int total = nrt * ntn;
  if (first >= total) return;
  const int nk = p.K / BK;

  wait_vm<0>();
  TileSrc<C> cur, nxt;
  int it = first;
  {
    int g, r0, r1, n0;
    item_coords<BM, BN>(p, list, nrt, ntn, it, g, r0, r1, n0);
    make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, g, r0, r1, n0, cur);
  }
#pragma unroll
  for (int s = 0; s < NST; ++s) issue_tile<BM, BN, BK, WGM, WGN, NST, WT>(p, cur, s, smem + s * C::STAGE);
  int issued = NST;
  wait_tiles<C::LOADS, NST - 1>(issued - 1);
  bar();
  Op fa[TM], fb0[TN], fb1[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[i] = lean_a<C, WGN>(smem, 0, i);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb0[j] = lean_b<C, WGN>(smem, 0, j);
  int gt = 0;
  constexpr int ST = EpiKind<EPI>::STAGED ? TM * (32 * WGM * (BN * EpiKind<EPI>::ELEM / 16)) / C::NT : 0;
  int st_tile = -1;

  for (;;) {
    const int itn = it + step;
    const bool has_next = itn < total;
    int ng = 0, nr0 = 0, nr1 = 0, nn0 = 0;
    if (has_next) item_coords<BM, BN>(p, list, nrt, ntn, itn, ng, nr0, nr1, nn0);
    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

    for (int kt = 0; kt < nk; ++kt) {
      const int sg = gt % NST;
      char* st = smem + sg * C::STAGE;
#pragma unroll
      for (int s = 0; s + 1 < S; ++s) {                  // steps 0 .. S-2 read steps 1 .. S-1
        if (s % 2 == 0) lean_step<C, WGN>(acc, fa, fb0, fb1, st, s + 1);
        else lean_step<C, WGN>(acc, fa, fb1, fb0, st, s + 1);
      }
      // refill stage sg with the k-tile NST ahead.  With 8 wavefronts its B
      // part (the weights, the loads that cost the most) goes out right after
      // the barrier and its A part after the tile's last step, so that their 64
      // loads do not all queue at the address unit at once; with 4 the whole
      // k-tile goes out after the barrier.
      constexpr int FIRST = C::NW == 8 ? 2 : 3;
      const int j = kt + NST;
      int refill = 0;                    // 1: k-tile j of this item, 2: k-tile j - nk of the next
      if (kt + 1 < nk || has_next) {
        wait_tile<C::LOADS, NST - 2, ST>(gt + 1, issued, st_tile);
        bar_lds();
        if (j < nk) {
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, FIRST>(p, cur, j, st);
          refill = 1;
          ++issued;
        } else if (has_next) {
          if (j == nk) make_src<BM, BN, BK, WGM, WGN, NST, WT>(p, ng, nr0, nr1, nn0, nxt);
          issue_tile<BM, BN, BK, WGM, WGN, NST, WT, FIRST>(p, nxt, j - nk, st);
          refill = 2;
          ++issued;
        }
        if (FIRST == 3) refill = 0;
      }
      // the last step reads step 0 of the next k-tile (after the last k-tile
      // of the last item they read a stale stage and are not used)
      lean_step<C, WGN>(acc, fa, fb1, fb0, smem + ((gt + 1) % NST) * C::STAGE, 0);
      if (refill == 1) issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, cur, j, st);
      else if (refill == 2) issue_tile<BM, BN, BK, WGM, WGN, NST, WT, 1>(p, nxt, j - nk, st);
      ++gt;
    }
    st_tile = issued - 1;
    epilogue_tile<BM, BN, BK, WGM, WGN, NST, WT, EPI>(p, cur.g, cur.r0, cur.r1, cur.n0,
                                                      smem + NST * C::STAGE, acc);
    if (!has_next) break;
    cur = nxt;
    it = itn;
  }
  bar_lds();
}

// Persistent kernel.  Phase 1 walks list 0 (row tiles of height <= BM, or the
// dense row blocks), phase 2 list 1 (row tiles of height <= BMS: the remainder
// of each expert's rows) with its own ring; p.lists selects the lists of a
// grouped launch (both, or one for a timing run per phase).  Block b takes the
// items of its XCD's slice of each round of gridDim.x items (block b runs on
// XCD b % 8), so consecutive items (the column tiles of one row tile, then the
// next row tiles of the same expert) share an L2.
template <int BM, int BN, int BMS, int WGM, int WGN, int BK1, int NST1, int BK2, int NST2, int WT,
          int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmArgs p) {
  extern __shared__ uint4 smem_u4[];
  char* smem = reinterpret_cast<char*>(smem_u4);
  const int G = gridDim.x;
  const int base = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int nrt0 = !p.tiles ? (p.M + BM - 1) / BM : (p.lists & 1) ? p.n_tiles[0] : 0;
  const int nrt1 = p.tiles && (p.lists & 2) ? p.n_tiles[1] : 0;
  if constexpr (WT != WT_NVFP4 && WGM * WGN == 8 && BK1 == 64 && BK2 == 64 && BMS > 0) {
    if (p.K >= 3 * BK1) {                    // three B stages of one tile
      gemm_stream_ab<BM, BN, BK1, WGM, WGN, NST1, WT, EPI>(p, smem, p.tiles, nrt0, base, G);
      if constexpr (BMS > 0)
        gemm_stream_ab<BMS, BN, BK2, WGM, WGN, NST2, WT, EPI>(p, smem, p.tiles2, nrt1, base, G);
    } else {
      gemm_stream_lean<BM, BN, BK1, WGM, WGN, NST1, WT, EPI>(p, smem, p.tiles, nrt0, base, G);
      if constexpr (BMS > 0)
        gemm_stream_lean<BMS, BN, BK2, WGM, WGN, NST2, WT, EPI>(p, smem, p.tiles2, nrt1, base, G);
    }
  } else if constexpr (WT != WT_NVFP4) {
    gemm_stream_lean<BM, BN, BK1, WGM, WGN, NST1, WT, EPI>(p, smem, p.tiles, nrt0, base, G);
    if constexpr (BMS > 0)
      gemm_stream_lean<BMS, BN, BK2, WGM, WGN, NST2, WT, EPI>(p, smem, p.tiles2, nrt1, base, G);
  } else {
    gemm_stream_fp4<BM, BN, BK1, WGM, WGN, NST1, EPI>(p, smem, p.tiles, nrt0, base, G);
    if constexpr (BMS > 0)
      gemm_stream_fp4<BMS, BN, BK2, WGM, WGN, NST2, EPI>(p, smem, p.tiles2, nrt1, base, G);
  }
}

// The remainder list (list 1) of NVFP4 weights as a launch of its own: 128 x
// 256 tiles on 4 wavefronts (1 x 4 grid) with two ring stages, two blocks per
// CU (66 KB of LDS and at most 256 registers each), so every SIMD runs
// wavefronts of two independent pipelines.  That phase is bound by latency,
// not by its MFMAs or weight bytes.
template <int BK, int NST, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_fp4_rem_kernel(GemmArgs p) {
  extern __shared__ uint4 smem_u4[];
  char* smem = reinterpret_cast<char*>(smem_u4);
  const int G = gridDim.x;
  const int base = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  gemm_stream_fp4<128, 256, BK, 1, 4, NST, EPI>(p, smem, p.tiles2, p.n_tiles[1], base, G);
}

namespace {

template <int BM, int BN, int BMS, int WGM, int WGN, int BK1, int NST1, int BK2, int NST2, int WT,
          int EPI>
hipError_t launch_one(const GemmArgs& a, int64_t total, int num_cu, hipStream_t s) {
  using C1 = TileCfg<BM, BN, BK1, WGM, WGN, NST1, WT>;
  using C2 = TileCfg<(BMS > 0 ? BMS : BM), BN, BK2, WGM, WGN, NST2, WT>;
  constexpr bool AB = WT != WT_NVFP4 && WGM * WGN == 8 && BK1 == 64 && BK2 == 64 && BMS > 0;
  constexpr size_t ab1 = AB ? (size_t)(2 * C1::A_BYTES + 3 * C1::B_BYTES) : 0;
  constexpr size_t ab2 = AB && BMS > 0 ? (size_t)(2 * C2::A_BYTES + 3 * C2::B_BYTES) : 0;
  constexpr size_t lds1 = (size_t)C1::LDS > ab1 ? (size_t)C1::LDS : ab1;
  constexpr size_t lds2 = BMS > 0 ? ((size_t)C2::LDS > ab2 ? (size_t)C2::LDS : ab2) : 0;
  constexpr size_t lds = lds1 > lds2 ? lds1 : lds2;
  static_assert(lds <= 160 * 1024, "LDS");
  auto* kern = gemm_bf16_kernel<BM, BN, BMS, WGM, WGN, BK1, NST1, BK2, NST2, WT, EPI>;
  // every stage of the ring holds a k-tile of the first output tile
  if (a.K / BK1 < NST1 || (BMS > 0 && a.K / BK2 < NST2)) return hipErrorInvalidValue;
  // the dynamic-LDS limit, set once per device (idempotent if two host
  // threads race on the first launch)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  // persistent grid: as many blocks as fit at once (a multiple of the 8 XCDs)
  const int per_cu = (int)((160 * 1024) / lds);
  const int64_t cap = ((int64_t)num_cu * (per_cu > 0 ? per_cu : 1)) & ~7LL;
  int grid = (int)(total < cap ? total : cap);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WGM * WGN), lds, s, a);
  return hipGetLastError();
}

// bf16: both lists with BK = 64 (fewer barriers per flop; 2 stages for
// 256x256 tiles, 3 for smaller ones).  NVFP4: BK = 64 with 3 stages (a raw
// stage is 5/8 of a bf16 one).  FP8 (K in 16-bit slots here): the bf16 rings
// with BK = 64, whole 64-code MFMA steps.  Short reductions (K = 64, 128) take
// rings that fit in K / BK k-tiles.
template <int BM, int BN, int BMS, int WGM, int WGN, int EPI, bool GROUPED>
hipError_t launch_epi(const GemmArgs& a, int wt, int64_t grid, int num_cu, hipStream_t s) {
  constexpr int NSTB = (BM == 256 && BN == 256) ? 2 : 3;
  constexpr bool Q8OUT = EPI == EPI_Q8 || EPI == EPI_SQRELU_Q8;
  if constexpr (GROUPED && !Q8OUT) {   // NVFP4 weights: grouped expert GEMMs only
    if (wt == WT_NVFP4) {
      if (a.K >= 192) return launch_one<BM, BN, BMS, WGM, WGN, 64, 3, 64, 3, WT_NVFP4, EPI>(a, grid, num_cu, s);
      if (a.K == 128) return launch_one<BM, BN, BMS, WGM, WGN, 64, 2, 64, 2, WT_NVFP4, EPI>(a, grid, num_cu, s);
      return launch_one<BM, BN, BMS, WGM, WGN, 32, 2, 32, 2, WT_NVFP4, EPI>(a, grid, num_cu, s);
    }
  }
  if (wt == WT_NVFP4) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_SQRELU_Q8 || EPI == EPI_BF16 || EPI == EPI_F32) {
    if (wt == WT_FP8) {
      if (a.K >= 192) return launch_one<BM, BN, BMS, WGM, WGN, 64, NSTB, 64, NSTB, WT_FP8, EPI>(a, grid, num_cu, s);
      if (a.K == 128) return launch_one<BM, BN, BMS, WGM, WGN, 64, 2, 64, 2, WT_FP8, EPI>(a, grid, num_cu, s);
      return hipErrorInvalidValue;
    }
  }
  if (wt != WT_BF16) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_SQRELU_Q8) {
    return hipErrorInvalidValue;       // quantised hidden rows only from FP8 GEMMs
  } else {
    if (a.K >= 192) return launch_one<BM, BN, BMS, WGM, WGN, 64, NSTB, 64, NSTB, WT_BF16, EPI>(a, grid, num_cu, s);
    if (a.K == 128) return launch_one<BM, BN, BMS, WGM, WGN, 32, 4, 32, 4, WT_BF16, EPI>(a, grid, num_cu, s);
    return launch_one<BM, BN, BMS, WGM, WGN, 32, 2, 32, 2, WT_BF16, EPI>(a, grid, num_cu, s);
  }
}

template <int BM, int BN, int BMS, int WGM, int WGN>
hipError_t launch_shape(const GemmArgs& a, int wt, int epi, int64_t grid, int num_cu, hipStream_t s) {
  if (a.tiles) {                   // grouped expert GEMMs: bf16, NVFP4 or FP8 weights
    if constexpr (BMS > 0) {
      switch (epi) {
        case EPI_SQRELU_BF16: return launch_epi<BM, BN, BMS, WGM, WGN, EPI_SQRELU_BF16, true>(a, wt, grid, num_cu, s);
        case EPI_BF16: return launch_epi<BM, BN, BMS, WGM, WGN, EPI_BF16, true>(a, wt, grid, num_cu, s);
        case EPI_SQRELU_Q8: return launch_epi<BM, BN, BMS, WGM, WGN, EPI_SQRELU_Q8, true>(a, wt, grid, num_cu, s);
        default: break;
      }
    }
    return hipErrorInvalidValue;
  }
  if (wt == WT_NVFP4 || BMS != 0) return hipErrorInvalidValue;   // dense GEMMs: no lists
  if (wt == WT_FP8) {              // FP8 dense GEMMs: the shared experts
    switch (epi) {
      case EPI_SQRELU_Q8: return launch_epi<BM, BN, 0, WGM, WGN, EPI_SQRELU_Q8, false>(a, wt, grid, num_cu, s);
      case EPI_F32: return launch_epi<BM, BN, 0, WGM, WGN, EPI_F32, false>(a, wt, grid, num_cu, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_SQRELU_BF16: return launch_epi<BM, BN, 0, WGM, WGN, EPI_SQRELU_BF16, false>(a, wt, grid, num_cu, s);
    case EPI_BF16: return launch_epi<BM, BN, 0, WGM, WGN, EPI_BF16, false>(a, wt, grid, num_cu, s);
    case EPI_Z: return launch_epi<BM, BN, 0, WGM, WGN, EPI_Z, false>(a, wt, grid, num_cu, s);
    case EPI_Z8: return launch_epi<BM, BN, 0, WGM, WGN, EPI_Z8, false>(a, wt, grid, num_cu, s);
    case EPI_Q8: return launch_epi<BM, BN, 0, WGM, WGN, EPI_Q8, false>(a, wt, grid, num_cu, s);
    case EPI_F32: return launch_epi<BM, BN, 0, WGM, WGN, EPI_F32, false>(a, wt, grid, num_cu, s);
    case EPI_BF16_ADD: return launch_epi<BM, BN, 0, WGM, WGN, EPI_BF16_ADD, false>(a, wt, grid, num_cu, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace {
template <int BK, int EPI>
hipError_t launch_fp4_rem_one(const GemmArgs& a, int64_t max_items, int num_cu, hipStream_t s) {
  using C = TileCfg<128, 256, BK, 1, 4, 2, WT_NVFP4>;
  static_assert(C::LDS <= 80 * 1024, "two blocks per CU");
  auto* kern = gemm_fp4_rem_kernel<BK, 2, EPI>;
  if (a.K / BK < 2) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  const int64_t cap = ((int64_t)num_cu * 2) & ~7LL;
  int grid = (int)(max_items < cap ? max_items : cap);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), C::LDS, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_fp4_rem(const GemmArgs& a, int epi, int64_t max_items, int num_cu, hipStream_t s) {
  if (!a.tiles2 || !a.n_tiles) return hipErrorInvalidValue;
  const bool wide = a.K >= 128;
  switch (epi) {
    case EPI_SQRELU_BF16:
      return wide ? launch_fp4_rem_one<64, EPI_SQRELU_BF16>(a, max_items, num_cu, s)
                  : launch_fp4_rem_one<32, EPI_SQRELU_BF16>(a, max_items, num_cu, s);
    case EPI_BF16:
      return wide ? launch_fp4_rem_one<64, EPI_BF16>(a, max_items, num_cu, s)
                  : launch_fp4_rem_one<32, EPI_BF16>(a, max_items, num_cu, s);
    default:
      return hipErrorInvalidValue;
  }
}

// Tile shapes: 256x256 (8 wavefronts, 2x4; 1x8 for grouped NVFP4 weights),
// 256x128 and 128x128 (4 wavefronts, 2x2).  Dense (a.tiles == nullptr): bms must be 0.  Grouped: list 0 of height
// bm, list 1 of height bms; max_items bounds the items for the grid size.
hipError_t launch_gemm_bf16(const GemmArgs& a0, int wt, int epi, int bm, int bn, int bms,
                            int64_t max_items, int num_cu, hipStream_t s) {
  if (!a0.tiles && bms != 0) return hipErrorInvalidValue;
  GemmArgs a = a0;
  if (wt == WT_FP8) {
    // two codes per 16-bit slot: the loads and the LDS layout of a bf16 GEMM
    // over K / 2
    if ((a.K | a.lda | a.ldb | a.b_gstride) & 1) return hipErrorInvalidValue;
    if (a.kseg < a.K && ((a.kseg | a.b_segstride) & 1)) return hipErrorInvalidValue;
    a.K /= 2; a.lda /= 2; a.ldb /= 2; a.b_gstride /= 2;
    if (a0.kseg < a0.K) { a.kseg /= 2; a.b_segstride /= 2; }
  }
  const int64_t total = a.tiles ? max_items
                                : (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  if (!a.tiles) {
    if (bm == 256 && bn == 256) return launch_shape<256, 256, 0, 2, 4>(a, wt, epi, total, num_cu, s);
    if (bm == 256 && bn == 128) return launch_shape<256, 128, 0, 2, 2>(a, wt, epi, total, num_cu, s);
    if (bm == 128 && bn == 128) return launch_shape<128, 128, 0, 2, 2>(a, wt, epi, total, num_cu, s);
    return hipErrorInvalidValue;
  }
  // NVFP4 weights: the 8 wavefronts side by side along the weight columns
  // (wavefront tile 256 x 32), so each decoded B fragment feeds 8 MFMAs
  // instead of 4 and every weight element is decoded once per tile, at twice
  // the A-fragment LDS reads (measured 3.5% faster than 2 x 4 on the Ultra-like
  // NVFP4 prefill's grouped GEMMs)
  if (bm == 256 && bn == 256 && bms == 128 && wt == WT_NVFP4)
    return launch_shape<256, 256, 128, 1, 8>(a, wt, epi, total, num_cu, s);
  if (bm == 256 && bn == 256 && bms == 128) return launch_shape<256, 256, 128, 2, 4>(a, wt, epi, total, num_cu, s);
  if (bm == 128 && bn == 128 && bms == 64) return launch_shape<128, 128, 64, 2, 2>(a, wt, epi, total, num_cu, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
