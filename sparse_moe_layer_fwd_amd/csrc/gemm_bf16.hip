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
// section 2.4 NVFP4 Training) are decoded exactly to bf16 inside LDS once per
// block and k-tile (every e2m1*e4m3 product is a bf16 value); the global scale
// multiplies the fp32 accumulator in the epilogue.
//
// Data movement: operands go global -> LDS with gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16*lane)
// through a ring of NST stages, so NST-1 k-tiles are in flight while one is
// multiplied and no VGPRs are spent on staging.  Each wavefront waits for its
// own loads with an explicit vmcnt, then a bare s_barrier publishes the stage.
// LDS rows hold BK bf16 as 16-byte chunks; chunk c of row r sits at c ^ f(r),
// which spreads the fragment reads of 8 or 16 consecutive rows over distinct
// bank groups.  The swizzle is applied on the global side (which chunk a lane
// fetches) because the LDS side of a direct load is fixed by the lane id.
//
// Tile BM x BN, WGM x WGN wavefronts, each owning (BM/WGM) x (BN/WGN) in 32x32
// MFMA blocks.  The MFMA computes C^T (weights as the A operand, activations as
// the B operand) so each lane holds 4 consecutive output columns of one row:
// 8- or 16-byte stores.
#include "common.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}
// 4-byte direct load (sub-dword LDS-DMA forms are not used: their LDS placement
// is not the 2- or 1-byte lane stride the packed layouts here would need)
template <int BYTES>
__device__ __forceinline__ void dma_small(const void* g, void* lds_wave_base) {
  static_assert(BYTES == 4, "dword LDS-DMA only");
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 4, 0, 0);
}

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

// NVFP4 decode with the gfx950 conversion v_cvt_scalef32_pk_bf16_fp4, which
// turns one byte (two E2M1 codes, low nibble first) into two bf16 multiplied by
// the power of two in its scale operand (only the scale's exponent is used).
// The E4M3 block scale s = 2^E * f is applied as 2^E in the conversion and f
// (a 4-bit significand with s's sign) as one fp32 multiply; both steps are
// exact because every e2m1 * e4m3 product fits in bf16.
struct Fp4Scale {
  float pow2, frac;
};
__device__ __forceinline__ Fp4Scale split_scale(uint32_t e4m3) {
  const float s = e4m3_to_f32(e4m3);
  const uint32_t b = __float_as_uint(s);
  Fp4Scale r;
  r.pow2 = __uint_as_float(b & 0x7F800000u);
  r.frac = s == 0.0f ? 0.0f : __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u);
  return r;
}
template <int BYTE>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, const Fp4Scale& sc) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const uint32_t pr = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc.pow2, BYTE));
  const float lo = __uint_as_float(pr << 16) * sc.frac;
  const float hi = __uint_as_float(pr & 0xFFFF0000u) * sc.frac;
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
// 8 codes (one dword) -> 8 bf16 (one uint4)
__device__ __forceinline__ uint4 fp4x8(uint32_t w, const Fp4Scale& sc) {
  return make_uint4(fp4_pair<0>(w, sc), fp4_pair<1>(w, sc), fp4_pair<2>(w, sc), fp4_pair<3>(w, sc));
}

}  // namespace

template <int BM, int BN, int BK, int WGM, int WGN, int NST, bool FP4>
struct TileCfg {
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per bf16 row
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int BQ_BYTES = BN * BK / 2;                 // NVFP4 codes
  static constexpr int BS_BYTES = BN * 4;                      // NVFP4 scales: one aligned dword per row
  static constexpr int B_BYTES = FP4 ? BQ_BYTES + BS_BYTES : BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int BDQ = FP4 ? BN * BK * 2 : 0;            // decoded B (double-buffered)
  static constexpr int LDS = NST * STAGE + 2 * BDQ;
  static constexpr int A_TOT = BM * CPR / 64;                  // 1 KB DMA blocks per k-tile
  static constexpr int B_TOT = FP4 ? BQ_BYTES / 1024 : BN * CPR / 64;
  static constexpr int S_TOT = FP4 ? BS_BYTES / 256 : 0;       // dword-per-lane DMA blocks
  static constexpr int A_PW = (A_TOT + NW - 1) / NW;           // per wavefront
  static constexpr int B_PW = (B_TOT + NW - 1) / NW;
  static constexpr int S_PW = (S_TOT + NW - 1) / NW;
  static constexpr int LOADS = A_PW + B_PW + S_PW;             // vm ops per wave per k-tile
  static_assert(A_TOT >= 1 && B_TOT >= 1 && (!FP4 || S_TOT >= 1), "tile too small");
  static_assert(LOADS * (NST - 2) < 64, "vmcnt range");
  static_assert(STAGE % 16 == 0, "stage alignment");
};

// One output tile: rows [r0, r1) (r1 - r0 <= BM) of group g, columns [n0, n0 + BN).
template <int BM, int BN, int BK, int WGM, int WGN, int NST, bool FP4, int EPI>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, char* smem, int g, int r0, int r1,
                                          int n0) {
  using C = TileCfg<BM, BN, BK, WGM, WGN, NST, FP4>;
  constexpr int CPR = C::CPR, NW = C::NW;
  constexpr int WM = BM / WGM, WN = BN / WGN;      // wavefront tile
  constexpr int TM = WM / 32, TN = WN / 32;        // 32x32 MFMA blocks per wavefront
  constexpr int S_PW1 = C::S_PW > 0 ? C::S_PW : 1;
  constexpr int S_TOT1 = C::S_TOT > 0 ? C::S_TOT : 1;
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int nk = p.K / BK;

  // the previous tile's stores must not be counted as in-flight loads below
  wait_vm<0>();

  // ---- per-lane global offsets of this lane's chunks (32-bit, from uniform bases)
  const uint16_t* Abase = (const uint16_t*)p.A;
  uint32_t aoff[C::A_PW];
#pragma unroll
  for (int j = 0; j < C::A_PW; ++j) {
    const int blk = (wave + j * NW) % C::A_TOT;
    const int q = blk * 64 + lane;                 // LDS chunk index in the A region
    const int row = q / CPR, pos = q % CPR;
    const int lr = min(r0 + row, r1 - 1);          // rows past the end re-read the last row
    const uint32_t pr = p.a_rows ? (uint32_t)p.a_rows[lr] : (uint32_t)lr;
    aoff[j] = pr * (uint32_t)p.lda + swz_chunk<CPR>(row, pos) * 8;
  }
  const char* Bbase = FP4 ? (const char*)p.B + (int64_t)g * p.b_gstride
                          : (const char*)((const uint16_t*)p.B + (int64_t)g * p.b_gstride);
  const char* Sbase = FP4 ? (const char*)p.b_scale + (int64_t)g * p.s_gstride : nullptr;
  uint32_t boff[C::B_PW], soff[S_PW1];
#pragma unroll
  for (int j = 0; j < C::B_PW; ++j) {
    const int blk = (wave + j * NW) % C::B_TOT;
    if (FP4) {                                     // BK/32 chunks of codes per row, unswizzled
      constexpr int QPR = BK / 32;
      const int q = blk * 64 + lane, row = q / QPR, pos = q % QPR;
      const uint32_t n = (uint32_t)min(n0 + row, p.N - 1);
      boff[j] = n * (uint32_t)p.ldb + pos * 16;    // bytes
    } else {
      const int q = blk * 64 + lane, row = q / CPR, pos = q % CPR;
      const uint32_t n = (uint32_t)min(n0 + row, p.N - 1);
      boff[j] = n * (uint32_t)p.ldb + swz_chunk<CPR>(row, pos) * 8;   // elements
    }
  }
#pragma unroll
  for (int j = 0; j < S_PW1; ++j) {
    const int blk = (wave + j * NW) % S_TOT1;
    const uint32_t n = (uint32_t)min(n0 + blk * 64 + lane, p.N - 1);
    soff[j] = n * (uint32_t)p.lds_scale;           // bytes; the k-tile's BK/16 scale bytes sit in
                                                   // the aligned dword loaded per row
  }

  // ---- issue the direct-to-LDS loads of k-tile kt into stage st
#define MOE_ISSUE(KT, ST)                                                                     \
  do {                                                                                        \
    char* S_ = smem + (ST) * C::STAGE;                                                        \
    const uint32_t k0_ = (uint32_t)(KT) * BK;                                                 \
    _Pragma("unroll") for (int j = 0; j < C::A_PW; ++j) {                                     \
      const int blk = (wave + j * NW) % C::A_TOT;                                             \
      dma16(Abase + (aoff[j] + k0_), S_ + blk * 1024);                                        \
    }                                                                                         \
    if (FP4) {                                                                                \
      _Pragma("unroll") for (int j = 0; j < C::B_PW; ++j) {                                   \
        const int blk = (wave + j * NW) % C::B_TOT;                                           \
        dma16(Bbase + (boff[j] + k0_ / 2), S_ + C::A_BYTES + blk * 1024);                     \
      }                                                                                       \
      _Pragma("unroll") for (int j = 0; j < C::S_PW; ++j) {                                   \
        const int blk = (wave + j * NW) % S_TOT1;                                             \
        dma_small<4>(Sbase + ((soff[j] + k0_ / 16) & ~3u), S_ + C::A_BYTES + C::BQ_BYTES + blk * 256); \
      }                                                                                       \
    } else {                                                                                  \
      const uint16_t* Bk_ = (const uint16_t*)Bbase + k0_;                                     \
      if (p.kseg < p.K) {             /* B stored as k segments (shared experts' W2) */       \
        const int seg_ = (int)(k0_ / (uint32_t)p.kseg);                                       \
        Bk_ = (const uint16_t*)Bbase + (int64_t)seg_ * p.b_segstride +                        \
              (k0_ - (uint32_t)seg_ * p.kseg);                                                \
      }                                                                                       \
      _Pragma("unroll") for (int j = 0; j < C::B_PW; ++j) {                                   \
        const int blk = (wave + j * NW) % C::B_TOT;                                           \
        dma16(Bk_ + boff[j], S_ + C::A_BYTES + blk * 1024);                                   \
      }                                                                                       \
    }                                                                                         \
  } while (0)

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // ---- NVFP4: decode raw k-tile KT (stage KT % NST) into bf16 buffer KT & 1
#define MOE_DECODE(KT)                                                                        \
  do {                                                                                        \
    const char* S_ = smem + ((KT) % NST) * C::STAGE;                                          \
    uint4* D_ = reinterpret_cast<uint4*>(smem + NST * C::STAGE + ((KT) & 1) * C::BDQ);         \
    const uint8_t* Q_ = reinterpret_cast<const uint8_t*>(S_ + C::A_BYTES);                    \
    const uint8_t* Sc_ = Q_ + C::BQ_BYTES;                                                    \
    constexpr int UNITS = BN * BK / 16;             /* one 16-code block per unit */            \
    _Pragma("unroll") for (int u0 = 0; u0 < UNITS; u0 += C::NT) {                             \
      const int u = u0 + tid;                                                                 \
      if (UNITS % C::NT == 0 || u < UNITS) {                                                  \
        const int row = u / (BK / 16), blk = u % (BK / 16);                                   \
        const uint2 q = *reinterpret_cast<const uint2*>(Q_ + row * (BK / 2) + blk * 8);       \
        const Fp4Scale sc = split_scale(Sc_[row * 4 + (((KT) * (BK / 16)) & 3) + blk]);       \
        D_[row * CPR + swz_chunk<CPR>(row, 2 * blk + 0)] = fp4x8(q.x, sc);                    \
        D_[row * CPR + swz_chunk<CPR>(row, 2 * blk + 1)] = fp4x8(q.y, sc);                    \
      }                                                                                       \
    }                                                                                         \
  } while (0)
  // wait until this wavefront's loads of some k-tile are done, given that at
  // most `pending` later k-tiles' loads may stay in flight (in-order completion)
#define MOE_WAIT(PENDING)                                                                     \
  do {                                                                                        \
    const int pd_ = (PENDING);                                                                \
    if (NST >= 4 && pd_ >= 2) wait_vm<(NST >= 4 ? 2 : 0) * C::LOADS>();                       \
    else if (pd_ >= 1) wait_vm<C::LOADS>();                                                   \
    else wait_vm<0>();                                                                        \
  } while (0)

#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) MOE_ISSUE(s, s);
  if (FP4) {                                        // decode k-tile 0 ahead of the loop
    MOE_WAIT(min(nk - 1, NST - 2));
    bar();
    MOE_DECODE(0);
  }

  for (int kt = 0; kt < nk; ++kt) {
    // bf16: k-tile kt must have landed.  NVFP4: the raw codes of kt + 1 too,
    // because they are decoded while k-tile kt is multiplied.
    const int need = FP4 ? min(kt + 1, nk - 1) : kt;
    MOE_WAIT(min(nk - 1 - need, NST - 2));
    if (FP4) bar_lds(); else bar();                 // stages (and decoded B) complete for all waves
    if (kt + NST - 1 < nk) MOE_ISSUE(kt + NST - 1, (kt + NST - 1) % NST);
    if (FP4 && kt + 1 < nk) MOE_DECODE(kt + 1);
    const char* S = smem + (kt % NST) * C::STAGE;
    const uint4* As = reinterpret_cast<const uint4*>(S);
    const uint4* Bs = FP4 ? reinterpret_cast<const uint4*>(smem + NST * C::STAGE + (kt & 1) * C::BDQ)
                          : reinterpret_cast<const uint4*>(S + C::A_BYTES);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ch = s * 2 + (lane >> 5);
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        a[i] = __builtin_bit_cast(bf16x8, As[row * CPR + swz_chunk<CPR>(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = wn * WN + j * 32 + (lane & 31);
        b[j] = __builtin_bit_cast(bf16x8, Bs[n * CPR + swz_chunk<CPR>(n, ch)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[j][i], 0, 0, 0);
    }
  }
#undef MOE_DECODE
#undef MOE_WAIT
#undef MOE_ISSUE
  bar_lds();   // every wave is done with the stages before the next tile's loads land

  // epilogue.  acc[j][i][r] = C[row][col] with row = i-block row (lane & 31),
  // col = j-block column 8*(r/4) + 4*(lane/32) + r%4: 4 consecutive columns per r/4.
  const float gs = (FP4 && p.b_gscale) ? p.b_gscale[g] : 1.0f;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = r0 + wm * WM + i * 32 + (lane & 31);
    if (row >= r1) continue;
    float rsc = gs;
    if (EPI == EPI_GATE_BF16) rsc *= p.row_scale[row];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
        if (col >= p.N) continue;
        float v0 = acc[j][i][4 * q + 0], v1 = acc[j][i][4 * q + 1];
        float v2 = acc[j][i][4 * q + 2], v3 = acc[j][i][4 * q + 3];
        const int64_t o = (int64_t)row * p.ldc + col;
        if (EPI == EPI_SQRELU_BF16) {
          v0 = fmaxf(v0 * gs, 0.f); v1 = fmaxf(v1 * gs, 0.f);
          v2 = fmaxf(v2 * gs, 0.f); v3 = fmaxf(v3 * gs, 0.f);
          v0 *= v0; v1 *= v1; v2 *= v2; v3 *= v3;
        } else {
          v0 *= rsc; v1 *= rsc; v2 *= rsc; v3 *= rsc;
        }
        if (EPI == EPI_F32) {
          *reinterpret_cast<float4*>((float*)p.C + o) = make_float4(v0, v1, v2, v3);
        } else if (EPI == EPI_Z) {
          *reinterpret_cast<float4*>((float*)p.C + o) = make_float4(v0, v1, v2, v3);
          *reinterpret_cast<uint2*>((uint16_t*)p.C2 + (int64_t)row * p.ldc2 + col) =
              make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
        } else {
          if (EPI == EPI_BF16_ADD) {
            const float4 ad = *reinterpret_cast<const float4*>(p.add + (int64_t)row * p.ld_add + col);
            v0 += ad.x; v1 += ad.y; v2 += ad.z; v3 += ad.w;
          }
          *reinterpret_cast<uint2*>((uint16_t*)p.C + o) =
              make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
        }
      }
    }
  }
}

// Persistent kernel over (row tile, column tile) items.  List 0 holds row tiles
// of height <= BM (p.tiles / n_tiles[0], or the dense row blocks); list 1, when
// BMS > 0, holds row tiles of height <= BMS (p.tiles2 / n_tiles[1]): the
// remainders of each expert's rows, processed with a shorter tile.
template <int BM, int BN, int BMS, int BK, int WGM, int WGN, int NST, bool FP4, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmArgs p) {
  extern __shared__ uint4 smem_u4[];
  char* smem = reinterpret_cast<char*>(smem_u4);
  const int ntn = (p.N + BN - 1) / BN;
  const int nrt0 = p.tiles ? p.n_tiles[0] : (p.M + BM - 1) / BM;
  const int nrt1 = BMS > 0 ? p.n_tiles[1] : 0;
  const int items0 = nrt0 * ntn;
  const int total = items0 + nrt1 * ntn;
  // Consecutive items (the column tiles of one row tile, then the next row
  // tiles of the same expert) go to blocks of the same XCD, which share an L2:
  // block b runs on XCD b % 8, so it takes the items of slice b % 8 of each
  // round of gridDim.x items.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = G >> 3;
  const int base = (G & 7) == 0 ? xcd * per_xcd + slot : blockIdx.x;
  for (int round = 0; round * G < total; ++round) {
    const int item = round * G + base;
    if (item >= total) continue;
    int it = item;
    const int4* list = p.tiles;
    if (it >= items0) { it -= items0; list = p.tiles2; }
    int rt = it / ntn, nt = it - rt * ntn;
    if (!list && ntn > 8) {
      // dense and wide: walk bands of 4 row tiles column by column, so the 32
      // consecutive items of one XCD reuse 4 A and 8 B strips from its L2
      const int band = it / (4 * ntn), in = it - band * 4 * ntn;
      const int rows = min(4, nrt0 - band * 4);
      rt = band * 4 + in % rows;
      nt = in / rows;
    }
    int g = 0, r0, r1;
    if (list) {
      const int4 tl = list[rt];
      g = tl.x; r0 = tl.y; r1 = tl.z;
    } else {
      r0 = rt * BM; r1 = min(p.M, r0 + BM);
    }
    if constexpr (BMS > 0) {
      if (item >= items0) {
        gemm_tile<BMS, BN, BK, WGM, WGN, NST, FP4, EPI>(p, smem, g, r0, r1, nt * BN);
        continue;
      }
    }
    gemm_tile<BM, BN, BK, WGM, WGN, NST, FP4, EPI>(p, smem, g, r0, r1, nt * BN);
  }
}

namespace {

template <int BM, int BN, int BMS, int BK, int WGM, int WGN, int NST, bool FP4, int EPI>
hipError_t launch_one(const GemmArgs& a, int64_t total, int num_cu, hipStream_t s) {
  constexpr size_t lds = (size_t)TileCfg<BM, BN, BK, WGM, WGN, NST, FP4>::LDS;
  static_assert(lds <= 160 * 1024, "LDS");
  auto* kern = gemm_bf16_kernel<BM, BN, BMS, BK, WGM, WGN, NST, FP4, EPI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // persistent grid: as many blocks as fit at once (a multiple of the 8 XCDs)
  const int per_cu = (int)((160 * 1024) / lds);
  const int64_t cap = ((int64_t)num_cu * (per_cu > 0 ? per_cu : 1)) & ~7LL;
  int grid = (int)(total < cap ? total : cap);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WGM * WGN), lds, s, a);
  return hipGetLastError();
}

// bf16: BK = 64 (fewer barriers per flop) with 2 stages for 256x256 tiles
// and 3 for the smaller ones.  NVFP4: BK = 32 with a 4-stage ring; the codes and
// scales are staged raw and decoded in LDS one k-tile ahead of the MFMAs.
template <int BM, int BN, int BMS, int WGM, int WGN>
hipError_t launch_shape(const GemmArgs& a, bool fp4, int epi, int64_t grid, int num_cu, hipStream_t s) {
  constexpr int NSTB = (BM == 256 && BN == 256) ? 2 : 3;
  if (fp4) {
    if (a.tiles) {              // NVFP4 is used for the grouped expert GEMMs only
      switch (epi) {
        case EPI_SQRELU_BF16: return launch_one<BM, BN, BMS, 32, WGM, WGN, 4, true, EPI_SQRELU_BF16>(a, grid, num_cu, s);
        case EPI_GATE_BF16: return launch_one<BM, BN, BMS, 32, WGM, WGN, 4, true, EPI_GATE_BF16>(a, grid, num_cu, s);
        default: break;
      }
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_SQRELU_BF16: return launch_one<BM, BN, BMS, 64, WGM, WGN, NSTB, false, EPI_SQRELU_BF16>(a, grid, num_cu, s);
    case EPI_GATE_BF16: return launch_one<BM, BN, BMS, 64, WGM, WGN, NSTB, false, EPI_GATE_BF16>(a, grid, num_cu, s);
    default: break;
  }
  if (BMS != 0) return hipErrorInvalidValue;     // dense epilogues have no tile lists
  switch (epi) {
    case EPI_BF16: return launch_one<BM, BN, 0, 64, WGM, WGN, NSTB, false, EPI_BF16>(a, grid, num_cu, s);
    case EPI_Z: return launch_one<BM, BN, 0, 64, WGM, WGN, NSTB, false, EPI_Z>(a, grid, num_cu, s);
    case EPI_F32: return launch_one<BM, BN, 0, 64, WGM, WGN, NSTB, false, EPI_F32>(a, grid, num_cu, s);
    case EPI_BF16_ADD: return launch_one<BM, BN, 0, 64, WGM, WGN, NSTB, false, EPI_BF16_ADD>(a, grid, num_cu, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Tile shapes: 256x256 (8 wavefronts, 2x4), 256x128 and 128x128 (4 wavefronts,
// 2x2).  Dense (a.tiles == nullptr): bms must be 0.  Grouped: list 0 of height
// bm, list 1 of height bms; max_items bounds the items for the grid size.
hipError_t launch_gemm_bf16(const GemmArgs& a, bool b_nvfp4, int epi, int bm, int bn, int bms,
                            int64_t max_items, int num_cu, hipStream_t s) {
  if (!a.tiles && bms != 0) return hipErrorInvalidValue;
  const int64_t total = a.tiles ? max_items
                                : (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  if (!a.tiles) {
    if (bm == 256 && bn == 256) return launch_shape<256, 256, 0, 2, 4>(a, b_nvfp4, epi, total, num_cu, s);
    if (bm == 256 && bn == 128) return launch_shape<256, 128, 0, 2, 2>(a, b_nvfp4, epi, total, num_cu, s);
    if (bm == 128 && bn == 128) return launch_shape<128, 128, 0, 2, 2>(a, b_nvfp4, epi, total, num_cu, s);
    return hipErrorInvalidValue;
  }
  if (bm == 256 && bn == 256 && bms == 0) return launch_shape<256, 256, 0, 2, 4>(a, b_nvfp4, epi, total, num_cu, s);
  if (bm == 256 && bn == 256 && bms == 128) return launch_shape<256, 256, 128, 2, 4>(a, b_nvfp4, epi, total, num_cu, s);
  if (bm == 256 && bn == 128 && bms == 64) return launch_shape<256, 128, 64, 2, 2>(a, b_nvfp4, epi, total, num_cu, s);
  if (bm == 128 && bn == 128 && bms == 64) return launch_shape<128, 128, 64, 2, 2>(a, b_nvfp4, epi, total, num_cu, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
