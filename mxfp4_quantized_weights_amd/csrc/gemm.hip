// Grouped expert GEMMs on MFMA (gfx950) and the routing-weighted combine.
//
// sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4 MoE
// on gfx950", Summary: gate and up projections are separate contiguous halves
// of w13 (rows [0, Ip) and [Ip, 2Ip)); the SwiGLU is clamped
// (swiglu_limit); block FP8 [128,128] weights with dynamic FP8 activations,
// or OCP MXFP4 1x32 weights and activations.  FreeToken PR #270
// "glm5_next: support GLM-5.3-Flash (hybrid KDA + DSA, mHC, NVFP4 expert
// offload)", Summary: silu(min(gate, lim)) * clamp(up, -lim, lim).
//
// Work decomposition.  An item is one (M block, N tile): block_m rows of the
// expert-sorted pair list (all of one expert) times 256 weight rows.
//   GEMM1: the N tile is 128 intermediate columns = 128 gate rows and the
//          matching 128 up rows of w13, so a lane holds the gate and up value
//          of the same column and the 1x128 requantisation group is whole.
//   GEMM2: the N tile is 256 output columns.
// One persistent workgroup per CU walks a list of items (the moe_gemm_stream
// kernel below); weight tiles and gathered activation rows stream into LDS.
//   FP8: each 128-wide K block is one scale block, so its fp32 partial sum is
//        scaled by act_scale(row) * w_scale(block) and added to the
//        accumulator (fp32 promotion per K block).  GEMM1 widens the FP8
//        operands to f16 and uses the f16 MFMA (exact fp32 sums); GEMM2 uses
//        the FP8 MFMA directly.
//   MX:  the scaled MFMA applies the E8M0 scales of both operands itself.
//   UE8M0 FP8 ("[AMD] [GLM5] Opt-in prefill-only FP8 dense projection GEMM
//        for MLA q_b/o_proj (gfx950)", Modifications: 128x128 UE8M0 weight
//        scales; 1x128 UE8M0 activation scales here): GEMM1 as block FP8
//        (f16 MFMA, promotion by the exact power-of-two scale product) with
//        UE8M0 re-quantisation; GEMM2 on the scaled FP8 MFMA, which applies
//        both power-of-two scales itself, so there is no promotion at all.
#include <math.h>

#include <utility>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Operand modes of the GEMM kernels (template parameter MODE).
constexpr int kGemmFp8 = 1;     // FP8 MFMA, fp32 promotion per K block, fp32 activation scales
constexpr int kGemmMx = 2;      // scaled FP4 MFMA, E8M0 scales per 1x32
constexpr int kGemmFp8F16 = 3;  // FP8 widened to f16, f16 MFMA, fp32 promotion, fp32 activation scales
constexpr int kGemmE8F16 = 4;   // as kGemmFp8F16 with UE8M0 activation-scale bytes
constexpr int kGemmE8 = 5;      // scaled FP8 MFMA with UE8M0 bytes for both operands, no promotion
static_assert(kGemmMx == kQuantMx, "MX tiles are sized by the quant mode");

// Activation scales arrive as E8M0 bytes (a dword holds 4 K blocks).
constexpr bool e8_tokens(int mode) { return mode == kGemmE8F16 || mode == kGemmE8; }
// FP8 operands widened to f16 for the f16 MFMA.
constexpr bool f16_path(int mode) { return mode == kGemmFp8F16 || mode == kGemmE8F16; }

// ===========================================================================
// The load ring and the per-K-block compute.
//
// Operands go from HBM to LDS with direct global->LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16*l), through a
// ring of S K-block slots, so S-1 K blocks are in flight per workgroup without
// holding them in registers.  The weight tiles are copied verbatim from the
// TILED_V2 layout, which already is MFMA fragment order and holds an item's
// 16 tiles of one K block as one contiguous run; the gathered token
// rows are placed in the same order by the per-lane source addresses.  Every
// wave issues the same number of loads per slot, so one s_waitcnt vmcnt(N)
// per K block plus a barrier make the slot visible to all waves.
//
// The MFMA runs transposed: the weight tile is operand A and the 16 tokens are
// operand B, so lane l holds 4 consecutive weight rows (output columns) of one
// token.  For block FP8 those 4 values share one 128x128 weight scale, and the
// per-K-block promotion costs one fma per output value.
//
// Waves: (wt, wn) = (wave / 4, wave % 4); wt picks 64 tokens (4 row tiles; a
// block of fewer than 64 rows has one token group), wn the wave's 4 weight
// tiles: GEMM1 gate tiles 2wn, 2wn+1 and the matching up tiles 8+2wn, 9+2wn
// of the N tile; GEMM2 tiles 4wn .. 4wn+3.
// ===========================================================================
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// A tail launch over W workgroups splits its leftover items (items mod W)
// only when they fill at most half a round: a lightly filled last round
// streams faster than a full one, and splitting a fuller one costs more in
// pieces and partial sums than it saves (decode, one MI355X: T = 16, 32, 64
// with 28-31% of a round left gain 1-5%; 69-82% left lose 2-14%).
__host__ __device__ inline bool tail_split_on(int items, int W) { return 2 * (items % W) <= W; }

// Kernel instances by split (template argument SPLIT): none; a K split of
// every item; a tail launch (GEMM1).  Each carries only its own epilogues,
// which keeps the plain and K-split kernels' register use as it is.
constexpr int kNoSplit = 0, kKSplit = 1, kTailSplit = 2;

// Waves of a workgroup: 4 column waves (the N tile's 16 weight tiles, 4 each)
// times WT token groups: BM/64 groups of 64 tokens (4 token tiles per wave)
// for BM >= 64, one group of BM/16 tiles below.  A wave multiplies MT token
// tiles by its 4 weight tiles.  (One group of 8 token tiles at BM = 128 --
// 1.5 instead of 2 FP8->f16 converts per MFMA on GEMM1's f16 path, one wave
// per SIMD -- measured 40% slower on the 4096-token prefill layer: the
// accumulators of 32 tiles leave too few registers, so MFMA partial sums go
// through AGPRs and the MFMA chains serialise.)
constexpr int ring_waves(int mode, int bm) {
  return (void)mode, bm >= 64 ? bm / 16 : 4;
}

template <int MODE, int BM>
struct Ring {
  static constexpr int NWAVE = ring_waves(MODE, BM);
  static constexpr int NTH = NWAVE * 64;
  static constexpr int TT = BM / 16;                             // token tiles per slot
  static constexpr int WT = NWAVE / 4;                           // token groups
  static constexpr int MT = TT / WT;                             // token tiles per wave
  static constexpr int MTH = MT >= 4 ? MT / 4 : 1;               // 64-token scale words per wave
  static constexpr int TILE = (MODE == kGemmMx) ? 1024 : 2048;  // one 16 x 128 operand tile
  static constexpr int HALVES = TILE / 1024;
  static constexpr int AROW = (MODE == kGemmMx) ? 64 : 128;     // token bytes per K block
  static constexpr int W_OFF = 0;                                // 16 weight tiles
  static constexpr int T_OFF = 16 * TILE;                        // TT token tiles
  static constexpr int TS_OFF = T_OFF + TT * TILE;               // token scales, 256 B per 64 tokens
  static constexpr int NTS = BM >= 64 ? BM / 64 : 1;
  static constexpr int TSW = 4 * NTS / NWAVE > 1 ? 4 * NTS / NWAVE : 1;  // 16-scale chunks per wave
  static constexpr int WSC_OFF = TS_OFF + NTS * 256;            // FP8: the K block's two weight scales
  static constexpr int SLOT = WSC_OFF + 16;
  static constexpr int WS_BYTES = 16 * 256;                      // MX: one group of weight scale dwords
  static constexpr int DW = 16 * HALVES / NWAVE;                 // weight loads per wave per slot
  static constexpr int NTD = TT * HALVES;                        // token loads per slot
  static constexpr int DT = (NTD + NWAVE - 1) / NWAVE;           // ... per wave (BM < 64: waves < NTD)
  static constexpr int DWS = (MODE == kGemmMx) ? 16 / NWAVE : 0;  // every 4th K block only
  // loads every wave issues in every K block (waits use this minimum; waves
  // that issue more only wait longer)
  static constexpr int D = DW + NTD / NWAVE + TSW;
  static_assert(16 * HALVES % NWAVE == 0 && (NTD % NWAVE == 0 || NTD < NWAVE), "load split");
};

// Direct global->LDS loads, written as inline assembly so that the compiler's
// automatic wait insertion does not see them (it would add vmcnt(0) in front
// of every LDS read of the ring); the kernel waits for them itself.  M0 holds
// the wave-uniform LDS base (one wait state before the load reads it); every
// caller's base is uniform by construction, and readfirstlane states it for
// bases the compiler cannot prove uniform (those that go through the item
// cursors).  The
// weight loads carry the non-temporal hint: weights are read once per launch.
#pragma clang diagnostic push
// M0 is reserved by the compiler, which cannot see these writes; the library
// relies on no compiler-generated code using M0 (no register-indexed moves,
// messages, GWS or buffer-to-LDS loads), which the test suite checks on the
// disassembly of the built code objects.
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wait until at most N of this wave's vector-memory loads are outstanding and
// its LDS operations are complete, then barrier.  The "memory" clobber keeps
// the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The same with at most min(later, R) * D loads left outstanding: the wait
// for a ring slot after which only `later` (wave-uniform) slots were issued.
template <int R, int D>
__device__ __forceinline__ void vm_wait_barrier_upto(int later) {
  if constexpr (R == 0) {
    vm_wait_barrier<0>();
  } else {
    if (later >= R)
      vm_wait_barrier<R * D>();
    else
      vm_wait_barrier_upto<R - 1, D>(later);
  }
}


// Per-lane source addresses of one wave's loads at K block 0.
template <int MODE, int BM>
struct RingSrc {
  using R = Ring<MODE, BM>;
  const uint8_t* w[R::DW];
  const uint8_t* t[R::DT];
  const uint8_t* ts[R::TSW];
  const uint8_t* ws[R::DWS > 0 ? R::DWS : 1];
  const uint8_t* wsc;  // FP8, lanes 0 and 1 of the last wave: weight-scale row of K block 0
  int wk;              // bytes between a weight tile's K blocks (tile run x tile bytes)
  int wsk;             // MX: bytes between a scale word row's groups of 4 K blocks
};

// Loads of K block kb into `slot`.  Token scales: chunk c (16 scales, 4 per
// 64-token group) is fetched by wave c / TSW (lanes 0..15 only), placed so
// that lane l of a compute wave finds the scales of 4 token tiles m, row
// l % 16, in one 16-byte word per 64 tokens.  FP8 weight scales: the last wave fetches the K block's two
// fp32 block scales (lanes 0 and 1).  MX weight scales (one dword holds 4 K
// blocks) are fetched only when `ws` is non-null, into that buffer.
// `part` (0..3) issues one of four groups of the loads: the first and second
// half of the weight loads, the token loads and token scales, and the weight
// scales; -1 issues all.  The compute interleaves the parts with its own
// work (ring_compute), so the loads of one K block do not queue up in front
// of the vector memory unit all at once.
template <int MODE, int BM>
__device__ __forceinline__ void ring_issue(const RingSrc<MODE, BM>& src, const uint8_t* slot, int wave, int kb,
                                           const uint8_t* ws, int part = -1) {
  using R = Ring<MODE, BM>;
  const int lane = threadIdx.x & 63;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(slot));
  constexpr int DWH = (R::DW + 1) / 2;
  if (part < 0 || part <= 1) {
#pragma unroll
    for (int q = 0; q < R::DW; ++q)
      if (part < 0 || (q < DWH) == (part == 0))
        dma16<true>(src.w[q] + (int64_t)kb * src.wk, base + R::W_OFF + (wave * R::DW + q) * 1024);
  }
  if (part < 0 || part == 2) {
#pragma unroll
    for (int q = 0; q < R::DT; ++q)
      if (wave * R::DT + q < R::NTD)
        dma16<false>(src.t[q] + kb * R::AROW, base + R::T_OFF + (wave * R::DT + q) * 1024);
    // token scales: fp32 per K block, or the E8M0 dword of K blocks kb & ~3 .. +3
    const int ts_off = e8_tokens(MODE) ? (kb & ~3) : kb * 4;
#pragma unroll
    for (int h = 0; h < R::TSW; ++h) {
      const int c = wave * R::TSW + h;
      if (lane < 16) dma4(src.ts[h] + ts_off, base + R::TS_OFF + (c >> 2) * 256 + (c & 3) * 64);
    }
  }
  if (part >= 0 && part != 3) return;
  if constexpr (MODE != kGemmMx) {
    if (wave == R::NWAVE - 1 && lane < 2) dma4(src.wsc + kb * 4, base + R::WSC_OFF);
  }
  if constexpr (R::DWS > 0) {
    if (ws != nullptr) {
      const uint32_t wbase = __builtin_amdgcn_readfirstlane(lds_addr(ws));
#pragma unroll
      for (int q = 0; q < R::DWS; ++q) dma4(src.ws[q] + (kb >> 2) * src.wsk, wbase + (wave * R::DWS + q) * 256);
    }
  }
}

// Per-lane row of the token-scale load of chunk c (see ring_issue): entry
// i = 16*(c%4) + lane of 64-token group c/4 holds token tile i % 4, row i / 4.
__device__ __forceinline__ int ring_scale_row(int c, int lane) {
  const int i = (c & 3) * 16 + (lane & 15);
  return (c >> 2) * 64 + (i & 3) * 16 + (i >> 2);
}

// FP8 token tile in LDS: load h of the tile holds, at lane j's 16 bytes, row
// j % 16 and K bytes 64h + 16(j/16) .. +16 (whole 64-byte row segments per
// load).  The MFMA fragment of lane l (row l % 16, K bytes 32(l/16) .. +32)
// is then the two 16-byte words below.
__device__ __forceinline__ v8i lds_tok32(const uint8_t* tile, int lane) {
  const int q = lane >> 4;
  const uint8_t* p = tile + (q >> 1) * 1024 + (q & 1) * 512 + (lane & 15) * 16;
  const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 256);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ v8i lds_frag32(const uint8_t* p) {  // 32 FP8 bytes: halves 1 KB apart
  const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 1024);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
__device__ __forceinline__ v8i lds_frag16(const uint8_t* p) {  // 32 E2M1 values
  const uint4 lo = *(const uint4*)p;
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
}

template <int OPA>
__device__ __forceinline__ v4f mfma_fp4_scaled_t(const v8i& w, const v8i& t, v4f c, int sw, int st) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, t, c, 4, 4, OPA, sw, 0, st);
}

// One K block of the wave's 4 token tiles x 4 weight tiles from slot `slot`.
// acc[m][j][i] = C[token (wt*4+m)*16 + lane%16][weight row 16*tile_j + 4*(lane/16) + i].
// Only the first `mv` token tiles hold real rows (an expert's last block is
// padded); the others are skipped (mv is wave-uniform, 1..MT), except in the
// scheduled f16 path of 4 token tiles.
// iss(part) issues load group `part` of the next K block (ring_issue).  The
// scheduled f16 path (GEMM1, block FP8, 4 token tiles per wave) issues the
// weight loads before its tiles and the token and scale loads two tile steps
// in, so the K block's loads reach the vector memory unit in two bursts while
// its long compute runs; every other path issues all of them first.  (Same
// MI355X, alternating runs: FP8 GEMM1 at prefill 750 -> 733 us, on the skewed
// batch 362 -> 348 us; the same split in GEMM2 and the MX GEMM1, whose
// compute is short, cost them 1-4%.)
template <int MODE, int BM, bool G1, typename ISS>
__device__ __forceinline__ void ring_compute(const uint8_t* slot, const uint8_t* ws, const int (&tiles)[4], int wt,
                                             int kb, float sw0, float sw1, int mv,
                                             v4f (&acc)[Ring<MODE, BM>::MT][4], ISS&& iss) {
  using R = Ring<MODE, BM>;
  constexpr bool SPREAD = f16_path(MODE) && Ring<MODE, BM>::MT == 4;
  if constexpr (!SPREAD) iss(-1);  // (a no-op: the caller issued them)
  const int lane = threadIdx.x & 63;
  const uint8_t* wl = slot + R::W_OFF + lane * 16;
  const uint8_t* tt = slot + R::T_OFF + wt * R::MT * R::TILE;  // the wave's MT token tiles
  const uint8_t* tl = tt + lane * 16;
  const uint8_t* tsl = slot + R::TS_OFF + wt * R::MTH * 256 + (lane & 15) * 16;
  constexpr int MT = R::MT;
  if constexpr (MODE == kGemmMx) {
    const uint4 tsd = *(const uint4*)tsl;
    const int sh = 8 * (lane >> 4);
    const int st[4] = {(int)((tsd.x >> sh) & 0xFFu), (int)((tsd.y >> sh) & 0xFFu), (int)((tsd.z >> sh) & 0xFFu),
                       (int)((tsd.w >> sh) & 0xFFu)};
    // weight scale dword: the E8M0 bytes of 4 consecutive K blocks; this one's is byte kb % 4
    const int wsh = 8 * (kb & 3);
    v8i w[4];
    int sw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = lds_frag16(wl + tiles[j] * R::TILE);
      sw[j] = (int)((*(const uint32_t*)(ws + tiles[j] * 256 + lane * 4) >> wsh) & 0xFFu);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < mv) {
        const v8i t = lds_frag16(tl + m * R::TILE);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = mfma_fp4_scaled_t<0>(w[j], t, acc[m][j], sw[j], st[m]);
      }
    }
  } else {
    // token scales of tiles m (row lane % 16), one 16-byte word per 4
    // tiles: fp32, or E8M0 bytes (byte kb % 4 of each dword) and their exact
    // fp32 values
    constexpr int NSC = 4 * R::MTH;
    float tsc[NSC];
    int tsb[NSC];
#pragma unroll
    for (int hh = 0; hh < R::MTH; ++hh) {
      if constexpr (e8_tokens(MODE)) {
        const uint4 tw = *(const uint4*)(tsl + hh * 256);
        const int sh = 8 * (kb & 3);
        const uint32_t w4[4] = {tw.x, tw.y, tw.z, tw.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          tsb[4 * hh + m] = (int)((w4[m] >> sh) & 0xFFu);
          tsc[4 * hh + m] = e8m0_value((uint32_t)tsb[4 * hh + m]);
        }
      } else {
        const float4 ts = *(const float4*)(tsl + hh * 256);
        tsc[4 * hh + 0] = ts.x; tsc[4 * hh + 1] = ts.y; tsc[4 * hh + 2] = ts.z; tsc[4 * hh + 3] = ts.w;
      }
    }
    // GEMM1: tiles 0,1 are gate rows (scale sw0), 2,3 up rows (sw1); GEMM2: all sw0
    if constexpr (MODE == kGemmE8) {
      // power-of-two weight scale as its E8M0 byte (2^-127 is 0x00400000 -> 0)
      const int swb = (int)(__float_as_uint(sw0) >> 23);
      v8i w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = lds_frag32(wl + tiles[j] * R::TILE);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mv) {
          const v8i t = lds_tok32(tt + m * R::TILE, lane);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][j] = mfma_fp8_scaled(w[j], t, acc[m][j], swb, tsb[m]);
        }
      }
    } else if constexpr (MODE == kGemmFp8) {
      v8i w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = lds_frag32(wl + tiles[j] * R::TILE);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mv) {
          const v8i t = lds_tok32(tt + m * R::TILE, lane);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float s = tsc[m] * ((G1 && j >= 2) ? sw1 : sw0);
            const v4f c = mfma_fp8(w[j], t, v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(c[i], s, acc[m][j][i]);
          }
        }
      }
    } else if constexpr (MT != 4) {
      // plain order: every weight tile widened once, then the token tiles
      v8h wh[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) widen_fp8(lds_frag32(wl + tiles[j] * R::TILE), wh[j]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mv) {
          v8h th[4];
          widen_fp8(lds_tok32(tt + m * R::TILE, lane), th);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float s = tsc[m] * ((G1 && j >= 2) ? sw1 : sw0);
            v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < 4; ++k) c = mfma_f16(wh[j][k], th[k], c);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(c[i], s, acc[m][j][i]);
          }
        }
      }
    } else {
      // FP8 -> f16 widening is the bulk of the VALU work; the 16 (weight,
      // token) tiles are visited in an order that needs a new operand only
      // every other tile, and each operand is widened during the MFMAs of the
      // tiles before its first use, so the MFMA and VALU pipes overlap.
      // raw fragments are read from LDS two tiles before they are widened.
      // All 4 token tiles are computed even when some are padding: branching
      // inside this schedule costs more than the skipped tiles save, and a
      // second, partial schedule beside it does not fit the register budget.
      // A wave whose token tiles are all padding skips the K block.
      if (mv == 0) {
        iss(-1);
        return;
      }
      // weights before the tiles, tokens and scales two tile steps in (the
      // addresses then leave the registers before the schedule's peak)
      iss(0);
      iss(1);
      v8i wraw[4], traw[4];
      wraw[0] = lds_frag32(wl + tiles[0] * R::TILE);
      wraw[1] = lds_frag32(wl + tiles[1] * R::TILE);
      traw[0] = lds_tok32(tt, lane);
      traw[1] = lds_tok32(tt + R::TILE, lane);
      constexpr int kRead[16] = {2, -1, 6, -1, 3, -1, 7, -1, -1, -1, -1, -1, -1, -1, -1, -1};
      v8h wh[4][4], th[4][4];
      widen_fp8(wraw[0], wh[0]);
      widen_fp8(traw[0], th[0]);
      // tile order (weight tile, token tile) and the widening done meanwhile:
      // kWiden[g] = 1 + operand (0..3 weights, 4..7 tokens) whose quarter
      // kPart[g] (of 4 steps, kSteps[g] steps) is widened during tile g
      constexpr int kW[16] = {0, 1, 0, 1, 2, 2, 0, 1, 2, 3, 3, 3, 0, 1, 2, 3};
      constexpr int kT[16] = {0, 0, 1, 1, 0, 1, 2, 2, 2, 0, 1, 2, 3, 3, 3, 3};
      constexpr int kOp[16] = {1, 5, 2, 2, 6, 6, 3, 3, 3, 7, 7, 7, -1, -1, -1, -1};
      constexpr int kFirst[16] = {0, 0, 0, 2, 0, 2, 0, 2, 3, 0, 2, 3, 0, 0, 0, 0};
      constexpr int kLast[16] = {4, 4, 2, 4, 2, 4, 2, 3, 4, 2, 3, 4, 0, 0, 0, 0};
      v4f prev = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int j = kW[g], m = kT[g];
        if (g == 2) {
          iss(2);
          iss(3);
        }
        v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) c = mfma_f16(wh[j][k], th[m][k], c);
        if (kRead[g] >= 4)
          traw[kRead[g] - 4] = lds_tok32(tt + (kRead[g] - 4) * R::TILE, lane);
        else if (kRead[g] >= 0)
          wraw[kRead[g]] = lds_frag32(wl + tiles[kRead[g]] * R::TILE);
        if (kOp[g] >= 0) {
#pragma unroll
          for (int st = kFirst[g]; st < kLast[g]; ++st) {
            const int op = kOp[g];
            const v8i& raw = (op < 4) ? wraw[op] : traw[op - 4];
            const uint32_t d0 = (uint32_t)raw[2 * st], d1 = (uint32_t)raw[2 * st + 1];
            const uint4 v = make_uint4(e4m3x2_to_f16x2<false>(d0), e4m3x2_to_f16x2<true>(d0),
                                       e4m3x2_to_f16x2<false>(d1), e4m3x2_to_f16x2<true>(d1));
            if (op < 4)
              wh[op][st] = __builtin_bit_cast(v8h, v);
            else
              th[op - 4][st] = __builtin_bit_cast(v8h, v);
          }
        }
        if (g > 0) {
          const int pj = kW[g - 1], pm = kT[g - 1];
          const float s = tsc[pm] * ((G1 && pj >= 2) ? sw1 : sw0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[pm][pj][i] = fmaf(prev[i], s, acc[pm][pj][i]);
        }
        prev = c;
      }
      {
        const float s = tsc[3] * ((G1) ? sw1 : sw0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[3][3][i] = fmaf(prev[i], s, acc[3][3][i]);
      }
    }
  }
}

// ===========================================================================
// Streaming kernel (every block_m).  One persistent workgroup per CU walks a
// list of (M block, N tile) items, and its load ring runs on across item
// boundaries: the first K blocks of the next item are in
// flight while the current item finishes and writes its epilogue, so the
// ring never drains.  Item metadata (sorted pair ids, the block's expert,
// and for GEMM2 the routing weights of those pairs) also arrives by
// direct-to-LDS loads, one item ahead, and the FP8 weight scales ride with
// their K block, so neither a load the compiler would wait on nor a scalar
// load (whose cache misses would stall the whole workgroup) sits in the
// stream.
// ===========================================================================
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// GEMM1 epilogue: lane l holds, for token t = (wt*MT + m)*16 + l%16, the
// intermediate columns 32*wn + 16*jj + 4*(l/16) + i of the N tile (gate in
// acc[m][jj], up in acc[m][jj+2]).  Clamped SwiGLU, then the row's 1x128
// amax across the 4 column waves (FP8, through LDS) or the wave's own 1x32
// amax (MX), RNE codes, stored straight from registers (4 FP8 codes or 4 E2M1
// nibbles per lane and 16-column group).  Pad rows give zero codes.
template <int MODE, int BM>
__device__ __forceinline__ void epilogue_gemm1_s(const GemmArgs& p, const v4f (&acc)[Ring<MODE, BM>::MT][4],
                                                 float (*red)[BM], const int32_t* sid, int row0, int nt, int wt,
                                                 int wn) {
  constexpr int MT = Ring<MODE, BM>::MT;
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  const float L = p.limit;
  constexpr bool MXQ = MODE == kGemmMx, E8Q = MODE == kGemmE8F16;
  float av[MT][2][4];
  float tmax[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const bool real = sid[(wt * MT + m) * 16 + c16] < p.num_pairs;
    float mx = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = real ? swiglu_clamped(acc[m][jj][i], acc[m][jj + 2][i], L) : 0.0f;
        av[m][jj][i] = a;
        mx = fmaxf(mx, fabsf(a));
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    tmax[m] = mx;
  }
  if constexpr (!MXQ) {
    if (q == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wn][(wt * MT + m) * 16 + c16] = tmax[m];
    }
    lds_barrier();
    const int nsc = p.Ip / 128;
    const int64_t ld_e8 = (nsc + 3) / 4 * 4;  // UE8M0 scale rows: whole dwords
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = (wt * MT + m) * 16 + c16;
      const float amax = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
      uint8_t* row = p.aq + (int64_t)(row0 + t) * p.Ip + nt * 128 + 32 * wn + 4 * q;
      if constexpr (E8Q) {
        const uint32_t b = ue8m0_byte(amax);
        const float inv = e8m0_inverse(b);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          uint32_t packed = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) packed |= ((amax > 0.0f) ? fp8e8_quant(av[m][jj][i], inv) : 0u) << (8 * i);
          *(uint32_t*)(row + 16 * jj) = packed;
        }
        if (wn == 0 && q == 0) ((uint8_t*)p.as)[(int64_t)(row0 + t) * ld_e8 + nt] = (uint8_t)b;
      } else {
        const float s = amax / kE4M3Max;
        const float inv = 1.0f / s;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          uint32_t packed = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) packed |= ((amax > 0.0f) ? fp8_quant_inv(av[m][jj][i], inv) : 0u) << (8 * i);
          *(uint32_t*)(row + 16 * jj) = packed;
        }
        if (wn == 0 && q == 0) ((float*)p.as)[(int64_t)(row0 + t) * nsc + nt] = (amax > 0.0f) ? s : 0.0f;
      }
    }
  } else {
    const int nsc = p.Ip / 32;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = (wt * MT + m) * 16 + c16;
      const uint32_t b = e8m0_byte(tmax[m]);
      const float inv = e8m0_inverse(b);
      uint8_t* row = p.aq + (int64_t)(row0 + t) * (p.Ip / 2) + nt * 64 + 16 * wn + 2 * q;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) packed |= mx_quant(av[m][jj][i], inv) << (4 * i);
        *(uint16_t*)(row + 8 * jj) = (uint16_t)packed;
      }
      if (q == 0) ((uint8_t*)p.as)[(int64_t)(row0 + t) * nsc + nt * 4 + wn] = (uint8_t)b;
    }
  }
}

// GEMM1 epilogue of a K piece: the fp32 partial sums of the gate and up
// columns of real rows, part[piece, pair, column] (gate columns [0, Ip), up
// columns [Ip, 2Ip)), in the lane layout of epilogue_gemm1_s.  Piece 0 also
// writes the zero codes and scales of the block's pad rows (this N tile's
// columns), and piece 0 of N tile 0 the sorted row of each real pair,
// part_row[pair] (after the partial sums: P int32).
template <int MODE, int MT>
__device__ __forceinline__ void epilogue_gemm1_part(const GemmArgs& p, const v4f (&acc)[MT][4], const int32_t* sid,
                                                    int row0, int ks, int nt, int wt, int wn) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  const int64_t ld = 2 * (int64_t)p.Ip;
  int32_t* part_row = (int32_t*)(p.part + ((int64_t)p.num_pairs << p.ks_log2) * ld);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = (wt * MT + m) * 16 + c16;
    const int s = sid[t];
    if (s < p.num_pairs) {
      float* row = p.part + ((int64_t)ks * p.num_pairs + s) * ld + nt * 128 + 32 * wn + 4 * q;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const v4f g = acc[m][jj], u = acc[m][jj + 2];
        *(float4*)(row + 16 * jj) = make_float4(g[0], g[1], g[2], g[3]);
        *(float4*)(row + p.Ip + 16 * jj) = make_float4(u[0], u[1], u[2], u[3]);
      }
      if (ks == 0 && nt == 0 && wn == 0 && q == 0) part_row[s] = row0 + t;
    } else if (ks == 0) {
      const int64_t r = row0 + t;
      if constexpr (MODE == kGemmMx) {
        uint8_t* row = p.aq + r * (p.Ip / 2) + nt * 64 + 16 * wn + 2 * q;
        *(uint16_t*)row = 0;
        *(uint16_t*)(row + 8) = 0;
        if (q == 0) ((uint8_t*)p.as)[r * (p.Ip / 32) + nt * 4 + wn] = 0;
      } else {
        uint8_t* row = p.aq + r * p.Ip + nt * 128 + 32 * wn + 4 * q;
        *(uint32_t*)row = 0u;
        *(uint32_t*)(row + 16) = 0u;
        if (wn == 0 && q == 0) {
          if constexpr (MODE == kGemmE8F16)
            ((uint8_t*)p.as)[r * e8_scale_ld(p.Ip) + nt] = 0;
          else
            ((float*)p.as)[r * (p.Ip / 128) + nt] = 0.0f;
        }
      }
    }
  }
}

// GEMM1 epilogue of a K piece of a tail launch's leftover item r: the fp32
// partial sums of every row of the block (pad rows too; the finishing kernel
// zeroes them) for the N tile's 128 gate and 128 up columns,
// part[piece][r][row][256] (gate 0..127, up 128..255) with r < gridDim.x,
// in the lane layout of epilogue_gemm1_s.
template <int MT, int BM>
__device__ __forceinline__ void epilogue_gemm1_tail(const GemmArgs& p, const v4f (&acc)[MT][4], int piece, int r,
                                                    int wt, int wn) {
  // the lane's offset is formed here, not hoisted out of the ring loop, where
  // it would hold registers for the whole launch
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, q = lane >> 4, c16 = lane & 15;
  float* item = p.part + ((int64_t)piece * gridDim.x + r) * BM * 256;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = (wt * MT + m) * 16 + c16;
    float* row = item + t * 256 + 32 * wn + 4 * q;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const v4f g = acc[m][jj], u = acc[m][jj + 2];
      *(float4*)(row + 16 * jj) = make_float4(g[0], g[1], g[2], g[3]);
      *(float4*)(row + 128 + 16 * jj) = make_float4(u[0], u[1], u[2], u[3]);
    }
  }
}

// GEMM2 epilogue: the weighted rows v = routing weight * C of real pairs, in
// y's block floating point (y_plane_bytes): int16 q = rint(v * 2^-s),
// saturated to the int16 range, with one exponent s = max(floor(log2
// max|v|) - 14, -128) per 64 columns of a row.  Lane l holds, for token t =
// (wt*MT + m)*16 + l%16, columns 64*wn + 16*j + 4*(l/16) + i of the N tile,
// so a row's 64-column group is the wave's and its 4 lanes (l/16 = 0..3)
// share the group's largest |v| through two lane exchanges; that maximum is
// |w| * max|C| (rounding is monotonic).  Within a group the values are stored
// in lane order (y_group_col): lane l's 16 values, (j, i) in order, fill
// positions 16*(l/16) .. +16, two 16-byte stores per token tile.  |v| * 2^-s < 2^15, so only a
// value that rounds to 2^15 saturates (to 32767), and v' = q * 2^s is within
// 2^s <= 2^-14 max|v| of v.  Routing weights come from LDS.  y holds the
// columns of this launch's N tiles (from nt0); a K piece writes its own
// plane.
template <int MT>
__device__ __forceinline__ void epilogue_gemm2_s(const GemmArgs& p, const v4f (&acc)[MT][4], const int32_t* sid,
                                                 const float* wts, int ks, int nt, int wt, int wn) {
  const int lane = threadIdx.x & 63, q = lane >> 4, c16 = lane & 15;
  uint8_t* plane = p.y + ks * p.yplane;
  const int col0 = (nt - p.nt0) * 256 + 64 * wn;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = (wt * MT + m) * 16 + c16;
    const int s = sid[t];
    const bool real = s < p.num_pairs;
    const float w = real ? wts[t] : 0.0f;
    float mc = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mc = fmaxf(mc, fabsf(acc[m][j][i]));
    mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    const float mx = fabsf(w) * mc;
    if (real) {
      // floor(log2 mx) from the exponent field (subnormals included)
      const int e = mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) - 1 : 0;
      const int sx = max(e - 14, -128);
      int16_t* ygrp = (int16_t*)plane + (int64_t)s * p.ldy + col0 + 16 * q;
      uint32_t pk[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int qv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = (int)__builtin_rintf(ldexpf(w * acc[m][j][i], -sx));
        pk[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(qv[0], qv[1]));
        pk[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(qv[2], qv[3]));
      }
      *(uint4*)ygrp = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *(uint4*)(ygrp + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      if (q == 0) ((int8_t*)(plane + p.yexp))[(int64_t)s * (p.ldy / 64) + col0 / 64] = (int8_t)sx;
    }
  }
}

// Any K works.  Item metadata of item ii+1 is loaded when the loads of item ii
// start; when an item has fewer than S K blocks that is too late for the
// ring's own waits to cover it (the S-1 K blocks of the prologue are issued
// without waits), and the kernel then waits for it explicitly.
template <int MODE, int BM, bool G1, int S, int SPLIT>
__global__ __launch_bounds__(ring_waves(MODE, BM) * 64) void moe_gemm_stream_kernel(GemmArgs p) {
  using R = Ring<MODE, BM>;
  static_assert(S >= 3 && S <= 5, "ring depth");
  constexpr int MT = R::MT;
  constexpr int NI = BM >= 64 ? BM / 64 : 1;  // dword loads that cover one BM-long array
  const bool id_lane = BM >= 64 || (int)(threadIdx.x & 63) < BM;
  // Item-metadata buffers.  While item c is multiplied, the loads run S-1 K
  // blocks ahead and the metadata one item further: with one K block per item
  // that is item c + S + 1, so S + 2 buffers keep item c's ids and weights.
  constexpr int NB = S + 2;
  constexpr int NWS = S + 1;   // MX weight-scale group buffers
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t slot3[S > 3 ? R::SLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t slot4[S > 4 ? R::SLOT : 16];
  __shared__ __attribute__((aligned(256))) int32_t ids_lds[NB][BM];
  __shared__ int32_t exp_lds[NB];
  __shared__ __attribute__((aligned(256))) float wts_lds[G1 ? 1 : NB][BM];
  __shared__ float red[4][BM];
  __shared__ __attribute__((aligned(256))) uint8_t ws_buf[MODE == kGemmMx ? NWS : 1][MODE == kGemmMx ? R::WS_BYTES : 16];
  auto slot = [&](auto ic) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(ic)::value;
    if constexpr (i == 0) return slot0;
    else if constexpr (i == 1) return slot1;
    else if constexpr (i == 2) return slot2;
    else if constexpr (i == 3) return slot3;
    else return slot4;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave >> 2, wn = wave & 3;
  // A workgroup's items: n_whole whole (M block, N tile) items, then n_tail
  // K pieces.  Pieces of one list are spread as the items of the plain
  // kernel: the list is cut into one contiguous chunk per XCD, and workgroup
  // j of the XCD takes pieces j, j + nw, j + 2 nw, ... of it (nw workgroups
  // per XCD; workgroups go to the XCDs round-robin).
  //   plain and K-split launches: no whole items; the list is every item
  //     cut into 2^KSL pieces (KSL = 0: the items themselves).
  //   tail launches (p.tail): the items that fill whole rounds of the grid
  //     (F per workgroup, XCD-chunked the same way), then the remaining
  //     items cut into 2^KSL pieces, whose fp32 partial sums a second
  //     kernel finishes (launch_gemm1_tail_finish) -- when the remaining
  //     items fill at most half a round (tail_split_on); else the launch
  //     runs every item whole, as the plain kernel.
  // A plain launch may group NTG N tiles of one M block into an item (when
  // K has fewer than S K blocks, so that every item streams at least S):
  // the item's K blocks run N tile by N tile, each with its own epilogue,
  // and the block's metadata serves them all.
  const int NTG = SPLIT == kNoSplit ? p.ntg : 1;
  const int n_grp = p.n_tiles / NTG;  // items per M block
  const int npp = __builtin_amdgcn_readfirstlane(*p.npp);
  const int nw = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, jw = blockIdx.x / kXcds;
  const int all_items = (npp / BM) * n_grp;
  const bool tail = SPLIT == kTailSplit && tail_split_on(all_items, (int)gridDim.x);
  const int KSL = SPLIT == kKSplit || tail ? p.ks_log2 : 0;  // K pieces per split item: 2^KSL
  int n_whole = 0, wbase = 0, tail_base = 0, list = all_items << KSL;
  if (tail) {
    const int F = all_items / (int)gridDim.x;
    n_whole = F;
    wbase = xcd * F * nw + jw;
    tail_base = F * (int)gridDim.x;
    list = (all_items - tail_base) << KSL;
  }
  const int per = (list + kXcds - 1) / kXcds;
  const int lo = xcd * per;
  const int hi = min(lo + per, list);
  const int first = lo + jw;
  const int n_tail = first < hi ? (hi - first + nw - 1) / nw : 0;
  const int n_my = n_whole + n_tail;
  if (n_my == 0) return;
  const int KB = p.K / 128;   // K blocks of a weight row
  const int KBP = KB >> KSL;  // K blocks of a piece
  const int NG = tiled_n_groups(p.N);  // N tiles of the weight matrix (TILED_V2)
  const int total = n_whole * KB + n_tail * KBP * NTG;
  // item -> (M block, N tile, K piece), K pieces innermost.  (Every lambda of
  // this kernel is always_inline: one left as a call makes the kernel keep
  // its arguments in scratch memory, which cost 4x at one token.)
  auto item_g = [&](int ii) __attribute__((always_inline)) {
    return ii < n_whole ? wbase + ii * nw : tail_base + ((first + (ii - n_whole) * nw) >> KSL);
  };
  auto item_m = [&](int ii) __attribute__((always_inline)) { return item_g(ii) / n_grp; };
  auto item_nt = [&](int ii) __attribute__((always_inline)) { return p.nt0 + item_g(ii) % n_grp * NTG; };  // first N tile
  auto item_ks = [&](int ii) __attribute__((always_inline)) { return ii < n_whole ? 0 : (first + (ii - n_whole) * nw) & ((1 << KSL) - 1); };
  auto item_kbs = [&](int ii) __attribute__((always_inline)) { return ii < n_whole ? KB : KBP; };  // per N tile
  auto item_kbi = [&](int ii) __attribute__((always_inline)) { return item_kbs(ii) * NTG; };
  // Items of fewer than S K blocks finish inside the prologue (which issues
  // S-1 K blocks without waiting) or within S-1 steps of the next item's
  // metadata loads: their metadata is waited for explicitly.
  auto short_item = [&](int ii) __attribute__((always_inline)) { return item_kbi(ii) < S; };

  // sorted pair ids of item ii -> ids_lds[ii % NB] (waves 0 .. NI-1), its
  // block's expert -> exp_lds[ii % NB] (lane 0 of the last wave)
  auto issue_ids = [&](int ii) __attribute__((always_inline)) {
    if (wave < NI && id_lane)
      dma4(p.sorted_ids + item_m(ii) * BM + wave * 64 + lane, lds_addr(&ids_lds[ii % NB][wave * 64]));
    if (wave == R::NWAVE - 1 && lane == 0) dma4(p.block_expert + item_m(ii), lds_addr(&exp_lds[ii % NB]));
  };
  // GEMM2: routing weight of each row of item ii (its ids must be visible)
  auto issue_wts = [&](int ii) __attribute__((always_inline)) {
    if constexpr (!G1) {
      if (wave >= NI && wave < 2 * NI && id_lane) {
        const int r0 = (wave - NI) * 64;
        const int s = ids_lds[ii % NB][r0 + lane];
        dma4(p.topk_w + (s < p.num_pairs ? s : 0), lds_addr(&wts_lds[ii % NB][r0]));
      }
    }
  };

  // ---- issue side: per-lane source addresses of the item being loaded
  RingSrc<MODE, BM> rs;
  rs.wk = p.tile_run * R::TILE;
  rs.wsk = p.tile_run * 256;
  int wts_step = -1, wts_item = 0;
  int i_e = 0, i_nt = 0;  // expert and N tile being loaded
  // weight-side sources of N tile nt of expert e from K block kb0
  auto setup_weights = [&](int e, int nt, int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < R::DW; ++q) {
      const int g = wave * R::DW + q, tile = g / R::HALVES, h = g % R::HALVES;
      rs.w[q] = p.B + tiled_index(p.tile_run, e, NG, nt, tile, KB, kb0) * R::TILE + h * 1024 + lane * 16;
    }
    if constexpr (MODE != kGemmMx) {
      // GEMM1: the gate and the up 128-row block of the N tile; GEMM2: the
      // N tile's two 128-row blocks (the second clamped to the last block)
      const int NB128 = p.N / 128;
      const int b0 = G1 ? nt : nt * 2, b1 = G1 ? p.Ip / 128 + nt : min(nt * 2 + 1, NB128 - 1);
      rs.wsc = (const uint8_t*)((const float*)p.Bs + ((int64_t)e * NB128 + ((lane & 1) ? b1 : b0)) * KB + kb0);
    }
    if constexpr (R::DWS > 0) {
      const int KBq = (KB + 3) / 4;
#pragma unroll
      for (int q = 0; q < R::DWS; ++q)
        rs.ws[q] = (const uint8_t*)p.Bs +
                   (tiled_index(p.tile_run, e, NG, nt, wave * R::DWS + q, KBq, kb0 / 4) * 64 + lane) * 4;
    }
  };
  auto setup_issue = [&](int ii, int s) __attribute__((always_inline)) {
    const int m = item_m(ii), nt = item_nt(ii);
    const int kb0 = item_ks(ii) * KBP;  // first K block of the item (0 for whole items)
    const int e = __builtin_amdgcn_readfirstlane(exp_lds[ii % NB]);
    i_e = e;
    i_nt = nt;
    setup_weights(e, nt, kb0);
    const int32_t* ids = ids_lds[ii % NB];
    // rows past BM (the unused scale entries of a small block) read row 0 / the block's first row
    auto row_of = [&](int r) -> int64_t {
      if constexpr (G1) {
        const int sid = r < BM ? ids[r] : p.num_pairs;
        return sid < p.num_pairs ? sid / p.top_k : 0;
      } else {
        return (int64_t)m * BM + (r < BM ? r : 0);
      }
    };
#pragma unroll
    for (int q = 0; q < R::DT; ++q) {
      const int g = wave * R::DT + q, mt = g / R::HALVES, h = g % R::HALVES;
      rs.t[q] = p.A + row_of(mt * 16 + (lane & 15)) * p.lda + kb0 * R::AROW + h * 64 + (lane >> 4) * 16;
    }
#pragma unroll
    for (int h = 0; h < R::TSW; ++h) {
      // scale bytes before K block kb0: fp32 and MX 4 per K block, UE8M0 1
      const int64_t row = row_of(ring_scale_row(wave * R::TSW + h, lane));
      rs.ts[h] = (MODE == kGemmMx) ? (const uint8_t*)p.As + row * p.ldas + kb0 * 4
                 : e8_tokens(MODE) ? (const uint8_t*)p.As + row * p.ldas + kb0
                                   : (const uint8_t*)p.As + row * p.ldas * 4 + kb0 * 4;
    }
    // metadata of the next item: ids now; GEMM2 weights S-1 steps later,
    // once the ring's waits have covered the ids (or right away after an
    // explicit wait when items are short)
    if (ii + 1 < n_my) {
      issue_ids(ii + 1);
      if (short_item(ii)) {
        vm_wait_barrier<0>();
        if constexpr (!G1) {
          issue_wts(ii + 1);
          vm_wait_barrier<0>();
        }
      } else {
        wts_step = s + S - 1;
        wts_item = ii + 1;
      }
    }
  };

  // ---- compute side: state of the item being multiplied
  int tiles[4];
  if constexpr (G1) {
    tiles[0] = 2 * wn; tiles[1] = 2 * wn + 1; tiles[2] = 8 + 2 * wn; tiles[3] = 9 + 2 * wn;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) tiles[j] = 4 * wn + j;
  }
  int c_nt = 0, c_row0 = 0, c_mv = MT, c_ks = 0, c_kbi = KB, c_g = 0, c_sub = 0;
  bool active = true;
  auto setup_compute = [&](int ii) __attribute__((always_inline)) {
    c_nt = item_nt(ii);
    c_ks = item_ks(ii);
    c_row0 = item_m(ii) * BM;
    c_kbi = item_kbs(ii);  // K blocks per N tile
    c_g = item_g(ii);
    c_sub = 0;
    if constexpr (!G1) active = c_nt * 256 + 64 * wn < p.N;
    // real rows are a prefix of the block: count the wave's token tiles
    // that start with one
    const int32_t* ids = ids_lds[ii % NB];
    int mv = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) mv += ids[(wt * MT + m) * 16] < p.num_pairs ? 1 : 0;
    c_mv = __builtin_amdgcn_readfirstlane(mv);
  };

  v4f acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // issue cursor (item, K block) and MX weight-scale groups: the group of up
  // to 4 K blocks that starts at K block kb (kb % 4 == 0) goes to
  // ws_buf[group count % NWS] with the loads of that K block
  int i_ii = 0, i_kb = 0, i_grp = 0, i_kbi = item_kbs(0), i_sub = 0;
  // the issue cursor's K block: issue_prep picks its MX weight-scale group
  // buffer, issue_part issues load group `part` (-1: all) into slot_c,
  // issue_step moves the cursor on
  const uint8_t* i_ws = nullptr;
  auto issue_prep = [&]() __attribute__((always_inline)) {
    i_ws = nullptr;
    if constexpr (MODE == kGemmMx) {
      if (i_ii < n_my && (i_kb & 3) == 0) i_ws = ws_buf[(i_grp++) % NWS];
    }
  };
  auto issue_part = [&](auto slot_c, int part) __attribute__((always_inline)) {
    if (i_ii < n_my) ring_issue<MODE, BM>(rs, slot(slot_c), wave, i_kb, i_ws, part);
  };
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    if (i_ii < n_my) {
      if (++i_kb == i_kbi) {
        i_kb = 0;
        if (++i_sub < NTG) {
          // the item's next N tile (grouped items are whole: from K block 0)
          setup_weights(i_e, ++i_nt, 0);
        } else if (++i_ii < n_my) {
          i_sub = 0;
          i_kbi = item_kbs(i_ii);
          setup_issue(i_ii, s);
        }
      }
    }
    // past the end of the stream nothing is issued: the waits of the last
    // S-2 steps count only the slots that exist
  };
  auto issue_next = [&](auto slot_c, int s) __attribute__((always_inline)) {
    issue_prep();
    issue_part(slot_c, -1);
    issue_step(s);
  };

  // prologue: metadata of item 0, then K blocks 0 .. S-2 of the stream
  issue_ids(0);
  vm_wait_barrier<0>();
  if constexpr (!G1) {
    issue_wts(0);
    vm_wait_barrier<0>();
  }
  setup_issue(0, -(S - 1));  // logically before the loads of stage 0
  setup_compute(0);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (issue_next(std::integral_constant<int, I>{}, I - (S - 1)), ...);
  }(std::make_integer_sequence<int, S - 1>{});

  int c_ii = 0, c_kb = 0, c_grp = 0;  // compute cursor
  const uint8_t* c_ws = ws_buf[0];
  auto step = [&](auto dc, int s) __attribute__((always_inline)) {
    constexpr int d = decltype(dc)::value;
    vm_wait_barrier_upto<S - 2, R::D>(total - 1 - s);  // slots issued after this one: up to S-2
    float sw0 = 0.0f, sw1 = 0.0f;
    if constexpr (MODE != kGemmMx) {
      // GEMM1: gate and up scale; GEMM2: the scale of the wave's 128-row block
      const float2 sc = *(const float2*)(slot(std::integral_constant<int, d>{}) + R::WSC_OFF);
      sw0 = (G1 || (wn >> 1) == 0) ? sc.x : sc.y;
      sw1 = sc.y;
    }
    if (s == wts_step) issue_wts(wts_item);
    // the loads of K block s + S - 1: in two groups during the compute of the
    // scheduled f16 path (ring_compute), else all of them first
    constexpr bool split = f16_path(MODE) && MT == 4;
    auto iss = [&](int part) __attribute__((always_inline)) {
      if constexpr (split) issue_part(std::integral_constant<int, (d + S - 1) % S>{}, part);
    };
    if constexpr (split)
      issue_prep();
    else
      issue_next(std::integral_constant<int, (d + S - 1) % S>{}, s);
    if constexpr (MODE == kGemmMx) {
      if ((c_kb & 3) == 0) c_ws = ws_buf[(c_grp++) % NWS];
    }
    if (active && c_mv > 0)
      ring_compute<MODE, BM, G1>(slot(std::integral_constant<int, d>{}), c_ws, tiles, wt, c_kb, sw0, sw1, c_mv, acc,
                                 iss);
    else
      iss(-1);
    if constexpr (split) issue_step(s);
    if (++c_kb == c_kbi) {
      const int32_t* ids = ids_lds[c_ii % NB];
      if constexpr (G1) {
        if constexpr (SPLIT == kKSplit) {
          epilogue_gemm1_part<MODE, MT>(p, acc, ids, c_row0, c_ks, c_nt, wt, wn);
        } else if constexpr (SPLIT == kTailSplit) {
          if (!tail || c_ii < n_whole)
            epilogue_gemm1_s<MODE, BM>(p, acc, red, ids, c_row0, c_nt, wt, wn);
          else
            epilogue_gemm1_tail<MT, BM>(p, acc, c_ks, c_g - tail_base, wt, wn);
        } else {
          epilogue_gemm1_s<MODE, BM>(p, acc, red, ids, c_row0, c_nt, wt, wn);
        }
      } else {
        if (active) epilogue_gemm2_s<MT>(p, acc, ids, wts_lds[c_ii % NB], c_ks, c_nt, wt, wn);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      c_kb = 0;
      if (++c_sub < NTG) {
        ++c_nt;
        if constexpr (!G1) active = c_nt * 256 + 64 * wn < p.N;
      } else if (++c_ii < n_my) {
        setup_compute(c_ii);
      }
    }
  };
  for (int s0 = 0; s0 < total; s0 += S) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((s0 + I < total ? step(std::integral_constant<int, I>{}, s0 + I) : void()), ...);
    }(std::make_integer_sequence<int, S>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS after the workgroup ends
}

#ifndef MOE_RING_S_FP8
#define MOE_RING_S_FP8 3
#endif
#ifndef MOE_RING_S_MX
#define MOE_RING_S_MX 5
#endif
#ifndef MOE_RING_S_SMALL
#define MOE_RING_S_SMALL 4
#endif

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

int gemm_grid_max() { return (device_cus() + kXcds - 1) / kXcds * kXcds; }

// Kernels with a K split (SPLIT) are separate instances, so that the plain
// ones carry none of its per-item state.
template <int MODE, bool G1, int SPLIT>
static hipError_t launch_gemm_split(int block_m, int nb, const GemmArgs& a, hipStream_t s) {
  constexpr int SR = (MODE == kGemmMx) ? MOE_RING_S_MX : MOE_RING_S_FP8;    // block_m 64 / 128
  constexpr int SD = (MODE == kGemmMx) ? MOE_RING_S_MX : MOE_RING_S_SMALL;  // block_m 16 / 32
  // One workgroup per CU (the ring's LDS use allows no more), fewer when
  // there are fewer items; a multiple of kXcds so that every XCD gets the
  // same number of workgroups.
  const int64_t items = ((int64_t)nb * (a.n_tiles / a.ntg)) << a.ks_log2;
  const int64_t wgs = gemm_grid_max();
  // a tail launch splits the items past the grid's whole rounds: all of it
  const dim3 grid((unsigned)(a.tail || items >= wgs ? wgs : (items + kXcds - 1) / kXcds * kXcds));
  switch (block_m) {
    case 16:
      hipLaunchKernelGGL((moe_gemm_stream_kernel<MODE, 16, G1, SD, SPLIT>), grid, dim3(Ring<MODE, 16>::NTH), 0, s,
                         a);
      break;
    case 32:
      hipLaunchKernelGGL((moe_gemm_stream_kernel<MODE, 32, G1, SD, SPLIT>), grid, dim3(Ring<MODE, 32>::NTH), 0, s,
                         a);
      break;
    case 64:
      hipLaunchKernelGGL((moe_gemm_stream_kernel<MODE, 64, G1, SR, SPLIT>), grid, dim3(Ring<MODE, 64>::NTH), 0, s,
                         a);
      break;
    default:
      hipLaunchKernelGGL((moe_gemm_stream_kernel<MODE, 128, G1, SR, SPLIT>), grid, dim3(Ring<MODE, 128>::NTH), 0, s,
                         a);
      break;
  }
  return hipGetLastError();
}

template <int MODE, bool G1>
static hipError_t launch_gemm_mode(int block_m, int nb, const GemmArgs& a, hipStream_t s) {
  if constexpr (G1) {
    if (a.tail) return launch_gemm_split<MODE, G1, kTailSplit>(block_m, nb, a, s);
  }
  return a.ks_log2 > 0 ? launch_gemm_split<MODE, G1, kKSplit>(block_m, nb, a, s)
                       : launch_gemm_split<MODE, G1, kNoSplit>(block_m, nb, a, s);
}

// Ring depth of a launch.
static int ring_depth(int gmode, int block_m) {
  if (gmode == kGemmMx) return MOE_RING_S_MX;
  return block_m >= 64 ? MOE_RING_S_FP8 : MOE_RING_S_SMALL;
}

// N tiles per item of a plain launch: 1, or when K has fewer K blocks than
// the ring's depth the smallest power of two (dividing the launch's N tiles)
// whose items stream at least that many, so that no item waits for its
// metadata (items of fewer K blocks than the depth must).
static int n_tile_group(int gmode, int block_m, const GemmArgs& a) {
  const int KB = a.K / 128, S = ring_depth(gmode, block_m);
  int g = 1;
  while (g * KB < S && a.n_tiles % (2 * g) == 0) g *= 2;
  return g;
}

// GEMM1's output is re-quantised, so its sum must be fp32-exact: block FP8
// (either scale format) runs on the f16 MFMA (FP8 storage, exact widening in
// registers).
hipError_t launch_gemm1(int mode, int block_m, int nb, const GemmArgs& a0, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  GemmArgs a = a0;
  a.ntg = 1;
  switch (mode) {
    case kQuantFp8: return launch_gemm_mode<kGemmFp8F16, true>(block_m, nb, a, s);
    case kQuantFp8E8: return launch_gemm_mode<kGemmE8F16, true>(block_m, nb, a, s);
    default: return launch_gemm_mode<kGemmMx, true>(block_m, nb, a, s);
  }
}

hipError_t launch_gemm2(int mode, int block_m, int nb, const GemmArgs& a0, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  GemmArgs a = a0;
  const int gm = mode == kQuantFp8 ? kGemmFp8 : mode == kQuantFp8E8 ? kGemmE8 : kGemmMx;
  a.ntg = a.ks_log2 > 0 ? 1 : n_tile_group(gm, block_m, a);
  switch (mode) {
    case kQuantFp8: return launch_gemm_mode<kGemmFp8, false>(block_m, nb, a, s);
    case kQuantFp8E8: return launch_gemm_mode<kGemmE8, false>(block_m, nb, a, s);
    default: return launch_gemm_mode<kGemmMx, false>(block_m, nb, a, s);
  }
}

// ---------------------------------------------------------------------------
// K split for small batches.

int ksplit_cap(int mode, int KB) {
  int ks = 1;
  while (ks < kSplitMax && ksplit_ok(mode, KB, 2 * ks)) ks *= 2;
  return ks;
}

bool ksplit_ok(int mode, int KB, int ks) {
  if (ks == 1) return true;
  if (ks != 2 && ks != 4 && ks != 8) return false;
  if (KB % ks != 0 || KB / ks < 4) return false;
  // MX and UE8M0 scale bytes come in dwords of 4 K blocks
  return mode == kQuantFp8 || (KB / ks) % 4 == 0;
}

// Expected (M block, N tile) items of a GEMM under uniform routing: active
// experts E * (1 - (1 - k/E)^T); blocks: one per active expert while an
// expert's share of pairs fits one block.
static double expected_items(int T, int E, int k, int block_m, int n_tiles) {
  const int64_t P = (int64_t)T * k;
  const double active = (double)E * (1.0 - pow(1.0 - (double)k / E, (double)T));
  const double share = (double)P / (active > 1.0 ? active : 1.0);
  const double blocks = share <= block_m ? active : (double)P / block_m + 0.5 * active;
  return blocks * n_tiles;
}

bool tail_split_plan_ok(int T, int E, int k, int block_m, int n_tiles) {
  // the kernel splits the leftover items only when they fill at most half a
  // round (tail_split_on); skip planning a tail launch (and its second,
  // finishing kernel) where the estimate leaves clearly more, with margin
  // for the estimate's error of a few experts
  const double W = (double)gemm_grid_max();
  const double items = expected_items(T, E, k, block_m, n_tiles);
  const double left = items - W * floor(items / W);
  // at block_m 64 / 128 only for a few rounds of items (one GPU's share of
  // a tensor-parallel layer, small batches), where the last round is a large
  // part of the launch: the estimate ignores experts with a second block,
  // which many-round prefill batches have
  if (block_m >= 64 && items >= 4 * W) return false;
  return T > 0 && left <= 0.7 * W;
}

int pick_ksplit(int mode, int T, int E, int k, int block_m, int KB, int n_tiles) {
  const int64_t P = (int64_t)T * k;
  if (P <= 0 || P > kSplitMaxPairs) return 1;
  const double items = expected_items(T, E, k, block_m, n_tiles);
  // a split only pays while workgroups would otherwise sit idle: once every
  // workgroup has an item, shorter pieces stream the same bytes per CU and
  // add the partial sums' round trip
  const double wgs = (double)((device_cus() + kXcds - 1) / kXcds * kXcds);
  int ks = 1;
  while (items * (2 * ks) <= wgs + 0.5 && ksplit_ok(mode, KB, 2 * ks)) ks *= 2;  // + 0.5: rounding of the estimate
  return ks;
}

// One workgroup per pair f (its sorted row r from part_row, which GEMM1's
// piece 0 wrote; the partial sums are read without waiting for it); a thread
// owns 4 consecutive intermediate columns, so a 1x128 group is 32 threads and
// a 1x32 group 8.  The code and scale decisions are those of
// epilogue_gemm1_s, on the same fp32 values.  Pad rows were zeroed by GEMM1.
template <int QMODE, int KS>
__global__ __launch_bounds__(256) void swiglu_requant_kernel(const float* __restrict__ part, int P, int Ip, float L,
                                                             uint8_t* __restrict__ aq, void* __restrict__ as) {
  const int f = blockIdx.x;
  const int64_t plane = (int64_t)P * 2 * Ip;
  const int r = ((const int32_t*)(part + plane * KS))[f];
  for (int c = threadIdx.x * 4; c < Ip; c += 1024) {
    float a[4];
    {
      // all pieces' loads first, then the sums in piece order
      const float* g = part + (int64_t)f * 2 * Ip + c;
      float4 gv[KS], uv[KS];
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        gv[i] = *(const float4*)(g + i * plane);
        uv[i] = *(const float4*)(g + i * plane + Ip);
      }
      float4 gs = gv[0], us = uv[0];
#pragma unroll
      for (int i = 1; i < KS; ++i) {
        gs.x += gv[i].x; gs.y += gv[i].y; gs.z += gv[i].z; gs.w += gv[i].w;
        us.x += uv[i].x; us.y += uv[i].y; us.z += uv[i].z; us.w += uv[i].w;
      }
      a[0] = swiglu_clamped(gs.x, us.x, L);
      a[1] = swiglu_clamped(gs.y, us.y, L);
      a[2] = swiglu_clamped(gs.z, us.z, L);
      a[3] = swiglu_clamped(gs.w, us.w, L);
    }
    float mx = fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3])));
    constexpr int GT = QMODE == kQuantMx ? 8 : 32;  // threads of one group
#pragma unroll
    for (int o = 1; o < GT; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const bool lead = (threadIdx.x & (GT - 1)) == 0;
    if constexpr (QMODE == kQuantMx) {
      const uint32_t b = e8m0_byte(mx);
      const float inv = e8m0_inverse(b);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= mx_quant(a[i], inv) << (4 * i);
      *(uint16_t*)(aq + (int64_t)r * (Ip / 2) + c / 2) = (uint16_t)packed;
      if (lead) ((uint8_t*)as)[(int64_t)r * (Ip / 32) + c / 32] = (uint8_t)b;
    } else if constexpr (QMODE == kQuantFp8E8) {
      const uint32_t b = ue8m0_byte(mx);
      const float inv = e8m0_inverse(b);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= ((mx > 0.0f) ? fp8e8_quant(a[i], inv) : 0u) << (8 * i);
      *(uint32_t*)(aq + (int64_t)r * Ip + c) = packed;
      if (lead) ((uint8_t*)as)[(int64_t)r * e8_scale_ld(Ip) + c / 128] = (uint8_t)b;
    } else {
      const float sc = mx / kE4M3Max;
      const float inv = 1.0f / sc;
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= ((mx > 0.0f) ? fp8_quant_inv(a[i], inv) : 0u) << (8 * i);
      *(uint32_t*)(aq + (int64_t)r * Ip + c) = packed;
      if (lead) ((float*)as)[(int64_t)r * (Ip / 128) + c / 128] = (mx > 0.0f) ? sc : 0.0f;
    }
  }
}

template <int QMODE>
static void launch_requant_mode(const float* part, int ks, int P, int Ip, float limit, uint8_t* aq, void* as,
                                hipStream_t s) {
  const dim3 grid((unsigned)P), block(256);
  switch (ks) {
    case 2: hipLaunchKernelGGL((swiglu_requant_kernel<QMODE, 2>), grid, block, 0, s, part, P, Ip, limit, aq, as); break;
    case 4: hipLaunchKernelGGL((swiglu_requant_kernel<QMODE, 4>), grid, block, 0, s, part, P, Ip, limit, aq, as); break;
    default: hipLaunchKernelGGL((swiglu_requant_kernel<QMODE, 8>), grid, block, 0, s, part, P, Ip, limit, aq, as); break;
  }
}

hipError_t launch_swiglu_requant(int mode, const float* part, int ks, int P, int Ip, float limit, uint8_t* aq,
                                 void* as, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  if (mode == kQuantFp8)
    launch_requant_mode<kQuantFp8>(part, ks, P, Ip, limit, aq, as, s);
  else if (mode == kQuantFp8E8)
    launch_requant_mode<kQuantFp8E8>(part, ks, P, Ip, limit, aq, as, s);
  else
    launch_requant_mode<kQuantMx>(part, ks, P, Ip, limit, aq, as, s);
  return hipGetLastError();
}

// Second kernel of a tail launch: workgroup r < (leftover items) finishes
// leftover item r (M block m, N tile nt of the items after the grid's whole
// rounds, the numbering of the GEMM kernel): per row, the KS pieces' fp32
// partial sums added in piece order, then the clamped SwiGLU and the
// re-quantisation of epilogue_gemm1_s for the N tile's 128 intermediate
// columns; pad rows get zero codes and scales.  Workgroup (r, c) takes rows
// 16c .. 16c+15 of the block: 32 threads per row (4 columns each), 8 rows at
// a time (one workgroup per 16 rows, so that a large block's partial sums
// are read by many compute units).
template <int QMODE, int KS, int BM>
__global__ __launch_bounds__(256) void gemm1_tail_finish_kernel(const float* __restrict__ part,
                                                                const int32_t* __restrict__ sorted_ids,
                                                                const int32_t* __restrict__ npp_p, int n_tiles, int W,
                                                                int P, int Ip, float L, uint8_t* __restrict__ aq,
                                                                void* __restrict__ as) {
  const int items = (*npp_p / BM) * n_tiles;
  const int F = items / W;
  const int r = blockIdx.x;
  if (!tail_split_on(items, W) || r >= items - F * W) return;
  const int g = F * W + r, m = g / n_tiles, nt = g % n_tiles;
  const int c = (threadIdx.x & 31) * 4;  // intermediate column within the N tile
  const int t_end = min(BM, 16 * ((int)blockIdx.y + 1));
  for (int t = 16 * blockIdx.y + (threadIdx.x >> 5); t < t_end; t += 8) {
    const int64_t row = (int64_t)m * BM + t;
    const bool real = sorted_ids[row] < P;
    float a[4];
    {
      // all pieces' loads first, then the sums in piece order
      float4 gv[KS], uv[KS];
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const float* src = part + (((int64_t)i * W + r) * BM + t) * 256 + c;
        gv[i] = *(const float4*)src;
        uv[i] = *(const float4*)(src + 128);
      }
      float4 gs = gv[0], us = uv[0];
#pragma unroll
      for (int i = 1; i < KS; ++i) {
        gs.x += gv[i].x; gs.y += gv[i].y; gs.z += gv[i].z; gs.w += gv[i].w;
        us.x += uv[i].x; us.y += uv[i].y; us.z += uv[i].z; us.w += uv[i].w;
      }
      a[0] = real ? swiglu_clamped(gs.x, us.x, L) : 0.0f;
      a[1] = real ? swiglu_clamped(gs.y, us.y, L) : 0.0f;
      a[2] = real ? swiglu_clamped(gs.z, us.z, L) : 0.0f;
      a[3] = real ? swiglu_clamped(gs.w, us.w, L) : 0.0f;
    }
    float mx = fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3])));
    constexpr int GT = QMODE == kQuantMx ? 8 : 32;  // threads of one group
#pragma unroll
    for (int o = 1; o < GT; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const bool lead = (threadIdx.x & (GT - 1)) == 0;
    const int col = nt * 128 + c;
    if constexpr (QMODE == kQuantMx) {
      const uint32_t b = e8m0_byte(mx);
      const float inv = e8m0_inverse(b);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= mx_quant(a[i], inv) << (4 * i);
      *(uint16_t*)(aq + row * (Ip / 2) + col / 2) = (uint16_t)packed;
      if (lead) ((uint8_t*)as)[row * (Ip / 32) + col / 32] = (uint8_t)b;
    } else if constexpr (QMODE == kQuantFp8E8) {
      const uint32_t b = ue8m0_byte(mx);
      const float inv = e8m0_inverse(b);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= ((mx > 0.0f) ? fp8e8_quant(a[i], inv) : 0u) << (8 * i);
      *(uint32_t*)(aq + row * Ip + col) = packed;
      if (lead) ((uint8_t*)as)[row * e8_scale_ld(Ip) + nt] = (uint8_t)b;
    } else {
      const float sc = mx / kE4M3Max;
      const float inv = 1.0f / sc;
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= ((mx > 0.0f) ? fp8_quant_inv(a[i], inv) : 0u) << (8 * i);
      *(uint32_t*)(aq + row * Ip + col) = packed;
      if (lead) ((float*)as)[row * (Ip / 128) + nt] = (mx > 0.0f) ? sc : 0.0f;
    }
  }
}

template <int QMODE, int BM>
static void launch_tail_finish_bm(int ks, const float* part, const int32_t* sorted, const int32_t* npp, int n_tiles,
                                  int W, int P, int Ip, float limit, uint8_t* aq, void* as, hipStream_t s) {
  const dim3 grid((unsigned)W, (unsigned)((BM + 15) / 16)), block(256);
  switch (ks) {
    case 2:
      hipLaunchKernelGGL((gemm1_tail_finish_kernel<QMODE, 2, BM>), grid, block, 0, s, part, sorted, npp, n_tiles, W,
                         P, Ip, limit, aq, as);
      break;
    case 4:
      hipLaunchKernelGGL((gemm1_tail_finish_kernel<QMODE, 4, BM>), grid, block, 0, s, part, sorted, npp, n_tiles, W,
                         P, Ip, limit, aq, as);
      break;
    default:
      hipLaunchKernelGGL((gemm1_tail_finish_kernel<QMODE, 8, BM>), grid, block, 0, s, part, sorted, npp, n_tiles, W,
                         P, Ip, limit, aq, as);
      break;
  }
}

template <int QMODE>
static void launch_tail_finish_mode(int ks, int block_m, const float* part, const int32_t* sorted,
                                    const int32_t* npp, int n_tiles, int W, int P, int Ip, float limit, uint8_t* aq,
                                    void* as, hipStream_t s) {
  if (block_m == 16)
    launch_tail_finish_bm<QMODE, 16>(ks, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
  else if (block_m == 32)
    launch_tail_finish_bm<QMODE, 32>(ks, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
  else if (block_m == 64)
    launch_tail_finish_bm<QMODE, 64>(ks, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
  else
    launch_tail_finish_bm<QMODE, 128>(ks, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
}

hipError_t launch_gemm1_tail_finish(int mode, int ks, int block_m, const float* part, const int32_t* sorted,
                                    const int32_t* npp, int n_tiles, int W, int P, int Ip, float limit, uint8_t* aq,
                                    void* as, hipStream_t s) {
  if (mode == kQuantFp8)
    launch_tail_finish_mode<kQuantFp8>(ks, block_m, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
  else if (mode == kQuantFp8E8)
    launch_tail_finish_mode<kQuantFp8E8>(ks, block_m, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
  else
    launch_tail_finish_mode<kQuantMx>(ks, block_m, part, sorted, npp, n_tiles, W, P, Ip, limit, aq, as, s);
  return hipGetLastError();
}

// out[t, c0 + h] = bf16(sum_j y[t*k + j, h]) with the slot sum in fp32 in
// order j = 0..k-1 (with K pieces: plane by plane, slots in order within
// each), for h < cols (a column chunk of the output).  Each y value is
// decoded exactly, q * 2^s (int16 q, the exponent of its 64-column group).
// 8 stored values per thread (one 16-byte non-temporal load per slot: y is
// read once): positions p .. p+7 of a 64-column group, which hold output
// columns y_group_col(p) .. +3 and 16 further .. +3; each four bf16 results
// go out as one 8-byte store when the row stride allows it.  The group lies
// inside the y rows GEMM2 wrote (the chunk width is a multiple of 256, or all
// Hp); only columns below `cols` are stored.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const uint8_t* __restrict__ y, int64_t yexp, int k, int cols,
                                                      int64_t ldy, int nplanes, int64_t plane,
                                                      uint16_t* __restrict__ out, int64_t ld_out, int vec_store) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const int t = blockIdx.y;
  // stored positions h .. h+7 of a row: output columns c and c + 16 (4 each)
  const int h = (blockIdx.x * 256 + threadIdx.x) * 8;
  if ((h & ~63) >= cols) return;
  const int c = y_group_col(h);
  const int64_t lde = ldy / 64;
  float a[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  // plane by plane (K pieces of GEMM2); in a plane every slot's loads are
  // issued before the first add (k <= KMAX)
  for (int ps = 0; ps < nplanes; ++ps) {
    const uint8_t* pl = y + ps * plane;
    const int16_t* base = (const int16_t*)pl + (int64_t)t * k * ldy + h;
    const int8_t* eb = (const int8_t*)(pl + yexp) + (int64_t)t * k * lde + h / 64;
    u4 v[KMAX];
    int ex[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        v[j] = __builtin_nontemporal_load((const u4*)(base + (int64_t)j * ldy));
        ex[j] = eb[(int64_t)j * lde];
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = v[j][d];
          a[2 * d] += ldexpf((float)(int)(int16_t)(wd & 0xFFFFu), ex[j]);
          a[2 * d + 1] += ldexpf((float)((int)wd >> 16), ex[j]);
        }
      }
    }
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int c0 = c + 16 * half;
    uint16_t* o = out + (int64_t)t * ld_out + c0;
    const float* av = a + 4 * half;
    if (vec_store && c0 + 4 <= cols) {
      *(uint2*)o = make_uint2((uint32_t)f32_to_bf16(av[0]) | ((uint32_t)f32_to_bf16(av[1]) << 16),
                              (uint32_t)f32_to_bf16(av[2]) | ((uint32_t)f32_to_bf16(av[3]) << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c0 + i < cols) o[i] = f32_to_bf16(av[i]);
    }
  }
}

hipError_t launch_combine(const uint8_t* y, int64_t yexp, int T, int k, int c0, int cols, int64_t ldy, int nplanes,
                          int64_t plane, uint16_t* out, int64_t ld_out, hipStream_t s) {
  if (T <= 0 || cols <= 0) return hipSuccess;
  uint16_t* o = out + c0;
  // 8-byte stores need every row start 8-byte aligned
  const int vec = ((uintptr_t)o % 8 == 0) && (ld_out % 4 == 0);
  dim3 grid((unsigned)((cols + 2047) / 2048), (unsigned)T), block(256);
  if (k <= 2)
    hipLaunchKernelGGL(combine_kernel<2>, grid, block, 0, s, y, yexp, k, cols, ldy, nplanes, plane, o, ld_out, vec);
  else if (k <= 4)
    hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, s, y, yexp, k, cols, ldy, nplanes, plane, o, ld_out, vec);
  else if (k <= 8)
    hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, s, y, yexp, k, cols, ldy, nplanes, plane, o, ld_out, vec);
  else
    hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, s, y, yexp, k, cols, ldy, nplanes, plane, o, ld_out, vec);
  return hipGetLastError();
}

}  // namespace moe
