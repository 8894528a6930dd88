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
// Work decomposition: one workgroup (4 waves) per (M block, N tile).  An M
// block is block_m rows of the expert-sorted pair list, all of one expert.
//   GEMM1: N tile = 128 intermediate columns = 256 w13 rows; wave w owns
//          intermediate columns 32w..32w+31, i.e. two 16-row gate tiles and
//          the two matching up tiles, so the SwiGLU pairs gate and up values
//          inside one lane.
//   GEMM2: N tile = 256 output columns; wave w owns rows 64w..64w+63.
// B (weights) goes straight from HBM into MFMA operand registers from the
// TILED_V1 layout (1 KB contiguous per wave load).  For block_m >= 64 the A
// (activation) tile of each 128-wide K block is staged through LDS (double
// buffered); for block_m <= 32 each lane loads its A fragments directly and
// the K loop has no barrier (see moe_gemm_direct_kernel).
//   FP8: each 128-wide K block is one scale block, so its fp32 partial sum
//        is scaled by act_scale(row) * w_scale(block) and added to the
//        accumulator (fp32 promotion per K block).  GEMM1 widens the FP8
//        operands to f16 and uses the f16 MFMA (exact fp32 sums); GEMM2 uses
//        the FP8 MFMA directly.
//   MX:  the scaled MFMA applies the E8M0 scales of A and B itself.
#include <utility>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int MODE>
struct GemmCfg {
  static constexpr int AROW = (MODE == kQuantMx) ? 64 : 128;        // A bytes per row per K block (HBM)
  static constexpr int LROW = (MODE == kQuantFp8F16) ? 256 : AROW;  // bytes per row in LDS
  static constexpr int ASTR = LROW + 16;                             // padded LDS row stride
  static constexpr int CPR = AROW / 16;                              // 16-byte chunks per A row
};

// ---------------------------------------------------------------------------
// One 128-wide K block of the wave's MT x 4 output tiles, on register operands.
//   a: A fragments of the MT row subtiles; b: the 4 B tiles (FP8 bytes, or
//   packed E2M1 in the low 4 dwords); FP8 modes add act scales sa (rows
//   4*(lane/16)+i of each subtile) and weight block scales sw (per tile).
// ---------------------------------------------------------------------------
template <int MT>
__device__ __forceinline__ void step_fp8(const v8i (&a)[MT], const float (&sa)[MT][4], const v8i (&b)[4],
                                         const float (&sw)[4], v4f (&acc)[MT][4]) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4f t = mfma_fp8(a[m], b[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[i], sa[m][i] * sw[j], acc[m][j][i]);
    }
}

// The lane's 32 FP8 bytes as four f16 operands: step st holds bytes
// 8st..8st+7, i.e. K = 32*(lane/16) + 8st + i for both A and B.
__device__ __forceinline__ void widen_fp8(const v8i& w, v8h (&h)[4]) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const uint32_t d0 = (uint32_t)w[2 * st], d1 = (uint32_t)w[2 * st + 1];
    const uint4 v = make_uint4(e4m3x2_to_f16x2<false>(d0), e4m3x2_to_f16x2<true>(d0),
                               e4m3x2_to_f16x2<false>(d1), e4m3x2_to_f16x2<true>(d1));
    h[st] = __builtin_bit_cast(v8h, v);
  }
}

template <int MT>
__device__ __forceinline__ void step_f16(const v8h (&a)[MT][4], const float (&sa)[MT][4], const v8i (&b)[4],
                                         const float (&sw)[4], v4f (&acc)[MT][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v8h bh[4];
    widen_fp8(b[j], bh);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      v4f t = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) t = mfma_f16(a[m][st], bh[st], t);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[i], sa[m][i] * sw[j], acc[m][j][i]);
    }
  }
}

template <int MT, int OPB>
__device__ __forceinline__ void step_mx(const v8i (&a)[MT], const int (&sa)[MT], const v8i (&b)[4],
                                        const int (&sb)[4], v4f (&acc)[MT][4]) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = mfma_fp4_scaled<OPB>(a[m], b[j], acc[m][j], sa[m], sb[j]);
}

template <int MT>
__device__ __forceinline__ void step_mx_kb(int kb, const v8i (&a)[MT], const int (&sa)[MT], const v8i (&b)[4],
                                           const int (&sb)[4], v4f (&acc)[MT][4]) {
  switch (kb & 3) {
    case 0: step_mx<MT, 0>(a, sa, b, sb, acc); break;
    case 1: step_mx<MT, 1>(a, sa, b, sb, acc); break;
    case 2: step_mx<MT, 2>(a, sa, b, sb, acc); break;
    default: step_mx<MT, 3>(a, sa, b, sb, acc); break;
  }
}

#ifndef MOE_NT_B
#define MOE_NT_B 1
#endif
#ifndef MOE_KROT
#define MOE_KROT 0
#endif

// Weights are read once per launch: optionally with a non-temporal hint.
__device__ __forceinline__ uint4 load_stream(const uint8_t* ptr) {
#if MOE_NT_B
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = __builtin_nontemporal_load((const u32x4*)ptr);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *(const uint4*)ptr;
#endif
}

// B operand registers for the wave's 4 tiles at K block kb (TILED_V1).
template <int MODE>
__device__ __forceinline__ void load_b(const GemmArgs& p, const int64_t (&tbase)[4], int kb, v8i (&b)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (MODE != kQuantMx) {
      const uint8_t* t = p.B + (tbase[j] + kb) * 2048 + lane * 16;
      uint4 lo = load_stream(t);
      uint4 hi = load_stream(t + 1024);
      b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      const uint8_t* t = p.B + (tbase[j] + kb) * 1024 + lane * 16;
      uint4 lo = load_stream(t);
      b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
    }
  }
}

// E8M0 dwords of the wave's B tiles for the group of 4 K blocks holding kb.
__device__ __forceinline__ void load_b_scales(const GemmArgs& p, int e, const int (&t16)[4], int kb, int (&sb)[4]) {
  const int lane = threadIdx.x & 63;
  const int KB = p.K / 128, NT16 = p.N / 16;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    sb[j] = (int)((const uint32_t*)p.Bs)[(((int64_t)e * NT16 + t16[j]) * ((KB + 3) / 4) + kb / 4) * 64 + lane];
}

// fp32 block scales of the wave's B tiles at kb (uniform per wave).
__device__ __forceinline__ void load_w_scales(const GemmArgs& p, int e, const int (&t16)[4], int kb, float (&sw)[4]) {
  const int KB = p.K / 128;
  const float* ws = (const float*)p.Bs;
#pragma unroll
  for (int j = 0; j < 4; ++j) sw[j] = ws[((int64_t)e * (p.N / 128) + t16[j] / 8) * KB + kb];
}

// ---------------------------------------------------------------------------
// Epilogues.  Lane holds acc[m][j][i] = C[row m*16 + 4*(lane/16) + i]
// [column 16*j + lane%16 of the wave's tiles].
// ---------------------------------------------------------------------------

// GEMM1: gate in acc[m][jj], up in acc[m][jj+2] (jj = 0, 1) for intermediate
// column 32*wave + 16*jj + lane%16 of the N tile.  SwiGLU, re-quantise the
// row per 1x128 (FP8, amax across the 4 waves) or per 1x32 (MX, the wave's
// own 32 columns), stage the codes in LDS, write 16-byte chunks.
template <int MODE, int BM>
__device__ __forceinline__ void epilogue_gemm1(const GemmArgs& p, const v4f (&acc)[BM / 16][4], float (*red)[BM],
                                               uint8_t* stage, int row0, int nt, int wave) {
  constexpr int MT = BM / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const float L = p.limit;
  float av[MT][2][4];
  float rmax[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float a = swiglu_clamped(acc[m][jj][i], acc[m][jj + 2][i], L);
        av[m][jj][i] = a;
        mx = fmaxf(mx, fabsf(a));
      }
      rmax[m][i] = group_max<16>(mx);
    }
  if constexpr (MODE != kQuantMx) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][m * 16 + 4 * (lane >> 4) + i] = rmax[m][i];
    }
    __syncthreads();
    const int nsc = p.Ip / 128;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + 4 * (lane >> 4) + i;
        float amax = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
        float s = amax / kE4M3Max;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          uint32_t code = (amax > 0.0f) ? fp8_quant(av[m][jj][i], s) : 0u;
          stage[r * 128 + 32 * wave + 16 * jj + (lane & 15)] = (uint8_t)code;
        }
        if (wave == 0 && (lane & 15) == 0) ((float*)p.as)[(int64_t)(row0 + r) * nsc + nt] = (amax > 0.0f) ? s : 0.0f;
      }
    __syncthreads();
    for (int c = tid; c < BM * 8; c += 256) {
      int r = c >> 3, cc = c & 7;
      *(uint4*)(p.aq + (int64_t)(row0 + r) * p.Ip + nt * 128 + cc * 16) = *(const uint4*)(&stage[r * 128 + cc * 16]);
    }
  } else {
    const int nsc = p.Ip / 32;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + 4 * (lane >> 4) + i;
        uint32_t b = e8m0_byte(rmax[m][i]);
        float inv = e8m0_inverse(b);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          stage[r * 128 + 32 * wave + 16 * jj + (lane & 15)] = (uint8_t)mx_quant(av[m][jj][i], inv);
        if ((lane & 15) == 0) ((uint8_t*)p.as)[(int64_t)(row0 + r) * nsc + nt * 4 + wave] = (uint8_t)b;
      }
    __syncthreads();
    for (int c = tid; c < BM * 4; c += 256) {
      int r = c >> 2, cc = c & 3;
      const uint8_t* src = &stage[r * 128 + cc * 32];
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) {
          uint32_t lo = src[q * 8 + 2 * b2], hi = src[q * 8 + 2 * b2 + 1];
          v |= (lo | (hi << 4)) << (8 * b2);
        }
        w[q] = v;
      }
      *(uint4*)(p.aq + (int64_t)(row0 + r) * (p.Ip / 2) + nt * 64 + cc * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// GEMM2: y[pair, column] = topk_w[pair] * C for the real pairs of the block.
template <int BM>
__device__ __forceinline__ void epilogue_gemm2(const GemmArgs& p, const v4f (&acc)[BM / 16][4], const int32_t* sid_lds,
                                               int nt, int wave) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < BM / 16; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m * 16 + 4 * (lane >> 4) + i;
      const int sid = sid_lds[r];
      if (sid < p.num_pairs) {
        const float wt = p.topk_w[sid];
        float* yrow = p.y + (int64_t)sid * p.N + nt * 256 + 64 * wave + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) yrow[16 * j] = wt * acc[m][j][i];
      }
    }
}

// The wave's four 16-row B tiles: GEMM1 gate tiles nt*8+2w, +1 and the
// matching up tiles Ip/16 + ...; GEMM2 rows nt*256 + 64w + 16j.
template <bool G1>
__device__ __forceinline__ bool wave_tiles(const GemmArgs& p, int nt, int wave, int (&t16)[4]) {
  if constexpr (G1) {
    const int ib = p.Ip / 16;
    t16[0] = nt * 8 + 2 * wave;
    t16[1] = t16[0] + 1;
    t16[2] = ib + t16[0];
    t16[3] = ib + t16[1];
    return true;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) t16[j] = nt * 16 + 4 * wave + j;
    return nt * 256 + 64 * wave < p.N;
  }
}

// ===========================================================================
// LDS-staged kernel (block_m 64 / 128): the A tile of each K block is loaded
// once per workgroup into LDS (double buffered) and read by the 4 waves.
// ===========================================================================
template <int MODE, int BM>
struct alignas(16) GemmSmem {
  uint8_t a[2][BM * GemmCfg<MODE>::ASTR];
  uint32_t asc[2][BM];  // FP8: f32 bits of the act scale; MX: 4 E8M0 bytes
  int32_t src[BM];      // A source row (token or sorted position), -1 = pad
  int32_t sid[BM];      // pair index of each row
  float red[4][BM];     // GEMM1 FP8 epilogue: per-wave row amax
};

template <int MODE, int BM>
__device__ __forceinline__ void load_a_regs(const GemmArgs& p, const GemmSmem<MODE, BM>& sm, int kb,
                                            uint4 (&ar)[(BM * GemmCfg<MODE>::CPR + 255) / 256], uint32_t& sr) {
  constexpr int CPR = GemmCfg<MODE>::CPR;
  constexpr int NCH = (BM * CPR + 255) / 256;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    int c = tid + 256 * i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c < BM * CPR) {
      int r = c / CPR, cc = c % CPR;
      int src = sm.src[r];
      if (src >= 0) v = *(const uint4*)(p.A + (int64_t)src * p.lda + (int64_t)kb * GemmCfg<MODE>::AROW + cc * 16);
    }
    ar[i] = v;
  }
  sr = 0;
  if (tid < BM) {
    int src = sm.src[tid];
    if (src >= 0) {
      if constexpr (MODE != kQuantMx)
        sr = ((const uint32_t*)p.As)[(int64_t)src * p.ldas + kb];
      else
        sr = *(const uint32_t*)((const uint8_t*)p.As + (int64_t)src * p.ldas + kb * 4);
    }
  }
}

template <int MODE, int BM>
__device__ __forceinline__ void store_a_lds(GemmSmem<MODE, BM>& sm, int buf,
                                            const uint4 (&ar)[(BM * GemmCfg<MODE>::CPR + 255) / 256], uint32_t sr) {
  constexpr int CPR = GemmCfg<MODE>::CPR;
  constexpr int NCH = (BM * CPR + 255) / 256;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    int c = tid + 256 * i;
    if (c < BM * CPR) {
      int r = c / CPR, cc = c % CPR;
      if constexpr (MODE == kQuantFp8F16) {
        // widen 16 e4m3 values to f16 (K order kept)
        const uint4 v = ar[i];
        uint4 lo = make_uint4(e4m3x2_to_f16x2<false>(v.x), e4m3x2_to_f16x2<true>(v.x),
                              e4m3x2_to_f16x2<false>(v.y), e4m3x2_to_f16x2<true>(v.y));
        uint4 hi = make_uint4(e4m3x2_to_f16x2<false>(v.z), e4m3x2_to_f16x2<true>(v.z),
                              e4m3x2_to_f16x2<false>(v.w), e4m3x2_to_f16x2<true>(v.w));
        *(uint4*)(&sm.a[buf][r * GemmCfg<MODE>::ASTR + cc * 32]) = lo;
        *(uint4*)(&sm.a[buf][r * GemmCfg<MODE>::ASTR + cc * 32 + 16]) = hi;
      } else {
        *(uint4*)(&sm.a[buf][r * GemmCfg<MODE>::ASTR + cc * 16]) = ar[i];
      }
    }
  }
  if (tid < BM) sm.asc[buf][tid] = sr;
}

template <int MODE, int BM, bool G1>
__global__ __launch_bounds__(256) void moe_gemm_lds_kernel(GemmArgs p) {
  constexpr int MT = BM / 16;
  constexpr int ASTR = GemmCfg<MODE>::ASTR;
  constexpr int NCH = (BM * GemmCfg<MODE>::CPR + 255) / 256;
  __shared__ GemmSmem<MODE, BM> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mblk = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x % p.n_tiles;
  const int npp = __builtin_amdgcn_readfirstlane(*p.npp);
  if (mblk * BM >= npp) return;
  const int e = __builtin_amdgcn_readfirstlane(p.block_expert[mblk]);
  const int row0 = mblk * BM;
  const int KB = p.K / 128;
  const int NT16 = p.N / 16;

  if (tid < BM) {
    int sid = p.sorted_ids[row0 + tid];
    bool valid = sid < p.num_pairs;
    sm.sid[tid] = sid;
    sm.src[tid] = valid ? (G1 ? sid / p.top_k : row0 + tid) : -1;
  }
  int t16[4];
  const bool wave_active = wave_tiles<G1>(p, nt, wave, t16);
  int64_t tbase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tbase[j] = ((int64_t)e * NT16 + (wave_active ? t16[j] : 0)) * KB;

  v4f acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  __syncthreads();
  uint4 ar[NCH];
  uint32_t sr;
  load_a_regs<MODE, BM>(p, sm, 0, ar, sr);
  store_a_lds<MODE, BM>(sm, 0, ar, sr);
  v8i bc[4], bn[4];
  if (wave_active) load_b<MODE>(p, tbase, 0, bc);
  int sbw[4] = {0, 0, 0, 0};
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < KB;
    if (more) {
      if (wave_active) load_b<MODE>(p, tbase, kb + 1, bn);
      load_a_regs<MODE, BM>(p, sm, kb + 1, ar, sr);
    }
    if (wave_active) {
      if constexpr (MODE == kQuantMx) {
        if ((kb & 3) == 0) load_b_scales(p, e, t16, kb, sbw);
        v8i a[MT];
        int sa[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int r = m * 16 + (lane & 15);
          uint4 a0 = *(const uint4*)(&sm.a[buf][r * ASTR + (lane >> 4) * 16]);
          a[m] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
          sa[m] = (int)((sm.asc[buf][r] >> (8 * (lane >> 4))) & 0xFFu);
        }
        step_mx_kb<MT>(kb, a, sa, bc, sbw, acc);
      } else {
        float sw[4];
        load_w_scales(p, e, t16, kb, sw);
        float sa[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint4 s4 = *(const uint4*)(&sm.asc[buf][m * 16 + (lane >> 4) * 4]);
          sa[m][0] = __uint_as_float(s4.x);
          sa[m][1] = __uint_as_float(s4.y);
          sa[m][2] = __uint_as_float(s4.z);
          sa[m][3] = __uint_as_float(s4.w);
        }
        if constexpr (MODE == kQuantFp8) {
          v8i a[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const uint8_t* ap = &sm.a[buf][(m * 16 + (lane & 15)) * ASTR + (lane >> 4) * 32];
            uint4 a0 = *(const uint4*)ap;
            uint4 a1 = *(const uint4*)(ap + 16);
            a[m] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          }
          step_fp8<MT>(a, sa, bc, sw, acc);
        } else {
          v8h a[MT][4];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const uint8_t* ap = &sm.a[buf][(m * 16 + (lane & 15)) * ASTR + (lane >> 4) * 64];
#pragma unroll
            for (int st = 0; st < 4; ++st) a[m][st] = *(const v8h*)(ap + 16 * st);
          }
          step_f16<MT>(a, sa, bc, sw, acc);
        }
      }
    }
    if (more) store_a_lds<MODE, BM>(sm, buf ^ 1, ar, sr);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int j = 0; j < 4; ++j) bc[j] = bn[j];
    }
  }

  if constexpr (G1) {
    epilogue_gemm1<MODE, BM>(p, acc, sm.red, &sm.a[0][0], row0, nt, wave);
  } else {
    if (!wave_active) return;
    epilogue_gemm2<BM>(p, acc, sm.sid, nt, wave);
  }
}

// ===========================================================================
// Direct kernel (block_m 16 / 32, decode shapes): no LDS in the K loop.
// Each lane loads its own A fragments from global memory (the few token rows
// stay in L2) and the waves stream their B tiles independently through a ring
// of PD K blocks in registers, so PD-1 blocks of weights are in flight while
// one is multiplied.
// ===========================================================================
template <int BM>
struct alignas(16) DirectSmem {
  int32_t src[BM];
  int32_t sid[BM];
  float red[4][BM];
  uint8_t stage[BM * 128];
};

template <int MODE>
struct RawA {                    // one A fragment in HBM format
  uint4 lo, hi;                  // FP8: 32 bytes; MX: lo = 16 bytes
};

template <int MODE, int BM, bool G1, int PD>
__global__ __launch_bounds__(256) void moe_gemm_direct_kernel(GemmArgs p) {
  constexpr int MT = BM / 16;
  constexpr bool FP8ANY = MODE != kQuantMx;
  __shared__ DirectSmem<BM> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mblk = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x % p.n_tiles;
  const int npp = __builtin_amdgcn_readfirstlane(*p.npp);
  if (mblk * BM >= npp) return;
  const int e = __builtin_amdgcn_readfirstlane(p.block_expert[mblk]);
  const int row0 = mblk * BM;
  const int KB = p.K / 128;
  const int NT16 = p.N / 16;

  if (tid < BM) {
    int sid = p.sorted_ids[row0 + tid];
    bool valid = sid < p.num_pairs;
    sm.sid[tid] = sid;
    sm.src[tid] = valid ? (G1 ? sid / p.top_k : row0 + tid) : -1;
  }
  int t16[4];
  const bool wave_active = wave_tiles<G1>(p, nt, wave, t16);
  int64_t tbase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tbase[j] = ((int64_t)e * NT16 + (wave_active ? t16[j] : 0)) * KB;
  __syncthreads();

  // this lane's A rows: fragment row m*16 + lane%16, scale rows m*16 + 4*(lane/16) + i
  int asrc[MT];
  int ssrc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    asrc[m] = sm.src[m * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 4; ++i) ssrc[m][i] = sm.src[m * 16 + 4 * (lane >> 4) + i];
  }

  v4f acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (wave_active) {
    v8i rb[PD][4];
    RawA<MODE> ra[PD][MT];
    float rsa[PD][MT][4];   // FP8: act scales
    int rsx[PD][MT];        // MX: act scale byte
    float rsw[PD][4];       // FP8: weight block scales
    int rsb[PD][4];         // MX: weight scale dwords

    auto load_slot = [&](auto d_c, int kb) {
      constexpr int d = decltype(d_c)::value;
      load_b<MODE>(p, tbase, kb, rb[d]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
        if (asrc[m] >= 0) {
          if constexpr (FP8ANY) {
            const uint8_t* ap = p.A + (int64_t)asrc[m] * p.lda + (int64_t)kb * 128 + (lane >> 4) * 32;
            lo = *(const uint4*)ap;
            hi = *(const uint4*)(ap + 16);
          } else {
            lo = *(const uint4*)(p.A + (int64_t)asrc[m] * p.lda + (int64_t)kb * 64 + (lane >> 4) * 16);
          }
        }
        ra[d][m].lo = lo;
        ra[d][m].hi = hi;
        if constexpr (FP8ANY) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            rsa[d][m][i] = ssrc[m][i] >= 0 ? ((const float*)p.As)[(int64_t)ssrc[m][i] * p.ldas + kb] : 0.0f;
        } else {
          rsx[d][m] = asrc[m] >= 0 ? (int)((const uint8_t*)p.As)[(int64_t)asrc[m] * p.ldas + kb * 4 + (lane >> 4)] : 0;
        }
      }
      if constexpr (FP8ANY)
        load_w_scales(p, e, t16, kb, rsw[d]);
      else
        load_b_scales(p, e, t16, kb, rsb[d]);
    };

    auto compute_slot = [&](auto d_c, int kb) {
      constexpr int d = decltype(d_c)::value;
      if constexpr (MODE == kQuantMx) {
        v8i a[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          a[m] = v8i{(int)ra[d][m].lo.x, (int)ra[d][m].lo.y, (int)ra[d][m].lo.z, (int)ra[d][m].lo.w, 0, 0, 0, 0};
        step_mx_kb<MT>(kb, a, rsx[d], rb[d], rsb[d], acc);
      } else if constexpr (MODE == kQuantFp8) {
        v8i a[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          a[m] = v8i{(int)ra[d][m].lo.x, (int)ra[d][m].lo.y, (int)ra[d][m].lo.z, (int)ra[d][m].lo.w,
                     (int)ra[d][m].hi.x, (int)ra[d][m].hi.y, (int)ra[d][m].hi.z, (int)ra[d][m].hi.w};
        step_fp8<MT>(a, rsa[d], rb[d], rsw[d], acc);
      } else {
        v8h a[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          v8i raw = v8i{(int)ra[d][m].lo.x, (int)ra[d][m].lo.y, (int)ra[d][m].lo.z, (int)ra[d][m].lo.w,
                        (int)ra[d][m].hi.x, (int)ra[d][m].hi.y, (int)ra[d][m].hi.z, (int)ra[d][m].hi.w};
          widen_fp8(raw, a[m]);
        }
        step_f16<MT>(a, rsa[d], rb[d], rsw[d], acc);
      }
    };

    // K blocks are visited from a per-workgroup starting block so that the
    // waves in flight do not all address the same offset of their streams.
#if MOE_KROT
    const int kstart = (int)(((unsigned)blockIdx.x * 7u) % (unsigned)KB);
#else
    const int kstart = 0;
#endif
    auto kmap = [&](int kk) { int kb = kk + kstart; return kb >= KB ? kb - KB : kb; };
    // prologue: fill the ring
    [&]<int... D>(std::integer_sequence<int, D...>) {
      ((D < KB ? load_slot(std::integral_constant<int, D>{}, kmap(D)) : void()), ...);
    }(std::make_integer_sequence<int, PD>{});

    for (int kb0 = 0; kb0 < KB; kb0 += PD) {
      [&]<int... D>(std::integer_sequence<int, D...>) {
        (([&] {
           const int kk = kb0 + D;
           if (kk < KB) {
             compute_slot(std::integral_constant<int, D>{}, kmap(kk));
             if (kk + PD < KB) load_slot(std::integral_constant<int, D>{}, kmap(kk + PD));
           }
         }()),
         ...);
      }(std::make_integer_sequence<int, PD>{});
    }
  }

  if constexpr (G1) {
    epilogue_gemm1<MODE, BM>(p, acc, sm.red, sm.stage, row0, nt, wave);
  } else {
    if (!wave_active) return;
    epilogue_gemm2<BM>(p, acc, sm.sid, nt, wave);
  }
}

#ifndef MOE_DIRECT_PD
#define MOE_DIRECT_PD 2
#endif

template <int MODE, bool G1>
static hipError_t launch_gemm_mode(int block_m, int nb, const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)nb * a.n_tiles)), block(256);
  switch (block_m) {
    case 16: hipLaunchKernelGGL((moe_gemm_direct_kernel<MODE, 16, G1, MOE_DIRECT_PD>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((moe_gemm_direct_kernel<MODE, 32, G1, MOE_DIRECT_PD>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((moe_gemm_lds_kernel<MODE, 64, G1>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((moe_gemm_lds_kernel<MODE, 128, G1>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// GEMM1's output is re-quantised, so its sum must be fp32-exact: block FP8
// runs on the f16 MFMA (FP8 storage, exact widening in registers).
hipError_t launch_gemm1(int mode, int block_m, int nb, const GemmArgs& a, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  return mode == kQuantFp8 ? launch_gemm_mode<kQuantFp8F16, true>(block_m, nb, a, s)
                           : launch_gemm_mode<kQuantMx, true>(block_m, nb, a, s);
}

hipError_t launch_gemm2(int mode, int block_m, int nb, const GemmArgs& a, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  return mode == kQuantFp8 ? launch_gemm_mode<kQuantFp8, false>(block_m, nb, a, s)
                           : launch_gemm_mode<kQuantMx, false>(block_m, nb, a, s);
}

// out[t, h] = bf16(sum_j y[t*k + j, h]) with the slot sum in order j = 0..k-1.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int k, int H, int Hp,
                                                      uint16_t* __restrict__ out, int64_t ld_out) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  const float* base = y + (int64_t)t * k * Hp + h;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    float4 v = *(const float4*)(base + (int64_t)j * Hp);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  uint16_t* o = out + (int64_t)t * ld_out + h;
  o[0] = f32_to_bf16(acc.x);
  if (h + 1 < H) o[1] = f32_to_bf16(acc.y);
  if (h + 2 < H) o[2] = f32_to_bf16(acc.z);
  if (h + 3 < H) o[3] = f32_to_bf16(acc.w);
}

hipError_t launch_combine(const float* y, int T, int k, int H, int Hp, uint16_t* out, int64_t ld_out,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid((unsigned)((H + 1023) / 1024), (unsigned)T), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, s, y, k, H, Hp, out, ld_out);
  return hipGetLastError();
}

}  // namespace moe
