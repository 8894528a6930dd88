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
// A (activations) is staged through LDS per 128-wide K block (double
// buffered); B (weights) goes straight from HBM into MFMA operand registers
// from the TILED_V1 layout (1 KB contiguous per wave load), one K block ahead.
//   FP8: each 16x16x128 MFMA covers exactly one 128-wide scale block, so its
//        fp32 result is scaled by act_scale(row) * w_scale(block) and added to
//        the accumulator (fp32 promotion per K block).
//   MX:  the scaled MFMA applies the E8M0 scales of A and B itself.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int MODE>
struct GemmCfg {
  static constexpr int AROW = (MODE == kQuantMx) ? 64 : 128;   // A bytes per row per K block (HBM)
  static constexpr int LROW = (MODE == kQuantFp8F16) ? 256 : AROW;  // bytes per row in LDS
  static constexpr int ASTR = LROW + 16;                        // padded LDS row stride
  static constexpr int CPR = AROW / 16;                         // 16-byte chunks per A row
};

template <int MODE, int BM>
struct alignas(16) GemmSmem {
  uint8_t a[2][BM * GemmCfg<MODE>::ASTR];
  uint32_t asc[2][BM];  // FP8: f32 bits of the act scale; MX: 4 E8M0 bytes
  int32_t src[BM];      // A source row (token or sorted position), -1 = pad
  int32_t sid[BM];      // pair index of each row (GEMM2 epilogue)
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

// B operand registers for the wave's 4 tiles at K block kb.
template <int MODE>
__device__ __forceinline__ void load_b(const GemmArgs& p, const int64_t (&tbase)[4], int kb, v8i (&b)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (MODE != kQuantMx) {
      const uint8_t* t = p.B + (tbase[j] + kb) * 2048 + lane * 16;
      uint4 lo = *(const uint4*)t;
      uint4 hi = *(const uint4*)(t + 1024);
      b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      const uint8_t* t = p.B + (tbase[j] + kb) * 1024 + lane * 16;
      uint4 lo = *(const uint4*)t;
      b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
    }
  }
}

template <int BM, int OPB>
__device__ __forceinline__ void mx_step(const GemmSmem<kQuantMx, BM>& sm, int buf, const v8i (&b)[4],
                                        const int (&sb)[4], v4f (&acc)[BM / 16][4]) {
  constexpr int ASTR = GemmCfg<kQuantMx>::ASTR;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < BM / 16; ++m) {
    const int r = m * 16 + (lane & 15);
    uint4 a0 = *(const uint4*)(&sm.a[buf][r * ASTR + (lane >> 4) * 16]);
    v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
    int sa = (int)((sm.asc[buf][r] >> (8 * (lane >> 4))) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = mfma_fp4_scaled<OPB>(a, b[j], acc[m][j], sa, sb[j]);
  }
}

template <int MODE, int BM, bool G1>
__global__ __launch_bounds__(256) void moe_gemm_kernel(GemmArgs p) {
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

  // the wave's four 16-row B tiles (global tile index, times KB)
  int t16[4];
  if constexpr (G1) {
    const int ib = p.Ip / 16;
    t16[0] = nt * 8 + 2 * wave;
    t16[1] = t16[0] + 1;
    t16[2] = ib + t16[0];
    t16[3] = ib + t16[1];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) t16[j] = nt * 16 + 4 * wave + j;
  }
  const bool wave_active = G1 ? true : (nt * 256 + 64 * wave < p.N);
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

  // FP8 weight block scales: block row of each tile (uniform per wave)
  const int NB128 = p.N / 128;
  const float* ws = (const float*)p.Bs;

  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < KB;
    if (more) {
      if (wave_active) load_b<MODE>(p, tbase, kb + 1, bn);
      load_a_regs<MODE, BM>(p, sm, kb + 1, ar, sr);
    }
    if (wave_active) {
      if constexpr (MODE == kQuantFp8) {
        float sw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sw[j] = ws[((int64_t)e * NB128 + t16[j] / 8) * KB + kb];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint8_t* ap = &sm.a[buf][(m * 16 + (lane & 15)) * ASTR + (lane >> 4) * 32];
          uint4 a0 = *(const uint4*)ap;
          uint4 a1 = *(const uint4*)(ap + 16);
          v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          const uint4 s4 = *(const uint4*)(&sm.asc[buf][m * 16 + (lane >> 4) * 4]);
          const float sa[4] = {__uint_as_float(s4.x), __uint_as_float(s4.y), __uint_as_float(s4.z),
                               __uint_as_float(s4.w)};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v4f t = mfma_fp8(a, bc[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[i], sa[i] * sw[j], acc[m][j][i]);
          }
        }
      } else if constexpr (MODE == kQuantFp8F16) {
        // widen the B tiles to f16: step s uses the lane's bytes 8s..8s+7
        // (K = 32*(lane/16) + 8s + i); A in LDS is read with the same K map
        float sw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sw[j] = ws[((int64_t)e * NB128 + t16[j] / 8) * KB + kb];
        v8h bh[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const uint32_t d0 = (uint32_t)bc[j][2 * st], d1 = (uint32_t)bc[j][2 * st + 1];
            const uint4 h = make_uint4(e4m3x2_to_f16x2<false>(d0), e4m3x2_to_f16x2<true>(d0),
                                       e4m3x2_to_f16x2<false>(d1), e4m3x2_to_f16x2<true>(d1));
            bh[j][st] = __builtin_bit_cast(v8h, h);
          }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint8_t* ap = &sm.a[buf][(m * 16 + (lane & 15)) * ASTR + (lane >> 4) * 64];
          v8h a[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) a[st] = *(const v8h*)(ap + 16 * st);
          const uint4 s4 = *(const uint4*)(&sm.asc[buf][m * 16 + (lane >> 4) * 4]);
          const float sa[4] = {__uint_as_float(s4.x), __uint_as_float(s4.y), __uint_as_float(s4.z),
                               __uint_as_float(s4.w)};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v4f t = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st) t = mfma_f16(a[st], bh[j][st], t);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[i], sa[i] * sw[j], acc[m][j][i]);
          }
        }
      } else {
        if ((kb & 3) == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t* sp = (const uint32_t*)p.Bs + (((int64_t)e * NT16 + t16[j]) * ((KB + 3) / 4) + kb / 4) * 64 + lane;
            sbw[j] = (int)*sp;
          }
        }
        switch (kb & 3) {
          case 0: mx_step<BM, 0>(sm, buf, bc, sbw, acc); break;
          case 1: mx_step<BM, 1>(sm, buf, bc, sbw, acc); break;
          case 2: mx_step<BM, 2>(sm, buf, bc, sbw, acc); break;
          default: mx_step<BM, 3>(sm, buf, bc, sbw, acc); break;
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
    // ---- SwiGLU + re-quantisation of the intermediate -------------------
    // lane holds rows m*16 + 4*(lane/16) + i, intermediate columns
    // 32*wave + 16*jj + lane%16 (jj = 0, 1): gate in acc[m][jj], up in acc[m][jj+2].
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
        rmax[m][i] = max_xor<16>(mx);
      }
    uint8_t* stage = &sm.a[0][0];  // BM x 128 code bytes (A buffers are free now)
    if constexpr (MODE != kQuantMx) {
      if ((lane & 15) == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.red[wave][m * 16 + 4 * (lane >> 4) + i] = rmax[m][i];
      }
      __syncthreads();
      const int nsc = p.Ip / 128;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m * 16 + 4 * (lane >> 4) + i;
          float amax = fmaxf(fmaxf(sm.red[0][r], sm.red[1][r]), fmaxf(sm.red[2][r], sm.red[3][r]));
          float s = amax / kE4M3Max;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            uint32_t code = (amax > 0.0f) ? fp8_quant(av[m][jj][i], s) : 0u;
            stage[r * 128 + 32 * wave + 16 * jj + (lane & 15)] = (uint8_t)code;
          }
          if (wave == 0 && (lane & 15) == 0) ((float*)p.as)[(int64_t)(row0 + r) * nsc + nt] = (amax > 0.0f) ? s : 0.0f;
        }
      __syncthreads();
      // copy out BM x 128 bytes, 16 bytes per chunk
      for (int c = tid; c < BM * 8; c += 256) {
        int r = c >> 3, cc = c & 7;
        *(uint4*)(p.aq + (int64_t)(row0 + r) * p.Ip + nt * 128 + cc * 16) = *(const uint4*)(&stage[r * 128 + cc * 16]);
      }
    } else {
      __syncthreads();  // every wave is done reading the A buffers
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
      // pack 32 codes -> 16 bytes per chunk
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
  } else {
    // ---- weighted per-pair output rows ------------------------------------
    if (!wave_active) return;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + 4 * (lane >> 4) + i;
        const int sid = sm.sid[r];
        if (sid < p.num_pairs) {
          const float wt = p.topk_w[sid];
          float* yrow = p.y + (int64_t)sid * p.N + nt * 256 + 64 * wave + (lane & 15);
#pragma unroll
          for (int j = 0; j < 4; ++j) yrow[16 * j] = wt * acc[m][j][i];
        }
      }
  }
}

template <int MODE, bool G1>
static hipError_t launch_gemm_mode(int block_m, int nb, const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)nb * a.n_tiles)), block(256);
  switch (block_m) {
    case 16: hipLaunchKernelGGL((moe_gemm_kernel<MODE, 16, G1>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((moe_gemm_kernel<MODE, 32, G1>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((moe_gemm_kernel<MODE, 64, G1>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((moe_gemm_kernel<MODE, 128, G1>), grid, block, 0, s, a); break;
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
