// Top-k routing and the padded stable expert permutation.
//
// Routing: FreeToken PR #270 "glm5_next: support GLM-5.3-Flash (hybrid KDA +
// DSA, mHC, NVFP4 expert offload)", Summary (288-expert top-8 routing; the
// fused router epilogue picks the same ids as a reference top-k).  Selection
// is on the raw logits, descending, ties to the lower expert id; weights are
// the softmax over the k selected logits.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// (value, id) is better than (ov, oid): larger value, ties to the lower id.
__device__ __forceinline__ bool better(float ov, int oid, float v, int id) {
  return ov > v || (ov == v && oid < id);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& id) {
  // lanes outside ROW_MASK keep their own value (old = src), which is a no-op
  float ov = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
  int oid = __builtin_amdgcn_update_dpp(id, id, CTRL, ROW_MASK, 0xF, false);
  if (better(ov, oid, v, id)) {
    v = ov;
    id = oid;
  }
}

// Wave-wide argmax with DPP row operations: quad swaps (xor 1, xor 2), half
// and full row mirrors make every 16-lane row uniform, row broadcasts of
// lanes 15 and 31 fold the rows into lane 63, which is read back uniformly.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  argmax_step<0xB1, 0xF>(v, id);   // quad_perm [1,0,3,2]
  argmax_step<0x4E, 0xF>(v, id);   // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xF>(v, id);  // row_half_mirror
  argmax_step<0x140, 0xF>(v, id);  // row_mirror
  argmax_step<0x142, 0xA>(v, id);  // row_bcast:15 into rows 1, 3
  argmax_step<0x143, 0xC>(v, id);  // row_bcast:31 into rows 2, 3
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  id = __builtin_amdgcn_readlane(id, 63);
}

// One wave per token.  Each lane holds the logits of experts lane + 64*i;
// k rounds of a wave-wide argmax pick the experts in slot order.  NaN logits
// compare as -inf.  The softmax denominator is summed in slot order.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    float x = (e < E) ? row[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
    if (e < E) avail |= 1u << i;
  }
  float my_v = -INFINITY;
  int my_e = 0;
  float lmax = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      if (((avail >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
    wave_argmax(bv, be);
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (j == 0) lmax = bv;
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float d = (my_v == lmax) ? 0.0f : (my_v - lmax);
  const float ex = (lane < k) ? expf(d) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  int vpl = (E + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 5)
    hipLaunchKernelGGL(route_topk_kernel<5>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permute-align: one workgroup of NW waves; wave w owns the token range
// [w*Tw, (w+1)*Tw).  The pairs of expert e in increasing f = t*k + j are, when
// no token lists an expert twice (what top-k routing produces), the tokens
// that chose e in increasing t, so:
//   pass 1: per-wave expert histograms (LDS atomics);
//   scan:   padded counts -> offsets; per-wave cursors = offset + pairs of
//           earlier waves;
//   pass 2: each wave walks its tokens 64 at a time (lane = token, its k ids
//           in registers); a 64-bit LDS mask per expert marks the lanes that
//           chose it, and a pair's position is its cursor + popcount(mask &
//           lanes below).
// If some token lists an expert twice, pass 2 instead ranks pairs with a
// ballot match loop over f order (same result definition, slower).
// ---------------------------------------------------------------------------
constexpr int kMaxTopK = 16;

template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch /* [NW] */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int tw = scratch[w];
    if (w < wave) base += tw;
    total += tw;
  }
  __syncthreads();
  return base + incl - v;
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void permute_align_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                                int BM, int nb, int32_t* __restrict__ sorted_ids,
                                                                int32_t* __restrict__ block_expert,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ npp) {
  constexpr int NT = 64 * NW;
  extern __shared__ __align__(16) unsigned char perm_smem[];
  int32_t* cur = (int32_t*)perm_smem;                     // [NW][E] pair counts, then positions
  uint32_t* mask = (uint32_t*)(cur + NW * E);             // [NW][E][2] lane masks (lo, hi)
  int32_t* scratch = (int32_t*)(mask + NW * E * 2);       // [NW] + duplicate flag
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = T * k;

  for (int i = tid; i < NW * E; i += NT) {
    cur[i] = 0;
    mask[2 * i] = 0;
    mask[2 * i + 1] = 0;
  }
  if (tid == 0) scratch[NW] = 0;
  __syncthreads();

  const int Tw = (T + NW - 1) / NW;
  const int t_begin = wave * Tw;
  const int t_end = min(T, t_begin + Tw);

  // pass 1: histograms; detect a token that lists an expert twice
  bool dup = false;
  for (int t = t_begin + lane; t < t_end; t += 64) {
    int ex[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) ex[j] = (j < k) ? ids[(size_t)t * k + j] : -1;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int e = ex[j];
      if (j >= k || e < 0 || e >= E) continue;
      atomicAdd(&cur[wave * E + e], 1);
#pragma unroll
      for (int j2 = 0; j2 < j; ++j2) dup |= (ex[j2] == e);
    }
  }
  if (dup) scratch[NW] = 1;
  __syncthreads();
  const bool any_dup = scratch[NW] != 0;

  // scan of padded counts (E <= 1024)
  constexpr int EPT = (1024 + NT - 1) / NT;
  int cnt[EPT], pc[EPT];
  int local = 0;
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    int e = tid * EPT + q;
    int c = 0;
    if (e < E)
      for (int w = 0; w < NW; ++w) c += cur[w * E + e];
    cnt[q] = c;
    pc[q] = ((c + BM - 1) / BM) * BM;
    local += pc[q];
  }
  int total;
  int off = block_exclusive_scan<NW>(local, scratch, total);
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    int e = tid * EPT + q;
    if (e < E) {
      offsets[e] = off;
      int base = off;
      for (int w = 0; w < NW; ++w) {
        const int c = cur[w * E + e];
        cur[w * E + e] = base;  // only this thread touches expert e
        base += c;
      }
      for (int r = off + cnt[q]; r < off + pc[q]; ++r) sorted_ids[r] = P;
      for (int b = off / BM; b < (off + pc[q]) / BM; ++b) block_expert[b] = e;
    }
    off += pc[q];
  }
  if (tid == 0) {
    offsets[E] = total;
    *npp = total;
  }
  for (int r = total + tid; r < nb * BM; r += NT) sorted_ids[r] = P;
  for (int b = total / BM + tid; b < nb; b += NT) block_expert[b] = -1;
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (!any_dup) {
    const int rounds = (Tw + 63) / 64;
    for (int r = 0; r < rounds; ++r) {
      const int t = t_begin + r * 64 + lane;
      const bool live = t < t_end;
      int ex[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        int e = (live && j < k) ? ids[(size_t)t * k + j] : -1;
        ex[j] = (e >= 0 && e < E) ? e : -1;
      }
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (ex[j] >= 0) atomicOr(&mask[(wave * E + ex[j]) * 2 + (lane >> 5)], 1u << (lane & 31));
      __syncthreads();
      uint64_t m[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        m[j] = 0;
        if (ex[j] >= 0) {
          const uint2 mm = *(const uint2*)&mask[(wave * E + ex[j]) * 2];
          m[j] = (uint64_t)mm.x | ((uint64_t)mm.y << 32);
          sorted_ids[cur[wave * E + ex[j]] + __popcll(m[j] & lt_mask)] = t * k + j;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (ex[j] >= 0 && (m[j] & lt_mask) == 0) {  // the expert's first lane
          cur[wave * E + ex[j]] += __popcll(m[j]);
          *(uint2*)&mask[(wave * E + ex[j]) * 2] = make_uint2(0u, 0u);
        }
      }
      __syncthreads();
    }
  } else {
    // general order: lane = pair, in f order over the wave's token range
    const int f_begin = t_begin * k, f_end = t_end * k;
    const int frounds = (Tw * k + 63) / 64;
    for (int r = 0; r < frounds; ++r) {
      const int f = f_begin + r * 64 + lane;
      const int e = (f < f_end) ? ids[f] : -1;
      const bool valid = e >= 0 && e < E;
      uint64_t active = __ballot(valid);
      int rank = 0;
      bool leader = false;
      int cnt_leader = 0;
      while (active) {
        const int ld = __ffsll((unsigned long long)active) - 1;
        const int le = __builtin_amdgcn_readlane(e, ld);
        const uint64_t mm = __ballot(valid && e == le);
        if (valid && e == le) rank = __popcll(mm & lt_mask);
        if (lane == ld) {
          leader = true;
          cnt_leader = __popcll(mm);
        }
        active &= ~mm;
      }
      if (valid) sorted_ids[cur[wave * E + e] + rank] = f;
      __syncthreads();
      if (leader) cur[wave * E + e] += cnt_leader;
      __syncthreads();
    }
  }
}

hipError_t launch_permute_align(const int32_t* ids, int T, int k, int E, int block_m, int nb, int32_t* sorted_ids,
                                int32_t* block_expert, int32_t* offsets, int32_t* npp, hipStream_t s) {
  // 16 waves when their per-wave tables fit in 64 KB of LDS and there are
  // enough tokens to share out, else 4 waves.
  const bool wide = T >= 1024 && (size_t)16 * E * 12 + 17 * 4 <= 65536;
  if (wide) {
    size_t smem = (size_t)16 * E * 12 + 17 * 4;
    hipLaunchKernelGGL(permute_align_kernel<16>, dim3(1), dim3(1024), smem, s, ids, T, k, E, block_m, nb,
                       sorted_ids, block_expert, offsets, npp);
  } else {
    size_t smem = (size_t)4 * E * 12 + 5 * 4;
    hipLaunchKernelGGL(permute_align_kernel<4>, dim3(1), dim3(256), smem, s, ids, T, k, E, block_m, nb, sorted_ids,
                       block_expert, offsets, npp);
  }
  return hipGetLastError();
}

}  // namespace moe
