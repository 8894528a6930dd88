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

// One wave per token.  Each lane holds the logits of experts lane + 64*i;
// k rounds of a wave-wide argmax (value descending, id ascending) pick the
// experts in slot order.  NaN logits compare as -inf.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
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
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      bool ok = (avail >> i) & 1u;
      if (ok && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  float lmax = __shfl(my_v, 0, 64);
  float d = (my_v == lmax) ? 0.0f : (my_v - lmax);
  float ex = (lane < k) ? expf(d) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  int vpl = (E + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permute-align: one workgroup of 1024 threads (16 waves).
//   1. histogram of expert ids (LDS atomics);
//   2. exclusive scan of the block_m-padded counts -> offsets, num_post_padded;
//   3. pad sentinels and block owners (disjoint from the scatter targets);
//   4. stable scatter in rounds of 1024 pairs: a pair's position is its
//      expert's cursor + same-expert pairs in earlier waves of the round +
//      its rank among same-expert lanes of its own wave (ballot match loop).
// ---------------------------------------------------------------------------
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

__global__ __launch_bounds__(1024) void permute_align_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             int BM, int nb,
                                                             int32_t* __restrict__ sorted_ids,
                                                             int32_t* __restrict__ block_expert,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ npp) {
  extern __shared__ __align__(16) unsigned char perm_smem[];
  int32_t* cnt = (int32_t*)perm_smem;                    // [E]
  int32_t* cursor = cnt + E;                             // [E]
  int32_t* wave_tot = cursor + E;                        // [16]
  uint8_t* wcnt = (uint8_t*)(wave_tot + kPermWaves);     // [16][E]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
  __syncthreads();

  for (int f = tid; f < P; f += kPermThreads) {
    int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // exclusive scan over experts (E <= 1024: one expert per thread)
  int c = (tid < E) ? cnt[tid] : 0;
  int pc = ((c + BM - 1) / BM) * BM;
  int incl = pc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int w = 0; w < kPermWaves; ++w) {
    int tw = wave_tot[w];
    if (w < wave) wbase += tw;
    total += tw;
  }
  int off_e = wbase + incl - pc;
  if (tid < E) {
    offsets[tid] = off_e;
    cursor[tid] = off_e;
    for (int r = off_e + c; r < off_e + pc; ++r) sorted_ids[r] = P;
    for (int b = off_e / BM; b < (off_e + pc) / BM; ++b) block_expert[b] = tid;
  }
  if (tid == 0) {
    offsets[E] = total;
    *npp = total;
  }
  for (int r = total + tid; r < nb * BM; r += kPermThreads) sorted_ids[r] = P;
  for (int b = total / BM + tid; b < nb; b += kPermThreads) block_expert[b] = -1;
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kPermThreads) {
    int f = base + tid;
    int e = (f < P) ? ids[f] : -1;
    bool valid = (e >= 0 && e < E);
    uint64_t active = __ballot(valid);
    int rank = 0;
    bool leader = false;
    while (active) {
      int ld = __ffsll((unsigned long long)active) - 1;
      int le = __shfl(e, ld, 64);
      uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) rank = __popcll(m & lt_mask);
      if (lane == ld) {
        leader = true;
        wcnt[wave * E + le] = (uint8_t)__popcll(m);
      }
      active &= ~m;
    }
    __syncthreads();
    if (valid) {
      int pos = cursor[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
      sorted_ids[pos] = f;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&cursor[e], (int)wcnt[wave * E + e]);
      wcnt[wave * E + e] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_permute_align(const int32_t* ids, int P, int E, int block_m, int nb,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                                int32_t* npp, hipStream_t s) {
  size_t smem = (size_t)E * 8 + kPermWaves * 4 + (size_t)kPermWaves * E;
  hipLaunchKernelGGL(permute_align_kernel, dim3(1), dim3(kPermThreads), smem, s, ids, P, E, block_m, nb,
                     sorted_ids, block_expert, offsets, npp);
  return hipGetLastError();
}

}  // namespace moe
