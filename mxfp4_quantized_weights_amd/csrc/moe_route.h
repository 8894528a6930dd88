// Top-k routing of one token by one wave (device code only; the routing
// kernels and the decode kernels that route their own tokens share it).
//
// FreeToken PR #270 "glm5_next: support GLM-5.3-Flash (hybrid KDA + DSA,
// mHC, NVFP4 expert offload)", Summary (288-expert top-8 routing; the fused
// router epilogue picks the same ids as a reference top-k).  Selection is on
// the raw logits, descending, ties to the lower expert id; weights are the
// softmax over the k selected logits.
#pragma once

#include <math.h>

#include "moe_device.h"

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

// A token's logits in a wave: lane holds experts lane + 64*i (NaN as -inf);
// bit i of avail marks those that exist (e < E).
template <int VPL>
__device__ __forceinline__ void route_load(const float* __restrict__ row, int E, float (&v)[VPL], uint32_t& avail) {
  const int lane = threadIdx.x & 63;
  avail = 0;
  // every load is issued (index clamped into the row, masked after), so the
  // VPL loads are in flight together
  float raw[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) raw[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    const float x = (e < E) ? raw[i] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
    if (e < E) avail |= 1u << i;
  }
}

// Top-k of one token by one wave from its loaded logits: k rounds of a
// wave-wide argmax pick the experts in slot order.  The softmax denominator
// is summed in slot order.  Lane j < k writes slot j to ids[j], w[j] and, if
// given, ids2[j].
template <int VPL>
__device__ __forceinline__ void route_select(const float (&v)[VPL], uint32_t avail, int k, int32_t* ids, float* w,
                                             int32_t* ids2) {
  const int lane = threadIdx.x & 63;
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
    ids[lane] = my_e;
    w[lane] = ex / sum;
    if (ids2) ids2[lane] = my_e;
  }
}

// Top-k of one token by one wave (route_load, then route_select).
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int32_t* ids, float* w,
                                            int32_t* ids2) {
  float v[VPL];
  uint32_t avail;
  route_load<VPL>(row, E, v, avail);
  route_select<VPL>(v, avail, k, ids, w, ids2);
}

}  // namespace moe
