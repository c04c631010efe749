// a0  Top-K routing.  "#1368 prefill: quantize each token's MoE input once and scatter it to its
// k rows", "Identity": the rows are routed as Prefill routes them, 10 of 512 experts per token.
// Each token takes the K largest logits (equal logits: the lower expert id first) and weights
// them with the softmax of those K logits.
//
// One wavefront per token: lane l holds logits l, l+64, ... in registers (coalesced loads); K
// rounds of a wave-wide (value desc, id asc) argmax pick the experts (a branch-free lane-local
// pass, DPP steps inside each row of 16 lanes, then the 4 rows' winners read into scalars: no LDS
// round trip on the chain); the pick is set to -inf in its lane; lane k keeps pick k and the
// weights come from one wave-wide sum.  (value desc, id asc) is a strict
// order on distinct ids, so the winner does not depend on the order of the comparisons.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One step of the wave-wide argmax: each lane takes the better of its (v, id) and that of the lane
// the DPP pattern CTRL names (a permutation inside each row of 16 lanes).
template <int CTRL>
__device__ __forceinline__ void dpp_best(float& v, int& id) {
  const float ov =
      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oid = __builtin_amdgcn_update_dpp(0, id, CTRL, 0xF, 0xF, false);
  if (better(ov, oid, v, id)) {
    v = ov;
    id = oid;
  }
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each row

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int K, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wavefront
  const float* l = logits + (size_t)t * E;
  // lane l holds logits l, l+64, ...; ids past E and picked entries read -inf (the logits are
  // finite, so such an entry never wins while K <= E)
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int id = j * 64 + lane;
    v[j] = id < E ? l[id] : -INFINITY;
  }
  float my_v = 0.0f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    // the lane's best: its ids grow with j, so only a strictly larger value displaces the best
    // so far (equal values keep the lower id), with no branch per entry
    float bv = v[0];
    int bj = 0;
#pragma unroll
    for (int j = 1; j < VPL; ++j) {
      const bool gt = v[j] > bv;
      bv = gt ? v[j] : bv;
      bj = gt ? j : bj;
    }
    int bid = bj * 64 + lane;
    // best within each row of 16 lanes (every lane of the row ends with it), then of the 4 rows
    dpp_best<kDppXor1>(bv, bid);
    dpp_best<kDppXor2>(bv, bid);
    dpp_best<kDppHalfMirror>(bv, bid);
    dpp_best<kDppMirror>(bv, bid);
    {
      float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
      int rid = __builtin_amdgcn_readlane(bid, 0);
#pragma unroll
      for (int r = 1; r < 4; ++r) {
        const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
        const int oid = __builtin_amdgcn_readlane(bid, 16 * r);
        if (better(ov, oid, rv, rid)) {
          rv = ov;
          rid = oid;
        }
      }
      bv = rv;
      bid = rid;
    }
    // the pick leaves its lane's candidates (pj, pl uniform)
    const int pj = bid >> 6, pl = bid & 63;
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] = (j == pj && lane == pl) ? -INFINITY : v[j];
    if (lane == k) {
      my_v = bv;
      my_id = bid;
    }
  }
  const float lmax = __shfl(my_v, 0);
  const float ex = lane < K ? expf(my_v - lmax) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < K) {
    idx[(size_t)t * K + lane] = my_id;
    w[(size_t)t * K + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                             hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, K, idx, w);
  else if (vpl <= 2)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, K, idx, w);
  else if (vpl <= 4)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, K, idx, w);
  else if (vpl <= 8)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, K, idx, w);
  else if (vpl <= 16)
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, K, idx, w);
  else
    route_topk_kernel<32><<<grid, block, 0, s>>>(logits, T, E, K, idx, w);
  return hipGetLastError();
}

}  // namespace moe
