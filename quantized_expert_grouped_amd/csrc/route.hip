// a0  Top-K routing.  "#1368 prefill: quantize each token's MoE input once and scatter it to its
// k rows", "Identity": the rows are routed as Prefill routes them, 10 of 512 experts per token.
// Each token takes the K largest logits (equal logits: the lower expert id first) and weights
// them with the softmax of those K logits.
//
// One wavefront per token: lane l holds logits l, l+64, ... in registers (coalesced loads); K
// rounds of a wave-wide (value desc, id asc) argmax pick the experts; lane k keeps pick k and the
// weights come from one wave-wide sum.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int K, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wavefront
  const float* l = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int id = j * 64 + lane;
    v[j] = id < E ? l[id] : 0.0f;
  }
  uint32_t taken = 0;
  float my_v = 0.0f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int id = j * 64 + lane;
      if (id < E && !((taken >> j) & 1u) && better(v[j], id, bv, bid)) {
        bv = v[j];
        bid = id;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oid = __shfl_xor(bid, off);
      if (better(ov, oid, bv, bid)) {
        bv = ov;
        bid = oid;
      }
    }
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
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
