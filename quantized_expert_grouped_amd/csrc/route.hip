// a0  Top-K routing.  "#1368 prefill: quantize each token's MoE input once and scatter it to its
// k rows", "Identity": the rows are routed as Prefill routes them, 10 of 512 experts per token.
// Each token takes the K largest logits (equal logits: the lower expert id first) and weights
// them with the softmax of those K logits.
//
// One wavefront per token: lane l holds logits l, l+64, ... in registers (coalesced loads) as
// order-preserving unsigned keys (the float's bits with the sign bit flipped for +0 and positive
// values, all bits flipped for negative ones; -0 is first made +0, so equal floats give equal
// keys).  K rounds of: each lane's best key (a branch-free pass where only a strictly larger key
// wins, so equal keys keep the lower id), the wavefront's largest key (DPP max steps inside each
// row of 16 lanes, then the 4 rows' results read into scalars), and a ballot of the lanes holding
// it: one lane is the winner; several (equal logits in several lanes) take the lowest id among
// them with one more reduction.  The pick's key becomes 0, below every finite logit's; lane k
// keeps pick k and the weights come from one wave-wide sum.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each row

// An order-preserving unsigned key of a finite float (and its inverse): larger float, larger key.
__device__ __forceinline__ uint32_t key_of(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);  // -0 becomes +0 (round to nearest)
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float float_of(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// The largest of the wavefront's 64 values: DPP steps leave each row of 16 lanes with its row's
// largest (pairs, quads, half rows, rows), then the 4 rows' values are read into scalars.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme(uint32_t v) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false));
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, false));
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xF, 0xF, false));
  uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row)
    r = pick(r, (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * row));
  return r;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int K, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wavefront
  const float* l = logits + (size_t)t * E;
  // lane l holds the keys of logits l, l+64, ...; ids past E and picked entries hold key 0,
  // below every finite logit's (the logits are finite, so such an entry never wins while K <= E)
  uint32_t key[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int id = j * 64 + lane;
    key[j] = id < E ? key_of(l[id]) : 0u;
  }
  uint32_t my_key = 0;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    // the lane's best: its ids grow with j, so only a strictly larger key displaces the best so
    // far (equal keys keep the lower id), with no branch per entry
    uint32_t bk = key[0];
    int bj = 0;
#pragma unroll
    for (int j = 1; j < VPL; ++j) {
      const bool gt = key[j] > bk;
      bk = gt ? key[j] : bk;
      bj = gt ? j : bj;
    }
    const uint32_t top = wave_extreme<true>(bk);
    const uint64_t at = ballot(bk == top);  // the lanes holding the largest key
    int bid;
    if (__popcll(at) == 1) {  // uniform: the usual case
      const int wl = (int)__builtin_ctzll(at);
      bid = __builtin_amdgcn_readlane(bj, wl) * 64 + wl;
    } else {  // equal logits in several lanes: the lowest id among them
      bid = (int)wave_extreme<false>(bk == top ? (uint32_t)(bj * 64 + lane) : 0xffffffffu);
    }
    // the pick leaves its lane's candidates (pj, pl uniform)
    const int pj = bid >> 6, pl = bid & 63;
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = (j == pj && lane == pl) ? 0u : key[j];
    if (lane == k) {
      my_key = top;
      my_id = bid;
    }
  }
  const float my_v = float_of(my_key);
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
