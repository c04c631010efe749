// a7  Combine.  "#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's least-routed
// experts to the idle CPU pool", "What it does": the expert output rows in Dm are unweighted and
// the combine weights them like any other row.  out[t,i] = sum_{k<K} w[t,k] * Dm[slot[t*K+k], i],
// k ascending (fp32 fused multiply-adds in that fixed order, so the result depends only on the
// token's own rows).
//
// One workgroup per token; each thread owns float4 columns of the row, reads the K routed rows
// with 16-byte loads, up to 8 rows' loads in flight before their fused multiply-adds, and
// writes the output once.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBatchK = 8;  // routed rows whose loads are in flight together

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Dm,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ w, int K, int H,
                                                      float* __restrict__ out) {
  __shared__ int32_t s_row[64];
  __shared__ float s_w[64];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    s_row[threadIdx.x] = slot[(size_t)t * K + threadIdx.x];
    s_w[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  const int n4 = H / 4;
  for (int c = threadIdx.x; c < n4; c += 256) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += kBatchK) {
      // the loads of up to kBatchK rows first (each row is read once: non-temporal), then the
      // fused multiply-adds in k order
      v4f d[kBatchK];
#pragma unroll
      for (int j = 0; j < kBatchK; ++j)
        if (k0 + j < K)
          d[j] = __builtin_nontemporal_load(
              reinterpret_cast<const v4f*>(Dm + (size_t)s_row[k0 + j] * H) + c);
#pragma unroll
      for (int j = 0; j < kBatchK; ++j) {
        if (k0 + j < K) {
          const float wk = s_w[k0 + j];
          acc.x = fmaf(wk, d[j].x, acc.x);
          acc.y = fmaf(wk, d[j].y, acc.y);
          acc.z = fmaf(wk, d[j].z, acc.z);
          acc.w = fmaf(wk, d[j].w, acc.w);
        }
      }
    }
    __builtin_nontemporal_store(acc, reinterpret_cast<v4f*>(out + (size_t)t * H) + c);
  }
}

}  // namespace

hipError_t launch_combine(const float* Dm, const int32_t* slot, const float* w, int T, int K,
                          int H, float* out, hipStream_t s) {
  combine_kernel<<<T, 256, 0, s>>>(Dm, slot, w, K, H, out);
  return hipGetLastError();
}

}  // namespace moe
