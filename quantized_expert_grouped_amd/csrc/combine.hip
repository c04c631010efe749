// a7  Combine.  "#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's least-routed
// experts to the idle CPU pool", "What it does": the expert output rows in Dm are unweighted and
// the combine applies the routing weights to them.
//   out[t,i] = sum_{k<K} w[t,k] * Dm[slot[t*K+k], i],
// k ascending (fp32 fused multiply-adds in that fixed order, so the result depends only on the
// token's own rows).
//
// A route with slot = -1 (its expert id was out of range, see the maps) adds nothing.
//
// One workgroup per token; each thread owns float4 columns of the row (two at a time), reads the
// K routed rows with 16-byte loads, up to 16 rows' loads per column in flight before their fused
// multiply-adds, and writes the output once.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBatchK = 16;  // routed rows whose loads are in flight together

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
  // two float4 columns per thread at a time (c and c + 256), so up to 2 * kBatchK loads are in
  // flight before the first is used
  for (int c = threadIdx.x; c < n4; c += 512) {
    const bool two = c + 256 < n4;
    v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += kBatchK) {
      // the loads of up to kBatchK rows first (each row is read once: non-temporal), then the
      // fused multiply-adds in k order
      v4f d0[kBatchK], d1[kBatchK];
#pragma unroll
      for (int j = 0; j < kBatchK; ++j) {
        if (k0 + j < K && s_row[k0 + j] >= 0) {
          const v4f* row = reinterpret_cast<const v4f*>(Dm + (size_t)s_row[k0 + j] * H);
          d0[j] = __builtin_nontemporal_load(row + c);
          if (two) d1[j] = __builtin_nontemporal_load(row + c + 256);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatchK; ++j) {
        if (k0 + j < K && s_row[k0 + j] >= 0) {
          const float wk = s_w[k0 + j];
          acc0.x = fmaf(wk, d0[j].x, acc0.x);
          acc0.y = fmaf(wk, d0[j].y, acc0.y);
          acc0.z = fmaf(wk, d0[j].z, acc0.z);
          acc0.w = fmaf(wk, d0[j].w, acc0.w);
          if (two) {
            acc1.x = fmaf(wk, d1[j].x, acc1.x);
            acc1.y = fmaf(wk, d1[j].y, acc1.y);
            acc1.z = fmaf(wk, d1[j].z, acc1.z);
            acc1.w = fmaf(wk, d1[j].w, acc1.w);
          }
        }
      }
    }
    v4f* o = reinterpret_cast<v4f*>(out + (size_t)t * H);
    __builtin_nontemporal_store(acc0, o + c);
    if (two) __builtin_nontemporal_store(acc1, o + c + 256);
  }
}

// One workgroup per staged row: 16-byte copies of the row into its place in Dm.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float* __restrict__ rows,
                                                          const int32_t* __restrict__ dst, int H,
                                                          float* __restrict__ Dm) {
  const int j = blockIdx.x;
  const v4f* src = reinterpret_cast<const v4f*>(rows + (size_t)j * H);
  v4f* d = reinterpret_cast<v4f*>(Dm + (size_t)dst[j] * H);
  for (int c = threadIdx.x; c < H / 4; c += 256) d[c] = src[c];
}

}  // namespace

hipError_t launch_scatter_rows(const float* rows, const int32_t* dst, int n, int H, float* Dm,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  scatter_rows_kernel<<<n, 256, 0, s>>>(rows, dst, H, Dm);
  return hipGetLastError();
}

hipError_t launch_combine(const float* Dm, const int32_t* slot, const float* w, int T, int K,
                          int H, float* out, hipStream_t s) {
  combine_kernel<<<T, 256, 0, s>>>(Dm, slot, w, K, H, out);
  return hipGetLastError();
}

}  // namespace moe
