// a3  The group gather.  "#439 prefill: a group's expert gathers in one launch", "What": one
// launch copies up to 16 experts into the MMQ group buffer (blockIdx.y = expert), and the same
// bytes land in the same places as with one copy per expert; its test covers batches of 1-16,
// positions starting mid-group and the unaligned / odd-size fallback.  "Prompt path: an MMQ
// group's experts gathered in one launch, after one wait, released by one event", "What
// changes": the same, one launch per group.
//
// gfx950 form: grid-stride 16-byte copies (global_load_dwordx4 / global_store_dwordx4), four
// loads in flight per lane before the stores, each load instruction covering 1 KiB of
// contiguous bytes across the wavefront.  A copy whose source, destination or size is not a
// multiple of 16 bytes takes a byte-wise loop instead (the decision is uniform per expert).
// The layer form walks every group of the layer in one launch (blockIdx.z = group): on a GPU
// with 288 GB of HBM every routed expert of a layer has its own group position, so there is no
// ring slot to wait for or give back between groups.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

__device__ __forceinline__ void copy_span(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst, size_t bytes, int part,
                                          int nparts) {
  const int tid = threadIdx.x;
  if ((((uintptr_t)src | (uintptr_t)dst | bytes) & 15) == 0) {
    const v4u* s4 = reinterpret_cast<const v4u*>(src);
    v4u* d4 = reinterpret_cast<v4u*>(dst);
    const size_t n16 = bytes >> 4;
    const size_t step = (size_t)nparts * kGatherThreads * kGatherUnroll;
    for (size_t base = (size_t)part * kGatherThreads * kGatherUnroll + tid; base < n16;
         base += step) {
      v4u v[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const size_t i = base + (size_t)u * kGatherThreads;
        if (i < n16) v[u] = __builtin_nontemporal_load(s4 + i);
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const size_t i = base + (size_t)u * kGatherThreads;
        if (i < n16) d4[i] = v[u];
      }
    }
  } else {
    const size_t step = (size_t)nparts * kGatherThreads;
    for (size_t i = (size_t)part * kGatherThreads + tid; i < bytes; i += step) dst[i] = src[i];
  }
}

__global__ __launch_bounds__(kGatherThreads) void gather_group_kernel(GatherPtrs p, size_t bytes,
                                                                      uint8_t* __restrict__ dst,
                                                                      int first_pos,
                                                                      size_t pos_stride) {
  const int j = blockIdx.y;
  copy_span(p.src[j], dst + (size_t)(first_pos + j) * pos_stride, bytes, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(kGatherThreads) void gather_all_kernel(
    const uint8_t* __restrict__ pool, const int64_t* __restrict__ expert_off,
    const int32_t* __restrict__ order, const int32_t* __restrict__ n_active, size_t bytes,
    uint8_t* __restrict__ dst, size_t stride) {
  const int pos = blockIdx.z * gridDim.y + blockIdx.y;  // group * group_size + position in group
  if (pos >= *n_active) return;
  copy_span(pool + expert_off[order[pos]], dst + (size_t)pos * stride, bytes, blockIdx.x,
            gridDim.x);
}

int parts_for(size_t bytes) {
  // about 4 grid-stride trips of 16 KiB per workgroup
  const size_t per = (size_t)kGatherThreads * kGatherUnroll * 16 * 4;
  size_t n = (bytes + per - 1) / per;
  if (n < 1) n = 1;
  if (n > 1024) n = 1024;
  return (int)n;
}

}  // namespace

hipError_t launch_gather_group(const GatherPtrs& p, int n, size_t bytes, uint8_t* dst,
                               int first_pos, size_t pos_stride, hipStream_t s) {
  const dim3 grid(parts_for(bytes), n);
  gather_group_kernel<<<grid, kGatherThreads, 0, s>>>(p, bytes, dst, first_pos, pos_stride);
  return hipGetLastError();
}

hipError_t launch_gather_all(const uint8_t* pool, const int64_t* expert_off, const int32_t* order,
                             const int32_t* n_active, int max_slots, int group_size, size_t bytes,
                             uint8_t* dst, size_t stride, hipStream_t s) {
  // blockIdx.z = group, blockIdx.y = expert within the group, as in one group's launch
  const int groups = (max_slots + group_size - 1) / group_size;
  const dim3 grid(parts_for(bytes), group_size, groups);
  gather_all_kernel<<<grid, kGatherThreads, 0, s>>>(pool, expert_off, order, n_active, bytes,
                                                    dst, stride);
  return hipGetLastError();
}

}  // namespace moe
