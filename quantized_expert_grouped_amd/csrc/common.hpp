// Device helpers shared by the gfx950 kernels of libmoe_prefill.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kQK = 32;          // values per quantisation block
constexpr int kDs4Vals = 128;    // values per q8_1 group (4 blocks)
constexpr int kDs4Bytes = 144;   // 16 B of (d, s) pairs + 128 B of q
constexpr int kWave = 64;        // CDNA wavefront width

__host__ __device__ constexpr int block_bytes(int wtype) { return wtype == 1 ? 20 : 34; }

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 in the default rounding mode).
__device__ __forceinline__ uint32_t f2h(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// The q8_1 s field is fp16(d * S) with the product rounded to fp32 first.  The compiler would
// otherwise fold the multiply and the conversion into one v_fma_mixlo_f16 (a single rounding
// straight to fp16), which rounds differently in rare cases; the empty asm keeps the fp32 product.
__device__ __forceinline__ uint32_t q8_1_scale_bits(float d, int S) {
  float p = d * (float)S;
  asm volatile("" : "+v"(p));
  return f2h(p);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

}  // namespace moe
