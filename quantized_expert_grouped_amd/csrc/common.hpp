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

// q[k] = roundf(v[k] / d) (the IEEE quotient rounded half away from zero) for a lane's 16 values
// of one q8_1 block, bit for bit, with one multiply per value in place of a division.  The block
// scale is d = amax / 127, so |v / d| <= 127.00001.  y = v * rcp(d), with rcp within 1 ulp, lies
// within |v / d| * (2^-23 + 2^-24) of v / d, and the correctly rounded quotient within half its
// ulp (2^-18): together under 2.7e-5, or 4.3e-5 were rcp off by 2 ulp.  So wherever y is more
// than 2^-14 away from every half-integer, the quotient lies strictly between the same two
// half-integers as y and both round to the nearest integer of y, rint(y).  Values within 2^-14
// of a half-integer (about one in 8,000), NaN, and a d outside rcp's exact range (a subnormal
// d) send the wavefront through the IEEE division for all its values.  `nz` false (an all-zero
// block, amax = 0) gives q = 0: there the multiplier is 0, so y = 0 (NaN values, which amax
// skips, also take the division, which then gives 0).
__device__ __forceinline__ void q8_round16(const float (&v)[16], float d, bool nz, int (&q)[16]) {
  const float r = nz ? __builtin_amdgcn_rcpf(d) : 0.0f;
  bool near = nz && !(d >= 0x1p-125f);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float y = v[k] * r;
    const float n = __builtin_rintf(y);
    near |= !(fabsf(y - n) < 0.5f - 0x1p-14f);  // y - n is exact; NaN compares false
    q[k] = (int)n;
  }
  if (__builtin_expect(ballot(near) != 0, 0)) {
#pragma unroll
    for (int k = 0; k < 16; ++k) q[k] = nz ? (int)roundf(v[k] / d) : 0;
  }
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

}  // namespace moe
