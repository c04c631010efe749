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

// The q8_1 bytes of a lane's 16 values of one block: q[k] = roundf(v[k] / d) (the IEEE quotient
// rounded half away from zero), bit for bit, packed four to a word (value 4i + j in byte j of
// word i), and their sum S; an all-zero block (`nz` false, amax = 0) gives q = 0.  No division
// per value: the block scale is d = amax / 127, so |v / d| <= 127.00001, and y = v * rcp(d) is
// taken exactly inside two fma.  y + 1.5 * 2^23, rounded once, is rint(y) + 1.5 * 2^23 (|y| <
// 2^22), whose low mantissa bits hold the integer in two's complement: its low byte is the q
// byte, and the words' sum less 16 * 0x4B400000 is S.  y - rint(y) comes from the second fma.
// With rcp within 1 ulp, |y - v / d| <= |v / d| * 2^-23, and the correctly rounded quotient lies
// within half its ulp (2^-18) of v / d: under 1.9e-5 in all (3.4e-5 were rcp off by 2 ulp).  So
// wherever y is more than 2^-14 away from every half-integer, the quotient lies strictly between
// the same two half-integers as y and both round to rint(y).  Values within 2^-14 of a
// half-integer (about one in 8,000), NaN, and a d outside rcp's exact range (a subnormal d) send
// the wavefront through the IEEE division for all its values (NaN values, which amax skips,
// then give what the division gives; with `nz` false the multiplier is 0).  The low bytes are
// gathered by v_perm, two per instruction.
__device__ __forceinline__ int q8_pack16(const float (&v)[16], float d, bool nz,
                                         uint32_t (&qw)[4]) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23, bits 0x4B400000
  const float r = nz ? __builtin_amdgcn_rcpf(d) : 0.0f;
  bool near = nz && !(d >= 0x1p-125f);
  int bits[16];
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float nm = fmaf(v[k], r, kMagic);
    const float n = nm - kMagic;  // exact
    near |= !(fabsf(fmaf(v[k], r, -n)) < 0.5f - 0x1p-14f);  // NaN compares false
    bits[k] = __float_as_int(nm);
    sum += (uint32_t)bits[k];
  }
  int S = (int)(sum - 16u * 0x4B400000u);  // modulo 2^32: the sum of the q
  if (__builtin_expect(ballot(near) != 0, 0)) {
    S = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      bits[k] = nz ? (int)roundf(v[k] / d) : 0;
      S += bits[k];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // bytes 0, 1 from values 4i, 4i + 1; 2, 3 from 4i + 2, 4i + 3
    const uint32_t b0 = (uint32_t)bits[4 * i], b1 = (uint32_t)bits[4 * i + 1];
    const uint32_t b2 = (uint32_t)bits[4 * i + 2], b3 = (uint32_t)bits[4 * i + 3];
    qw[i] = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
  }
  return S;
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
