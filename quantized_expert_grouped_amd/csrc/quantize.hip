// a2  q8_1 quantisation of the layer input.  "#1368 prefill: quantize each token's MoE input once
// and scatter it to its k rows (the same bytes)", opening section: the per-row form quantises
// the T*K rows in expert order and so reads each token's input K times; the scatter form
// quantises each token once and writes the same block to every row slot[t*K+k].
//
// Block arithmetic (identical in both forms): amax = max|v|; d = amax/127 (IEEE division);
// q = roundf(v/d) (the IEEE quotient, ties away from zero: taken through a reciprocal, with the
// division itself only near half-integers, which gives the same q); S = sum q; stored
// d16 = fp16(d), s16 = fp16(d * S); an all-zero block stores zeros.  Row layout (DS4): 144 B per
// 128 values = 4 x (d16, s16) then 4 x 32 q.  The D4 layout, which the page names for Q8_0, keeps
// the 4 blocks' fp32 d in the same 16 header bytes instead (the same q, no s).
//
// A route whose expert id was out of range has slot = -1 (and its row src = -1, see the maps):
// nothing is written for it.
//
// One wavefront per token (scatter) or per row (per-row form).  A lane owns 16 consecutive
// values (four coalesced float4 loads), so a block of 32 is a lane pair: one xor-shuffle for
// amax and one for S.  The chunk's 1152 output bytes (8 groups of 144) are then permuted across
// the lanes so that each destination row takes two stores of consecutive 16-byte pieces, and
// every 128-byte line is written whole by one instruction.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

template <int MODE, int D4>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ x, int T, int H,
                                                       int K, const int32_t* __restrict__ slot,
                                                       const int32_t* __restrict__ src,
                                                       uint8_t* __restrict__ q8) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nunits = MODE == 0 ? T : T * K;
  if (unit >= nunits) return;  // uniform per wavefront
  // a row whose route named no real expert has src = -1 (and its entry slot = -1): no bytes
  const int sr = MODE == 0 ? 0 : src[unit];
  if (sr < 0) return;
  const int t = MODE == 0 ? unit : sr / K;
  const float* xr = x + (size_t)t * H;
  const size_t rb = (size_t)(H / kDs4Vals) * kDs4Bytes;
  int my_row = unit;
  if (MODE == 0) my_row = lane < K ? slot[(size_t)t * K + lane] : 0;
  const int nrows = MODE == 0 ? K : 1;

  // The row is taken in chunks of 1024 values (16 per lane), two chunks' loads in flight at a
  // time so that the second chunk's latency overlaps the first's quantisation and stores.
  auto load = [&](int c0, float (&v)[16]) {
    const int v0 = c0 + lane * 16;
    if (v0 < H) {  // H is a multiple of 128: whole 8-lane groups
      const float4* p = reinterpret_cast<const float4*>(xr + v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = p[i];
        v[4 * i + 0] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
  };
  auto quantize_chunk = [&](int c0, const float (&v)[16]) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    am = fmaxf(am, __shfl_xor(am, 1));
    const bool nz = am > 0.0f;
    const float d = am / 127.0f;
    uint32_t qw[4];
    int S = q8_pack16(v, d, nz, qw);
    S += __shfl_xor(S, 1);
    const uint32_t hdr =
        !nz ? 0u : D4 ? __float_as_uint(d) : (f2h(d) | (q8_1_scale_bits(d, S) << 16));
    const uint32_t h1 = __shfl_down(hdr, 2);
    const uint32_t h2 = __shfl_down(hdr, 4);
    const uint32_t h3 = __shfl_down(hdr, 6);
    // The chunk's 8 groups are 72 consecutive 16-byte pieces of a row (a group: its header
    // piece, then its 8 q pieces).  Lane l holds q piece l % 8 of group l / 8 and lanes 8g the
    // headers; piece i goes out from lane i (i < 64), pieces 64..71 from lanes 0..7, so every
    // 128-byte line of the row is written whole by one store instruction.
    const int g0 = c0 / kDs4Vals;                       // the chunk's first group in the row
    const int pg = lane / 9, pp = lane % 9;             // piece `lane`: group, part
    const int src = 8 * pg + (pp == 0 ? 0 : pp - 1);
    const uint32_t hx0 = __shfl(hdr, src), hx1 = __shfl(h1, src), hx2 = __shfl(h2, src),
                   hx3 = __shfl(h3, src);
    const uint32_t qx0 = __shfl(qw[0], src), qx1 = __shfl(qw[1], src), qx2 = __shfl(qw[2], src),
                   qx3 = __shfl(qw[3], src);
    const uint4 p0 = pp == 0 ? make_uint4(hx0, hx1, hx2, hx3) : make_uint4(qx0, qx1, qx2, qx3);
    const uint4 p1 = make_uint4(__shfl(qw[0], 56 + (lane & 7)), __shfl(qw[1], 56 + (lane & 7)),
                                __shfl(qw[2], 56 + (lane & 7)), __shfl(qw[3], 56 + (lane & 7)));
    const int ngroups = min(8, (H - c0) / kDs4Vals);    // whole groups in this chunk
    const int npieces = 9 * ngroups;
    for (int k = 0; k < nrows; ++k) {
      const int r = MODE == 0 ? __shfl(my_row, k) : my_row;
      if (r < 0) continue;  // uniform: a route to no real expert
      uint8_t* seg = q8 + (size_t)r * rb + (size_t)g0 * kDs4Bytes;
      if (lane < npieces) *reinterpret_cast<uint4*>(seg + 16 * lane) = p0;
      if (lane < 8 && 64 + lane < npieces) *reinterpret_cast<uint4*>(seg + 16 * (64 + lane)) = p1;
    }
  };
  for (int c0 = 0; c0 < H; c0 += 2 * 64 * 16) {
    float va[16], vb[16];
    load(c0, va);
    const bool second = c0 + 64 * 16 < H;
    if (second) load(c0 + 64 * 16, vb);
    quantize_chunk(c0, va);
    if (second) quantize_chunk(c0 + 64 * 16, vb);
  }
}

}  // namespace

hipError_t launch_quantize(const float* x, int T, int H, int K, const int32_t* slot,
                           const int32_t* src, int mode, uint8_t* q8, hipStream_t s) {
  const bool gather = (mode & kQuantPerRow) != 0, d4 = (mode & kQuantD4) != 0;
  const int nunits = gather ? T * K : T;
  const dim3 grid((nunits + 3) / 4), block(256);
  if (!gather && !d4)
    quantize_kernel<0, 0><<<grid, block, 0, s>>>(x, T, H, K, slot, src, q8);
  else if (!gather)
    quantize_kernel<0, 1><<<grid, block, 0, s>>>(x, T, H, K, slot, src, q8);
  else if (!d4)
    quantize_kernel<1, 0><<<grid, block, 0, s>>>(x, T, H, K, slot, src, q8);
  else
    quantize_kernel<1, 1><<<grid, block, 0, s>>>(x, T, H, K, slot, src, q8);
  return hipGetLastError();
}

}  // namespace moe
