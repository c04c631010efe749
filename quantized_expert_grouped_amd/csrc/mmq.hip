// a4..a6  Grouped quantised matmul (MMQ) on q8_1 activations.  "Prompt path: an MMQ group's
// experts gathered in one launch, after one wait, released by one event", "What changes": the
// products of a group's experts and their order are unchanged by how the group is gathered;
// "#1368 prefill: quantize each token's MoE input once and scatter it to its k rows", opening
// section: the down projection's input is quantised to q8_1 again.
//
// For weight row n and activation row r, block b (32 values):
//   I_b = sum_j qw_j * qx_j                      (exact int32, v_mfma_i32_32x32x32_i8: K = 32
//                                                 is exactly one block)
//   y_b = dw * dx * I_b   (+ mw * sx for Q4_1)   (fp32, fused multiply-adds, b ascending)
// Each output element is accumulated by one lane in one fixed order whatever the tiling, so
// results do not depend on group size, ring start or the row's place in its tile.
//
// Workgroup tile: 64 activation rows (one m-tile of one expert) x 128 weight rows, 4 wavefronts.
// Wavefront (wr, wc) computes rows 32*wr.. with two 32x32 MFMA tiles:
//   MOE_EPI_SWIGLU_Q8_1: gate rows f0+32wc.. and up rows F+f0+32wc.. (the same 32 features), so
//     h = silu(g) * u is formed in registers and requantised along F across the 32 lanes that
//     hold one block of 32 features;
//   otherwise: weight rows n0+64wc.. and n0+64wc+32...
// K loop: 4 blocks (128 values, one q8_1 group) per LDS stage.  Weights are unpacked while
// staging: Q8_0's 34-byte blocks are realigned with v_alignbit, Q4_1's nibbles are split into
// bytes (element j low nibble, j+16 high), so both types feed the same int8 MFMA; per-block
// scales are converted to fp32 tables in LDS.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kRowsM = kMmqRows;   // 64 activation rows per workgroup
constexpr int kRowsN = 128;        // weight rows per workgroup
constexpr int kKB = 4;             // blocks per stage
constexpr int kAStride = 144;      // LDS bytes per activation row (the raw q8_1 group)
constexpr int kBStride = 144;      // LDS bytes per weight row (4 x 32 unpacked int8 + pad)

struct Lds {
  uint8_t a[kRowsM * kAStride];
  float dx[kKB][kRowsM];
  float sx[kKB][kRowsM];
  uint8_t b[kRowsN * kBStride];
  float dw[kKB][kRowsN];
  float mw[kKB][kRowsN];
};

template <int WT>
__device__ __forceinline__ void stage_weights(Lds& L, const uint8_t* __restrict__ W,
                                              size_t row_bytes, int stage, int epi, int n0,
                                              int n_out) {
  const int tid = threadIdx.x;
  if (WT == 0) {
    // 128 rows x 2 pairs of 34-byte blocks = 256 items, 17 dwords each
    const int nb = tid >> 1, pair = tid & 1;
    const int wrow = epi == 1 ? (nb < 64 ? n0 + nb : n_out + n0 + nb - 64) : n0 + nb;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        W + (size_t)wrow * row_bytes + (size_t)stage * (kKB * 34) + pair * 68);
    uint32_t w[17];
#pragma unroll
    for (int i = 0; i < 17; ++i) w[i] = src[i];
    uint32_t q0[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q0[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], 16);
    uint8_t* dst = L.b + nb * kBStride + (2 * pair) * 32;
    *reinterpret_cast<uint4*>(dst) = make_uint4(q0[0], q0[1], q0[2], q0[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(q0[4], q0[5], q0[6], q0[7]);
    *reinterpret_cast<uint4*>(dst + 32) = make_uint4(w[9], w[10], w[11], w[12]);
    *reinterpret_cast<uint4*>(dst + 48) = make_uint4(w[13], w[14], w[15], w[16]);
    L.dw[2 * pair][nb] = h2f(w[0] & 0xffffu);
    L.dw[2 * pair + 1][nb] = h2f(w[8] >> 16);
  } else {
    // 128 rows x 4 blocks of 20 bytes = 512 items, two per thread
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + it * 256;
      const int nb = item >> 2, blk = item & 3;
      const int wrow = epi == 1 ? (nb < 64 ? n0 + nb : n_out + n0 + nb - 64) : n0 + nb;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          W + (size_t)wrow * row_bytes + (size_t)(stage * kKB + blk) * 20);
      uint32_t w[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) w[i] = src[i];
      uint8_t* dst = L.b + nb * kBStride + blk * 32;
      *reinterpret_cast<uint4*>(dst) =
          make_uint4(w[1] & 0x0f0f0f0fu, w[2] & 0x0f0f0f0fu, w[3] & 0x0f0f0f0fu,
                     w[4] & 0x0f0f0f0fu);
      *reinterpret_cast<uint4*>(dst + 16) =
          make_uint4((w[1] >> 4) & 0x0f0f0f0fu, (w[2] >> 4) & 0x0f0f0f0fu,
                     (w[3] >> 4) & 0x0f0f0f0fu, (w[4] >> 4) & 0x0f0f0f0fu);
      L.dw[blk][nb] = h2f(w[0] & 0xffffu);
      L.mw[blk][nb] = h2f(w[0] >> 16);
    }
  }
}

__device__ __forceinline__ void stage_acts(Lds& L, const uint8_t* __restrict__ act,
                                           size_t act_row_bytes, int row0, int nrows, int stage) {
  for (int c = threadIdx.x; c < kRowsM * 9; c += 256) {
    const int row = c / 9, part = c - row * 9;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < nrows)
      v = *reinterpret_cast<const uint4*>(act + (size_t)(row0 + row) * act_row_bytes +
                                          (size_t)stage * kDs4Bytes + part * 16);
    *reinterpret_cast<uint4*>(L.a + row * kAStride + part * 16) = v;
    if (part == 0) {
      const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        L.dx[b][row] = h2f(h[b] & 0xffffu);
        L.sx[b][row] = h2f(h[b] >> 16);
      }
    }
  }
}

template <int WT, int EPI>
__device__ __forceinline__ void mmq_tile(Lds& L, const MmqProblem& p, const uint8_t* W, int row0,
                                         int nrows, int ntile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int nblk = p.k_in / kQK;
  const size_t row_bytes = (size_t)nblk * block_bytes(WT);
  const size_t act_row_bytes = (size_t)(p.k_in / kDs4Vals) * kDs4Bytes;
  const int n0 = EPI == 1 ? ntile * 64 : ntile * kRowsN;
  // LDS weight rows of this wavefront's two MFMA tiles
  const int tb0 = EPI == 1 ? 32 * wc : 64 * wc;
  const int tb1 = EPI == 1 ? 64 + 32 * wc : 64 * wc + 32;

  float acc0[16], acc1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc0[i] = 0.0f;
    acc1[i] = 0.0f;
  }
  const v16i zero = {0};
  const int nstages = p.k_in / kDs4Vals;
  for (int s = 0; s < nstages; ++s) {
    __syncthreads();
    stage_acts(L, p.act, act_row_bytes, row0, nrows, s);
    stage_weights<WT>(L, W, row_bytes, s, EPI, n0, p.n_out);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kKB; ++b) {
      const v4i a = *reinterpret_cast<const v4i*>(L.a + (32 * wr + l32) * kAStride + 16 + b * 32 +
                                                  half * 16);
      const v4i b0 = *reinterpret_cast<const v4i*>(L.b + (tb0 + l32) * kBStride + b * 32 +
                                                   half * 16);
      const v4i b1 = *reinterpret_cast<const v4i*>(L.b + (tb1 + l32) * kBStride + b * 32 +
                                                   half * 16);
      const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, zero, 0, 0, 0);
      const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, zero, 0, 0, 0);
      if (EPI == 2) {
        int32_t* out = reinterpret_cast<int32_t*>(p.out);
        const int kb = s * kKB + b;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 32 * wr + 8 * (i >> 2) + 4 * half + (i & 3);
          if (row < nrows) {
            const size_t r = (size_t)(row0 + row);
            out[(r * p.n_out + n0 + tb0 + l32) * nblk + kb] = I0[i];
            out[(r * p.n_out + n0 + tb1 + l32) * nblk + kb] = I1[i];
          }
        }
        continue;
      }
      const float dw0 = L.dw[b][tb0 + l32];
      const float dw1 = L.dw[b][tb1 + l32];
      float dx[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 d4 = *reinterpret_cast<const float4*>(&L.dx[b][32 * wr + 8 * j + 4 * half]);
        dx[4 * j + 0] = d4.x;
        dx[4 * j + 1] = d4.y;
        dx[4 * j + 2] = d4.z;
        dx[4 * j + 3] = d4.w;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc0[i] = fmaf((float)I0[i], dx[i] * dw0, acc0[i]);
        acc1[i] = fmaf((float)I1[i], dx[i] * dw1, acc1[i]);
      }
      if (WT == 1) {
        const float mw0 = L.mw[b][tb0 + l32];
        const float mw1 = L.mw[b][tb1 + l32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 s4 =
              *reinterpret_cast<const float4*>(&L.sx[b][32 * wr + 8 * j + 4 * half]);
          const float sx[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc0[4 * j + q] = fmaf(mw0, sx[q], acc0[4 * j + q]);
            acc1[4 * j + q] = fmaf(mw1, sx[q], acc1[4 * j + q]);
          }
        }
      }
    }
  }
  if (EPI == 2) return;

  if (EPI == 0) {
    float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * wr + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < nrows) {
        float* o = out + (size_t)(row0 + row) * p.n_out + n0;
        o[tb0 + l32] = acc0[i];
        o[tb1 + l32] = acc1[i];
      }
    }
    return;
  }

  // EPI == 1: h = silu(g) * u, then q8_1 along F: the 32 lanes of a half hold one block
  const int f = n0 + 32 * wc + l32;
  const int fb = (n0 + 32 * wc) / kQK;  // block index along F
  const size_t h_row_bytes = (size_t)(p.n_out / kDs4Vals) * kDs4Bytes;
  const size_t hoff = (size_t)(fb >> 2) * kDs4Bytes;
  const size_t qoff = hoff + 16 + (fb & 3) * 32 + l32;
  uint8_t* hq = reinterpret_cast<uint8_t*>(p.out);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 32 * wr + 8 * (i >> 2) + 4 * half + (i & 3);
    const float g = acc0[i], u = acc1[i];
    const float h = g / (1.0f + expf(-g)) * u;
    float am = fabsf(h);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    const bool nz = am > 0.0f;
    const float d = am / 127.0f;
    const int q = nz ? (int)roundf(h / d) : 0;
    int S = q;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) S += __shfl_xor(S, off);
    if (row < nrows) {
      const size_t r = (size_t)(row0 + row);
      uint8_t* dst = hq + r * h_row_bytes;
      dst[qoff] = (uint8_t)(q & 0xff);
      if (l32 == 0) {
        const uint32_t hdr = nz ? (f2h(d) | (q8_1_scale_bits(d, S) << 16)) : 0u;
        *reinterpret_cast<uint32_t*>(dst + hoff + (fb & 3) * 4) = hdr;
      }
      if (p.debug_h != nullptr) p.debug_h[r * p.n_out + f] = h;
    }
  }
}

template <int WT, int EPI>
__global__ __launch_bounds__(256) void mmq_layer_kernel(MmqProblem p) {
  __shared__ Lds L;
  const int mt = blockIdx.y;
  if (mt >= *p.n_tiles) return;
  const MTile t = p.tiles[mt];
  const uint8_t* W = p.wbase + (size_t)t.ordinal * p.pos_stride + p.mat_offset;
  mmq_tile<WT, EPI>(L, p, W, t.row0, t.nrows, blockIdx.x);
}

template <int WT, int EPI>
__global__ __launch_bounds__(256) void mmq_group_kernel(MmqProblem p) {
  __shared__ Lds L;
  const int j = blockIdx.z;
  const int e = p.experts[j];
  const int r0 = p.offsets[e], cnt = p.offsets[e + 1] - r0;
  const uint8_t* W = p.wbase + (size_t)j * p.pos_stride + p.mat_offset;
  for (int m = blockIdx.y; m * kRowsM < cnt; m += gridDim.y)
    mmq_tile<WT, EPI>(L, p, W, r0 + m * kRowsM, min(kRowsM, cnt - m * kRowsM), blockIdx.x);
}

template <int WT, int EPI>
hipError_t launch_typed(const MmqProblem& p, hipStream_t s) {
  const int ntiles = EPI == 1 ? p.n_out / 64 : p.n_out / kRowsN;
  if (p.tiles != nullptr) {
    const dim3 grid(ntiles, p.max_tiles);
    mmq_layer_kernel<WT, EPI><<<grid, 256, 0, s>>>(p);
  } else {
    const dim3 grid(ntiles, 16, p.n_group);
    mmq_group_kernel<WT, EPI><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq(const MmqProblem& p, hipStream_t s) {
  if (p.wtype == 0) {
    if (p.epilogue == 0) return launch_typed<0, 0>(p, s);
    if (p.epilogue == 1) return launch_typed<0, 1>(p, s);
    return launch_typed<0, 2>(p, s);
  }
  if (p.epilogue == 0) return launch_typed<1, 0>(p, s);
  if (p.epilogue == 1) return launch_typed<1, 1>(p, s);
  return launch_typed<1, 2>(p, s);
}

}  // namespace moe
