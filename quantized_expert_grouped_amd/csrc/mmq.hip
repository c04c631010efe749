// a4..a6  Grouped quantised matmul (MMQ) on q8_1 activations.  "Prompt path: an MMQ group's
// experts gathered in one launch, after one wait, released by one event", "What changes": the
// products of a group's experts and their order are unchanged by how the group is gathered;
// "#1368 prefill: quantize each token's MoE input once and scatter it to its k rows", opening
// section: the down projection's input is quantised to q8_1 again.
//
// For weight row n and activation row r, block b (32 values):
//   I_b = sum_j qw_j * qx_j                 exact int32: one v_mfma_i32_32x32x32_i8 per block
//                                           (K = 32 is exactly one block)
//   S_b = dx_b * dw_b                       exact in fp32 (two fp16 significands): for a whole
//                                           32x32 tile this is an outer product, one
//                                           v_mfma_f32_32x32x16_f16 with a single nonzero k
//   acc = fma(float(I_b), S_b, acc)         the only per-element VALU work (convert + fma)
//   Q4_1 adds sum_b mw_b * sx_b             a true sum over blocks: an f16 MFMA whose C input
//                                           is the accumulator itself
// Blocks are taken in ascending order and every output element is accumulated by one lane in
// one fixed instruction sequence, so results do not depend on the tiling, the group size, the
// ring start or the row's place in its tile.
//
// Workgroup: 64 activation rows (one m-tile of one expert) x 128 weight rows, 4 wavefronts.
// Wavefront (wr, wc) owns rows 32*wr.. and two 32-row column tiles of the weights:
//   MOE_EPI_SWIGLU_Q8_1: gate features f0+32wc.. and the up rows of the same features, so
//     h = silu(g) * u is formed in registers and requantised along F across the 32 lanes that
//     hold one block of 32 features;
//   otherwise: weight rows n0+64wc.. and n0+64wc+32...
// K loop: stages of 4 blocks (128 values, one q8_1 group).  The next stage's global loads are
// issued before the current stage's MFMAs and land in the other half of a double-buffered LDS,
// so each stage costs one barrier.  Weights are unpacked while staging: Q8_0's 34-byte blocks
// are realigned with v_alignbit, Q4_1's nibbles split into bytes (element j low nibble, j+16
// high), so both types feed the same int8 MFMA.  Scales stay fp16 bits in LDS and become f16
// MFMA operands directly.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kRowsM = kMmqRows;  // 64 activation rows per workgroup
constexpr int kRowsN = 128;       // weight rows per workgroup
constexpr int kKB = 4;            // blocks per stage
constexpr int kStride = 144;      // LDS bytes per row of q: 4 x 32 + 16 of padding

struct Buf {
  uint8_t aq[kRowsM * kStride];   // activation q, [row][block][32]
  uint8_t bq[kRowsN * kStride];   // weight q as int8, [row][block][32]
  uint16_t dx[kKB][2][32];        // [block][row tile][row]: fp16 d of the activation rows
  uint16_t dw[kKB][4][32];        // [block][col tile][row]: fp16 d of the weight rows
  uint32_t sx[kRowsM][2];         // [row][pair]: fp16 s of blocks (2p, 2p+1)
  uint32_t mw[kRowsN][2];         // [weight row][pair]: fp16 m of blocks (2p, 2p+1)
};

// The upper 32 lanes feed zeros into the single-k f16 outer products; they read them from
// this shadow, which has the layout of Buf::dx / Buf::dw and stays zero.
struct Zeros {
  uint16_t dx[kKB][2][32];
  uint16_t dw[kKB][4][32];
};

struct Stage {  // one thread's share of a stage's global loads, held in registers
  uint4 a[3];
  uint32_t w[17];
};

__device__ __forceinline__ int weight_row(int epi, int nb, int n0, int n_out) {
  // SwiGLU tiles hold gate features n0.. in LDS rows 0..63 and the same up features in 64..127
  return epi == 1 ? (nb < 64 ? n0 + nb : n_out + n0 + nb - 64) : n0 + nb;
}

template <int WT>
__device__ __forceinline__ void load_stage(Stage& st, const uint8_t* __restrict__ act,
                                           size_t act_row_bytes, int row0, int nrows,
                                           const uint8_t* __restrict__ W, size_t row_bytes,
                                           int s, int epi, int n0, int n_out) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int c = tid + 256 * j;  // 64 rows x 9 chunks of 16 bytes
    const int row = c / 9, part = c - row * 9;
    st.a[j] = make_uint4(0u, 0u, 0u, 0u);
    if (c < kRowsM * 9 && row < nrows)
      st.a[j] = *reinterpret_cast<const uint4*>(act + (size_t)(row0 + row) * act_row_bytes +
                                                (size_t)s * kDs4Bytes + part * 16);
  }
  const int nb = tid >> 1, pair = tid & 1;  // 128 weight rows x 2 pairs of blocks
  const uint8_t* src = W + (size_t)weight_row(epi, nb, n0, n_out) * row_bytes;
  if (WT == 0) {
    const uint32_t* p =
        reinterpret_cast<const uint32_t*>(src + (size_t)s * (kKB * 34) + pair * 68);
#pragma unroll
    for (int i = 0; i < 17; ++i) st.w[i] = p[i];
  } else {
    const uint2* p =
        reinterpret_cast<const uint2*>(src + (size_t)(s * kKB + 2 * pair) * 20);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint2 v = p[i];
      st.w[2 * i] = v.x;
      st.w[2 * i + 1] = v.y;
    }
  }
}

template <int WT>
__device__ __forceinline__ void store_stage(Buf& B, const Stage& st) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int c = tid + 256 * j;
    if (c < kRowsM * 9) {
      const int row = c / 9, part = c - row * 9;
      const int rt = row >> 5, rl = row & 31;
      if (part == 0) {
        const uint32_t h[4] = {st.a[j].x, st.a[j].y, st.a[j].z, st.a[j].w};
#pragma unroll
        for (int b = 0; b < 4; ++b) B.dx[b][rt][rl] = (uint16_t)(h[b] & 0xffffu);
        B.sx[row][0] = (h[0] >> 16) | (h[1] & 0xffff0000u);
        B.sx[row][1] = (h[2] >> 16) | (h[3] & 0xffff0000u);
      } else {
        *reinterpret_cast<uint4*>(B.aq + row * kStride + (part - 1) * 16) = st.a[j];
      }
    }
  }
  const int nb = tid >> 1, pair = tid & 1;
  const int ct = nb >> 5, cl = nb & 31;
  uint8_t* dst = B.bq + nb * kStride + (2 * pair) * 32;
  if (WT == 0) {
    const uint32_t* w = st.w;
    uint32_t q0[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q0[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], 16);
    *reinterpret_cast<uint4*>(dst) = make_uint4(q0[0], q0[1], q0[2], q0[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(q0[4], q0[5], q0[6], q0[7]);
    *reinterpret_cast<uint4*>(dst + 32) = make_uint4(w[9], w[10], w[11], w[12]);
    *reinterpret_cast<uint4*>(dst + 48) = make_uint4(w[13], w[14], w[15], w[16]);
    B.dw[2 * pair][ct][cl] = (uint16_t)(w[0] & 0xffffu);
    B.dw[2 * pair + 1][ct][cl] = (uint16_t)(w[8] >> 16);
  } else {
    B.mw[nb][pair] = (st.w[0] >> 16) | (st.w[5] & 0xffff0000u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t* w = st.w + 5 * j;
      *reinterpret_cast<uint4*>(dst + 32 * j) =
          make_uint4(w[1] & 0x0f0f0f0fu, w[2] & 0x0f0f0f0fu, w[3] & 0x0f0f0f0fu,
                     w[4] & 0x0f0f0f0fu);
      *reinterpret_cast<uint4*>(dst + 32 * j + 16) =
          make_uint4((w[1] >> 4) & 0x0f0f0f0fu, (w[2] >> 4) & 0x0f0f0f0fu,
                     (w[3] >> 4) & 0x0f0f0f0fu, (w[4] >> 4) & 0x0f0f0f0fu);
      B.dw[2 * pair + j][ct][cl] = (uint16_t)(w[0] & 0xffffu);
    }
  }
}

__device__ __forceinline__ void zero_shadow(Zeros& Z) {
  uint32_t* p = reinterpret_cast<uint32_t*>(&Z);
  for (int i = threadIdx.x; i < (int)(sizeof(Zeros) / 4); i += 256) p[i] = 0u;
}

template <int WT, int EPI>
__device__ __forceinline__ void mmq_tile(Buf (&L)[2], const Zeros& Z, const MmqProblem& p,
                                         const uint8_t* W, int row0, int nrows, int ntile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int nblk = p.k_in / kQK;
  const size_t row_bytes = (size_t)nblk * block_bytes(WT);
  const size_t act_row_bytes = (size_t)(p.k_in / kDs4Vals) * kDs4Bytes;
  const int n0 = EPI == 1 ? ntile * 64 : ntile * kRowsN;
  // the wavefront's two column tiles (32 LDS weight rows each)
  const int ct0 = EPI == 1 ? wc : 2 * wc;
  const int ct1 = EPI == 1 ? 2 + wc : 2 * wc + 1;
  const bool live = 32 * wr < nrows;  // a row tile past the expert's rows does no math

  v16f acc0, acc1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc0[i] = 0.0f;
    acc1[i] = 0.0f;
  }
  const v16i izero = {0};
  const v16f fzero = {0.0f};
  const int nstages = p.k_in / kDs4Vals;

  // f16 MFMA operands: element 0 carries the value, the other three dwords stay zero
  v4i op_dx = {0, 0, 0, 0}, op_dw0 = {0, 0, 0, 0}, op_dw1 = {0, 0, 0, 0};

  Stage st;
  load_stage<WT>(st, p.act, act_row_bytes, row0, nrows, W, row_bytes, 0, EPI, n0, p.n_out);
  __syncthreads();  // the previous tile's readers are done with both buffers
  store_stage<WT>(L[0], st);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    if (s + 1 < nstages)
      load_stage<WT>(st, p.act, act_row_bytes, row0, nrows, W, row_bytes, s + 1, EPI, n0,
                     p.n_out);
    const Buf& B = L[s & 1];
    if (live) {
      const uint8_t* arow = B.aq + (32 * wr + l32) * kStride + half * 16;
      const uint8_t* brow0 = B.bq + (32 * ct0 + l32) * kStride + half * 16;
      const uint8_t* brow1 = B.bq + (32 * ct1 + l32) * kStride + half * 16;
      if (EPI == 2) {
        int32_t* out = reinterpret_cast<int32_t*>(p.out);
#pragma unroll
        for (int b = 0; b < kKB; ++b) {
          const v4i a = *reinterpret_cast<const v4i*>(arow + b * 32);
          const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              a, *reinterpret_cast<const v4i*>(brow0 + b * 32), izero, 0, 0, 0);
          const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              a, *reinterpret_cast<const v4i*>(brow1 + b * 32), izero, 0, 0, 0);
          const int kb = s * kKB + b;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 32 * wr + 8 * (i >> 2) + 4 * half + (i & 3);
            if (row < nrows) {
              const size_t r = (size_t)(row0 + row);
              out[(r * p.n_out + n0 + 32 * ct0 + l32) * nblk + kb] = I0[i];
              out[(r * p.n_out + n0 + 32 * ct1 + l32) * nblk + kb] = I1[i];
            }
          }
        }
      } else {
        // f16 outer-product operands: the lower 32 lanes carry this stage's d values in k slot 0,
        // the upper 32 lanes read the zero shadow
        const uint16_t* dxp = half ? &Z.dx[0][wr][l32] : &B.dx[0][wr][l32];
        const uint16_t* dwp0 = half ? &Z.dw[0][ct0][l32] : &B.dw[0][ct0][l32];
        const uint16_t* dwp1 = half ? &Z.dw[0][ct1][l32] : &B.dw[0][ct1][l32];
        constexpr int kDxB = 2 * 32, kDwB = 4 * 32;  // element strides between blocks
        v16i I0, I1;
        v16f S0, S1;
        auto issue = [&](int b) {
          const v4i a = *reinterpret_cast<const v4i*>(arow + b * 32);
          I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              a, *reinterpret_cast<const v4i*>(brow0 + b * 32), izero, 0, 0, 0);
          I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              a, *reinterpret_cast<const v4i*>(brow1 + b * 32), izero, 0, 0, 0);
          op_dx[0] = dxp[b * kDxB];
          op_dw0[0] = dwp0[b * kDwB];
          op_dw1[0] = dwp1[b * kDwB];
          const v8h sdx = __builtin_bit_cast(v8h, op_dx);
          S0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              sdx, __builtin_bit_cast(v8h, op_dw0), fzero, 0, 0, 0);
          S1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              sdx, __builtin_bit_cast(v8h, op_dw1), fzero, 0, 0, 0);
        };
#pragma unroll
        for (int b = 0; b < kKB; ++b) {
          // (issuing the next block's MFMAs ahead of this block's VALU needs ~290 registers and
          // halves the occupancy; two resident wavefronts per SIMD interleave instead)
          issue(b);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            acc0[i] = fmaf((float)I0[i], S0[i], acc0[i]);
            acc1[i] = fmaf((float)I1[i], S1[i], acc1[i]);
          }
        }
        if (WT == 1) {
          // sum over the stage's 4 blocks of mw * sx: lanes 0..31 carry blocks 0,1 and lanes
          // 32..63 blocks 2,3 of the same rows, so no k slot is wasted on zeros
          op_dx[0] = (int)B.sx[32 * wr + l32][half];
          op_dw0[0] = (int)B.mw[32 * ct0 + l32][half];
          op_dw1[0] = (int)B.mw[32 * ct1 + l32][half];
          const v8h sxo = __builtin_bit_cast(v8h, op_dx);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sxo, __builtin_bit_cast(v8h, op_dw0),
                                                        acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sxo, __builtin_bit_cast(v8h, op_dw1),
                                                        acc1, 0, 0, 0);
        }
      }
    }
    if (s + 1 < nstages) store_stage<WT>(L[(s + 1) & 1], st);
    __syncthreads();
  }
  if (EPI == 2 || !live) return;

  if (EPI == 0) {
    float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * wr + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < nrows) {
        float* o = out + (size_t)(row0 + row) * p.n_out + n0;
        o[32 * ct0 + l32] = acc0[i];
        o[32 * ct1 + l32] = acc1[i];
      }
    }
    return;
  }

  // EPI == 1: h = silu(g) * u, then q8_1 along F: the 32 lanes of a half hold one block.
  // silu uses the hardware exp and reciprocal (h only has to be accurate); the quantisation of
  // h is the exact q8_1 arithmetic.
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
    const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
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
  __shared__ Buf L[2];
  __shared__ Zeros Z;
  const int mt = blockIdx.y;
  if (mt >= *p.n_tiles) return;
  zero_shadow(Z);
  const MTile t = p.tiles[mt];
  const uint8_t* W = p.wbase + (size_t)t.ordinal * p.pos_stride + p.mat_offset;
  mmq_tile<WT, EPI>(L, Z, p, W, t.row0, t.nrows, blockIdx.x);
}

template <int WT, int EPI>
__global__ __launch_bounds__(256) void mmq_group_kernel(MmqProblem p) {
  __shared__ Buf L[2];
  __shared__ Zeros Z;
  zero_shadow(Z);
  const int j = blockIdx.z;
  const int e = p.experts[j];
  const int r0 = p.offsets[e], cnt = p.offsets[e + 1] - r0;
  const uint8_t* W = p.wbase + (size_t)j * p.pos_stride + p.mat_offset;
  for (int m = blockIdx.y; m * kRowsM < cnt; m += gridDim.y)
    mmq_tile<WT, EPI>(L, Z, p, W, r0 + m * kRowsM, min(kRowsM, cnt - m * kRowsM),
                      blockIdx.x);
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
