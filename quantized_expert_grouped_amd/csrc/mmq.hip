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
// high), so both types feed the same int8 MFMA.  Scales stay fp16 bits, laid out in LDS as the
// f16 MFMA operands (with the unused k slots zero).
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
  uint16_t dx[kKB][2][64];        // [block][row tile][lane]: d of row (lane < 32), else 0
  uint16_t dw[kKB][4][64];        // [block][col tile][lane]: d of weight row, else 0
  uint16_t sx[2][64][8];          // [row tile][lane][k]: s of the stage's 4 blocks, rest 0
  uint16_t mw[4][64][8];          // [col tile][lane][k]: m of the stage's 4 blocks, rest 0
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
        for (int b = 0; b < 4; ++b) {
          B.dx[b][rt][rl] = (uint16_t)(h[b] & 0xffffu);
          B.sx[rt][rl][b] = (uint16_t)(h[b] >> 16);
        }
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
      B.mw[ct][cl][2 * pair + j] = (uint16_t)(w[0] >> 16);
    }
  }
}

__device__ __forceinline__ void zero_tables(Buf& B) {
  // the f16 operands' unused halves (lanes 32..63, k slots 4..7) stay zero for the whole kernel
  uint32_t* p = reinterpret_cast<uint32_t*>(&B.dx[0][0][0]);
  const int n = (int)((sizeof(B.dx) + sizeof(B.dw) + sizeof(B.sx) + sizeof(B.mw)) / 4);
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

__device__ __forceinline__ v8h f16_operand(uint32_t lo) {
  return __builtin_bit_cast(v8h, (v4i){(int)lo, 0, 0, 0});
}

template <int WT, int EPI>
__device__ __forceinline__ void mmq_tile(Buf (&L)[2], const MmqProblem& p, const uint8_t* W,
                                         int row0, int nrows, int ntile) {
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

  Stage st;
  __syncthreads();  // the previous tile's readers are done with both buffers
  zero_tables(L[0]);
  zero_tables(L[1]);
  load_stage<WT>(st, p.act, act_row_bytes, row0, nrows, W, row_bytes, 0, EPI, n0, p.n_out);
  __syncthreads();
  store_stage<WT>(L[0], st);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    if (s + 1 < nstages)
      load_stage<WT>(st, p.act, act_row_bytes, row0, nrows, W, row_bytes, s + 1, EPI, n0,
                     p.n_out);
    const Buf& B = L[s & 1];
    if (live) {
#pragma unroll
      for (int b = 0; b < kKB; ++b) {
        const v4i a = *reinterpret_cast<const v4i*>(B.aq + (32 * wr + l32) * kStride + b * 32 +
                                                    half * 16);
        const v4i b0 = *reinterpret_cast<const v4i*>(B.bq + (32 * ct0 + l32) * kStride +
                                                     b * 32 + half * 16);
        const v4i b1 = *reinterpret_cast<const v4i*>(B.bq + (32 * ct1 + l32) * kStride +
                                                     b * 32 + half * 16);
        const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, izero, 0, 0, 0);
        const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, izero, 0, 0, 0);
        if (EPI == 2) {
          int32_t* out = reinterpret_cast<int32_t*>(p.out);
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
          continue;
        }
        const v8h sdx = f16_operand(B.dx[b][wr][lane]);
        const v16f S0 =
            __builtin_amdgcn_mfma_f32_32x32x16_f16(sdx, f16_operand(B.dw[b][ct0][lane]), fzero,
                                                    0, 0, 0);
        const v16f S1 =
            __builtin_amdgcn_mfma_f32_32x32x16_f16(sdx, f16_operand(B.dw[b][ct1][lane]), fzero,
                                                    0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc0[i] = fmaf((float)I0[i], S0[i], acc0[i]);
          acc1[i] = fmaf((float)I1[i], S1[i], acc1[i]);
        }
      }
      if (WT == 1 && EPI != 2) {
        const v8h sxo = *reinterpret_cast<const v8h*>(&B.sx[wr][lane][0]);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            sxo, *reinterpret_cast<const v8h*>(&B.mw[ct0][lane][0]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            sxo, *reinterpret_cast<const v8h*>(&B.mw[ct1][lane][0]), acc1, 0, 0, 0);
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
  __shared__ Buf L[2];
  const int mt = blockIdx.y;
  if (mt >= *p.n_tiles) return;
  const MTile t = p.tiles[mt];
  const uint8_t* W = p.wbase + (size_t)t.ordinal * p.pos_stride + p.mat_offset;
  mmq_tile<WT, EPI>(L, p, W, t.row0, t.nrows, blockIdx.x);
}

template <int WT, int EPI>
__global__ __launch_bounds__(256) void mmq_group_kernel(MmqProblem p) {
  __shared__ Buf L[2];
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
