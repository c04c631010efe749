// Microbenchmark of the MMQ's compute core on gfx950, registers only (no LDS, no global loads in
// the loop, no barriers), so that what it times is the instruction mix alone.
//
// Part 1, MFMA throughput: every wavefront runs independent accumulator chains of one MFMA shape;
// the result is the time per MFMA per SIMD and the chip-wide rate it implies.
//
// Part 2, the MMQ's per-block work for one wavefront's two 32x32 output tiles (what the grouped
// matmul issues per 32-value block): two v_mfma_i32_32x32x32_i8 (the block dots I), two
// v_mfma_f32_32x32x16_f16 (the scale products S), and per output element a convert of I to fp32
// and one fma into the accumulator.  Mixes (the time is per such "wave-block", per SIMD):
//   full             the kernel's mix
//   no convert       fma on I's bits (wrong values, timing only)
//   no f16 MFMA      S held in registers
//   no i8 MFMA       I held in registers
//   MFMAs only       the four MFMAs, two VALU ops to keep their results live
//   VALU only        32 convert + 32 fma on register operands
//   bias + add       the i8 MFMA's C input set to the bits of 1.5 * 2^23 and an fp32 add in place
//                    of the convert (exact for |I| < 2^22)
//   pipelined        block b+1's MFMAs interleaved with block b's convert + fma (two register
//                    sets), one MFMA then 16 VALU ops
//   i8 into AGPRs    the int8 MFMAs write accumulation registers (inline asm), each element is
//                    read back before its convert
//   VALU scales      no f16 MFMA: the scale products come from the VALU, S = dx * dw exactly with
//                    one v_fma_mix_f32 (fp16 operands, zero addend) per element; the 16 weight
//                    scales of a lane's 16 output elements are read from LDS every block (two
//                    16-byte reads per tile, one address per half-wavefront), dx is one fp16 per
//                    lane.  The orientation this needs: lanes = activation rows, registers =
//                    weight rows.
// each at 2, 3 and 4 wavefronts per SIMD (set by the LDS a workgroup reserves).
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                    \
      return -1.0;                                                                      \
    }                                                                                   \
  } while (0)

// ---- part 1 ------------------------------------------------------------------------------------
enum { R_I8_32 = 0, R_F16_32 = 1, R_I8_16 = 2, R_F16_16 = 3 };

template <int S>
__global__ __launch_bounds__(256, 2) void rate_kernel(const int* __restrict__ in,
                                                      float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const v4i a = {in[lane], in[lane + 64], in[lane + 128], in[lane + 192]};
  const v4i b = {in[lane + 256], in[lane + 320], in[lane + 384], in[lane + 448]};
  float t = 0.f;
  if (S == R_I8_32 || S == R_F16_32) {
    v16i ci[4];
    v16f cf[4];
    for (int j = 0; j < 4; ++j) {
      ci[j] = (v16i){0};
      cf[j] = (v16f){0.f};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (S == R_I8_32)
          ci[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, ci[j], 0, 0, 0);
        else
          cf[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                         __builtin_bit_cast(v8h, b), cf[j], 0, 0, 0);
      }
    }
    for (int j = 0; j < 4; ++j)
      for (int i = 0; i < 16; ++i) t += (float)ci[j][i] + cf[j][i];
  } else {
    v4i ci[8];
    v4f cf[8];
    for (int j = 0; j < 8; ++j) {
      ci[j] = (v4i){0, 0, 0, 0};
      cf[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (S == R_I8_16)
          ci[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, ci[j], 0, 0, 0);
        else
          cf[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                         __builtin_bit_cast(v8h, b), cf[j], 0, 0, 0);
      }
    }
    for (int j = 0; j < 8; ++j)
      for (int i = 0; i < 4; ++i) t += (float)ci[j][i] + cf[j][i];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = t;
}

template <int S>
double rate(int ncu, const int* din, float* dout, double macs, int per_iter, double* tops) {
  const int grid = ncu * 2, iters = 4096;  // two wavefronts per SIMD
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  rate_kernel<S><<<grid, 256>>>(din, dout, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  rate_kernel<S><<<grid, 256>>>(din, dout, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  const double per_simd = 2.0 * iters * per_iter;
  *tops = 2.0 * macs * per_simd * ncu * 4 / (ms * 1e-3) / 1e12;
  return ms * 1e6 / per_simd;
}

// ---- part 2 ------------------------------------------------------------------------------------
enum { M_FULL, M_NOCVT, M_NOF16, M_NOI8, M_MFMA, M_VALU, M_BIAS, M_PIPE, M_AGPR, M_VS, M_COUNT };
static const char* kMixName[M_COUNT] = {"full", "no convert", "no f16 MFMA", "no i8 MFMA",
                                        "MFMAs only", "VALU only", "bias + add", "pipelined",
                                        "i8 into AGPRs", "VALU scales"};

template <int M, int W>
__global__ __launch_bounds__(256, W) void mix_kernel(const int* __restrict__ in,
                                                     float* __restrict__ out, int nblocks) {
  extern __shared__ int lds_reserve[];  // sized by the host to set the occupancy
  const int lane = threadIdx.x & 63;
  v4i a = {in[lane], in[lane + 64], in[lane + 128], in[lane + 192]};
  v4i b0 = {in[lane + 256], in[lane + 320], in[lane + 384], in[lane + 448]};
  v4i b1 = {in[lane + 512], in[lane + 576], in[lane + 640], in[lane + 704]};
  v4i sa = {in[lane + 768] & 0xffff, 0, 0, 0};
  const v4i hw = {in[lane + 832], in[lane + 896], 0, 0};
  const v8h hw0 = __builtin_bit_cast(v8h, hw);
  const v16i izero = {0};
  const v16f fzero = {0.0f};
  int bias_bits;
  asm volatile("s_mov_b32 %0, 0x4b400000" : "=s"(bias_bits));  // 1.5 * 2^23
  float nbias;
  asm volatile("s_mov_b32 %0, 0xcb400000" : "=s"(nbias));       // -1.5 * 2^23
  v16i ibias;
  for (int i = 0; i < 16; ++i) ibias[i] = bias_bits;
  v16f acc0 = fzero, acc1 = fzero, Sr = fzero;
  v16i Ir = izero;
  for (int i = 0; i < 16; ++i) {
    Sr[i] = (float)in[lane + 960 + i];
    Ir[i] = in[lane + 1024 + i];
  }
  auto next_operands = [&](int blk) {  // the operands change every block (nothing is hoisted)
    a[0] ^= blk;
    b0[1] += blk;
    b1[2] += blk;
    sa[0] = (sa[0] + 1) & 0x3fff;
  };
  if (M == M_VS) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    // 8 blocks x 2 tiles x 2 half-wavefronts x 16 fp16 weight scales in LDS (as packed pairs)
    uint32_t* ws = reinterpret_cast<uint32_t*>(lds_reserve);
    for (int i = threadIdx.x; i < 8 * 2 * 2 * 8; i += blockDim.x) {
      const h2 v = {(_Float16)(1.0f + (float)(in[(2 * i) & 1023] & 1023) / 1024.0f),
                    (_Float16)(1.0f + (float)(in[(2 * i + 1) & 1023] & 1023) / 1024.0f)};
      ws[i] = __builtin_bit_cast(uint32_t, v);
    }
    __syncthreads();
    const int half = lane >> 5;
    for (int blk = 0; blk < nblocks; ++blk) {
      next_operands(blk);
      const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, izero, 0, 0, 0);
      const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, izero, 0, 0, 0);
      const _Float16 dx = __builtin_bit_cast(h2, sa[0]).x;
      const uint32_t* w0 = ws + ((blk & 7) * 4 + half) * 8;
      const uint32_t* w1 = w0 + 16;
      h2 d0[8], d1[8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(w0 + 4 * j);
        const uint4 x1 = *reinterpret_cast<const uint4*>(w1 + 4 * j);
        d0[4 * j] = __builtin_bit_cast(h2, x0.x);
        d0[4 * j + 1] = __builtin_bit_cast(h2, x0.y);
        d0[4 * j + 2] = __builtin_bit_cast(h2, x0.z);
        d0[4 * j + 3] = __builtin_bit_cast(h2, x0.w);
        d1[4 * j] = __builtin_bit_cast(h2, x1.x);
        d1[4 * j + 1] = __builtin_bit_cast(h2, x1.y);
        d1[4 * j + 2] = __builtin_bit_cast(h2, x1.z);
        d1[4 * j + 3] = __builtin_bit_cast(h2, x1.w);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float S0 = __builtin_fmaf((float)dx, (float)(i & 1 ? d0[i >> 1].y : d0[i >> 1].x), 0.0f);
        acc0[i] = fmaf((float)I0[i], S0, acc0[i]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float S1 = __builtin_fmaf((float)dx, (float)(i & 1 ? d1[i >> 1].y : d1[i >> 1].x), 0.0f);
        acc1[i] = fmaf((float)I1[i], S1, acc1[i]);
      }
    }
  } else if (M == M_PIPE) {
    v16i Ia0 = izero, Ia1 = izero, Ib0, Ib1;
    v16f Sa0 = fzero, Sa1 = fzero, Sb0, Sb1;
    auto step = [&](int blk, v16i& nI0, v16i& nI1, v16f& nS0, v16f& nS1, const v16i& I0,
                    const v16i& I1, const v16f& S0, const v16f& S1) {
      next_operands(blk);
      const v8h sx = __builtin_bit_cast(v8h, sa);
      float f0[16], f1[16];
      nI0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, izero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) f0[i] = (float)I0[i];
      nS0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sx, hw0, fzero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc0[i] = fmaf(f0[i], S0[i], acc0[i]);
      nI1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, izero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) f1[i] = (float)I1[i];
      nS1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(hw0, sx, fzero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc1[i] = fmaf(f1[i], S1[i], acc1[i]);
      for (int g = 0; g < 4; ++g) {  // one MFMA, then 16 VALU ops
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
      }
    };
    for (int blk = 0; blk < nblocks; blk += 2) {
      step(blk, Ib0, Ib1, Sb0, Sb1, Ia0, Ia1, Sa0, Sa1);
      step(blk + 1, Ia0, Ia1, Sa0, Sa1, Ib0, Ib1, Sb0, Sb1);
    }
    for (int i = 0; i < 16; ++i) {
      acc0[i] = fmaf((float)Ia0[i], Sa0[i], acc0[i]);
      acc1[i] = fmaf((float)Ia1[i], Sa1[i], acc1[i]);
    }
  } else {
    for (int blk = 0; blk < nblocks; ++blk) {
      next_operands(blk);
      const v8h sx = __builtin_bit_cast(v8h, sa);
      v16i I0, I1;
      v16f S0, S1;
      if (M == M_NOI8 || M == M_VALU) {
        I0 = Ir;
        I1 = Ir;
        I0[0] += blk;
      } else if (M == M_BIAS) {
        I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, ibias, 0, 0, 0);
        I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, ibias, 0, 0, 0);
      } else if (M == M_AGPR) {  // results in accumulation registers, read back per element
        asm("v_mfma_i32_32x32x32_i8 %0, %1, %2, 0" : "=a"(I0) : "v"(a), "v"(b0));
        asm("v_mfma_i32_32x32x32_i8 %0, %1, %2, 0" : "=a"(I1) : "v"(a), "v"(b1));
      } else {
        I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, izero, 0, 0, 0);
        I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, izero, 0, 0, 0);
      }
      if (M == M_NOF16 || M == M_VALU) {
        S0 = Sr;
        S1 = Sr;
        S0[1] += (float)blk;
      } else {
        S0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sx, hw0, fzero, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(hw0, sx, fzero, 0, 0, 0);
      }
      if (M == M_MFMA) {
        acc0[0] += __int_as_float(I0[blk & 15] ^ I1[(blk + 5) & 15]);
        acc1[0] += S0[blk & 15] * S1[(blk + 7) & 15];
        continue;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float f0, f1;
        if (M == M_NOCVT) {
          f0 = __int_as_float(I0[i]);
          f1 = __int_as_float(I1[i]);
        } else if (M == M_BIAS) {
          f0 = __int_as_float(I0[i]) + nbias;
          f1 = __int_as_float(I1[i]) + nbias;
        } else {
          f0 = (float)I0[i];
          f1 = (float)I1[i];
        }
        acc0[i] = fmaf(f0, S0[i], acc0[i]);
        acc1[i] = fmaf(f1, S1[i], acc1[i]);
      }
    }
  }
  float t0 = 0.f, t1 = 0.f;
  for (int i = 0; i < 16; ++i) {
    t0 += acc0[i];
    t1 += acc1[i];
  }
  float* o = out + ((size_t)blockIdx.x * 256 + threadIdx.x) * 2;
  o[0] = t0;
  o[1] = t1;
  if (lds_reserve[0] == 12345) o[0] = 0.f;  // keeps the reservation
}

// ns per wave-block per SIMD
template <int M, int W>
double mix1(int ncu, const int* din, float* dout) {
  const int nblocks = 512;
  size_t lds = (160 * 1024) / W - 1024;  // W workgroups per CU (one wavefront per SIMD each)
  if (lds > 65536) lds = 65536;
  const int grid = ncu * W * 4;
  CHECK(hipFuncSetAttribute((const void*)mix_kernel<M, W>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  mix_kernel<M, W><<<grid, 256, lds>>>(din, dout, nblocks);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  mix_kernel<M, W><<<grid, 256, lds>>>(din, dout, nblocks);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return ms * 1e6 / ((double)grid * 4 * nblocks / (ncu * 4.0));
}

template <int M>
void mix_row(int ncu, const int* din, float* dout) {
  printf("| %-12s | %7.1f | %7.1f | %7.1f |\n", kMixName[M], mix1<M, 2>(ncu, din, dout),
         mix1<M, 3>(ncu, din, dout), mix1<M, 4>(ncu, din, dout));
}

int main() {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, 0) != hipSuccess) return 1;
  const int ncu = p.multiProcessorCount;
  printf("device %s, %d CUs\n\n", p.gcnArchName, ncu);
  int h[2048];
  for (int i = 0; i < 2048; ++i) h[i] = (int)((i * 2654435761u) >> 7);
  int* din = nullptr;
  float* dout = nullptr;
  if (hipMalloc(&din, sizeof h) != hipSuccess ||
      hipMalloc(&dout, (size_t)ncu * 16 * 256 * 2 * sizeof(float)) != hipSuccess ||
      hipMemcpy(din, h, sizeof h, hipMemcpyHostToDevice) != hipSuccess)
    return 1;
  printf("MFMA throughput (independent chains, 2 wavefronts per SIMD):\n\n");
  printf("| MFMA | ns per MFMA per SIMD | chip TOP/s |\n|---|---:|---:|\n");
  double t;
  double ns = rate<R_I8_32>(ncu, din, dout, 32.0 * 32 * 32, 4, &t);
  printf("| v_mfma_i32_32x32x32_i8 | %.2f | %.0f |\n", ns, t);
  ns = rate<R_F16_32>(ncu, din, dout, 32.0 * 32 * 16, 4, &t);
  printf("| v_mfma_f32_32x32x16_f16 | %.2f | %.0f |\n", ns, t);
  ns = rate<R_I8_16>(ncu, din, dout, 16.0 * 16 * 64, 8, &t);
  printf("| v_mfma_i32_16x16x64_i8 | %.2f | %.0f |\n", ns, t);
  ns = rate<R_F16_16>(ncu, din, dout, 16.0 * 16 * 32, 8, &t);
  printf("| v_mfma_f32_16x16x32_f16 | %.2f | %.0f |\n", ns, t);
  printf("\nThe MMQ's per-block mix, ns per wave-block per SIMD, at 2 / 3 / 4 wavefronts per "
         "SIMD:\n\n");
  printf("| mix | 2 | 3 | 4 |\n|---|---:|---:|---:|\n");
  mix_row<M_FULL>(ncu, din, dout);
  mix_row<M_NOCVT>(ncu, din, dout);
  mix_row<M_NOF16>(ncu, din, dout);
  mix_row<M_NOI8>(ncu, din, dout);
  mix_row<M_MFMA>(ncu, din, dout);
  mix_row<M_VALU>(ncu, din, dout);
  mix_row<M_BIAS>(ncu, din, dout);
  mix_row<M_PIPE>(ncu, din, dout);
  mix_row<M_AGPR>(ncu, din, dout);
  mix_row<M_VS>(ncu, din, dout);
  const hipError_t e = hipDeviceSynchronize();
  printf("\nstatus %s\n", hipGetErrorString(e));
  return e == hipSuccess ? 0 : 1;
}
