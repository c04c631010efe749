// a4..a6  Grouped quantised matmul (MMQ) on q8_1 activations.  "Prompt path: an MMQ group's
// experts gathered in one launch, after one wait, released by one event", "What changes": how
// a group is gathered alters neither which products its experts compute nor their order;
// "#1368 prefill: quantize each token's MoE input once and scatter it to its k rows", opening
// section: the down projection's input is quantised to q8_1 again.
//
// For weight row n and activation row r, block b (32 values):
//   I_b = sum_j qw_j * qx_j                 exact int32: one v_mfma_i32_32x32x32_i8 per block
//                                           (K = 32 is exactly one block)
//   S_b = dx_b * dw_b                       exact in fp32 (two fp16 significands); for a whole
//                                           32x32 tile an outer product: one
//                                           v_mfma_f32_32x32x8_f16 (on gfx950 it issues faster
//                                           than the 32x32x16 form, and one K-slot is all an
//                                           outer product needs)
//   acc = fma(float(I_b), S_b, acc)         the only per-element VALU work (convert + fma)
//   Q4_1 adds sum_b mw_b * sx_b             a true sum over blocks: an f16 MFMA whose C input
//                                           is the accumulator itself, once per stage
// The f16 MFMAs' K-sum runs over both lane halves.  In the fp32-output kernel the second half's
// activation-scale operand is zero, so each product dx_b * dw_b (and mw_b * sx_b) enters once;
// the SwiGLU kernel feeds the scale from both halves, so it gets exactly 2*S_b and 2*mw_b*sx_b,
// and its epilogue takes the factor 2 out inside silu's argument and with one final quarter,
// which in binary floating point changes no rounding (instead of masks held in registers).
// Blocks are taken in ascending order and every output element is accumulated by one lane in
// one fixed instruction sequence, so results do not depend on the tiling, the group size, the
// ring start or the row's place in its tile.
//
// Workgroup: 64 activation rows (one m-tile of one expert) x 128 weight rows, 4 wavefronts; the
// fp32-output kernel's workgroup goes on through up to 4 such weight-row tiles (n-tiles) in turn.
// Wavefront (wr, wc) owns rows 32*wr.. and two 32-row column tiles of the weights:
//   MOE_EPI_SWIGLU_Q8_1: gate features f0+32wc.. and the up rows of the same features, so
//     h = silu(g) * u is formed in registers and requantised along F across the 32 lanes that
//     hold one block of 32 features;
//   otherwise: weight rows n0+64wc.. and n0+64wc+32...
// K loop: stages of 4 blocks (128 values, one q8_1 group).  Stages stream into a ring of two LDS
// buffers with direct global->LDS loads (global_load_lds_dwordx4), one stage ahead of the
// MFMAs, at three or four workgroups per CU, so the registers hold no staged data and no VALU
// moves it.
// The weights come from the group buffer's MMQ layout (64-row tiles of one stage, each
// contiguous, every row's block headers first), so a workgroup's weight stage is two contiguous
// runs, and in LDS the rows sit 80 (Q4_1) or 136 (Q8_0) bytes apart.  q8_1 rows keep their
// 144-byte groups.  LDS serves 8-byte reads 32 lanes and 16-byte reads 16 lanes at a time over
// 64 four-byte banks: the 16-byte reads at both strides and Q8_0's 8-byte pairs are
// conflict-free; Q4_1's 8-byte weight reads conflict 2-way (reading two blocks' halves with one
// 16-byte read instead measured no faster).  A lane half h takes elements 16h..16h+15 of a block
// on both operands: one 16-byte activation read (an 8-byte pair 16 bytes apart would conflict
// 2-way on the 144-byte row stride) and, for Q4_1, the block's 8-byte half h, whose low and
// high nibbles the gather arranged to be exactly those elements, split with two masks.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

constexpr int kRowsM = kMmqRows;  // 64 activation rows per workgroup
constexpr int kRowsN = 128;       // weight rows per workgroup
constexpr int kKB = 4;            // blocks per stage
constexpr int kARow = 144;        // bytes of one q8_1 group (the stage's slice of a row)
constexpr int kAInstr = kRowsM * kARow / (64 * 16);  // 9 DMA instructions per stage

// Weights arrive in the MMQ layout the gather writes: each matrix as tiles of 64 rows by one
// stage (4 blocks), every tile-stage contiguous, a row's 4 blocks headers first (Q4_1: 4 x (d, m)
// then 4 x 16 packed bytes, each block's byte 8h + i holding elements 16h + i and 16h + 8 + i,
// 80 B; Q8_0: 4 x d then 4 x q[32], 136 B).  A workgroup's stage is two such
// tile-stages, copied verbatim into LDS rows 0..63 and 64..127.
template <int WT>
struct Geo {
  static constexpr int kBRow = WT == 1 ? 4 * 20 : 4 * 34;          // bytes of a row per stage
  static constexpr int kTilePieces = 64 * kBRow / 16;              // 16-byte pieces per tile-stage
  static constexpr int kBInstr = 2 * kTilePieces / 64;             // 17 or 10
  static constexpr int kBPerWave = (kBInstr + 3) / 4;              // 5 or 3
};

template <int WT>
struct alignas(16) StageBuf {
  uint8_t a[kRowsM * kARow];
  uint8_t b[kRowsN * Geo<WT>::kBRow];
};

// LDS stage buffers per workgroup: two (19.5 KB for Q4_1, 26.6 KB for Q8_0; one stage in flight
// ahead of the MFMAs), so that three workgroups fit in a CU's 160 KB and in 168 VGPRs: three
// wavefronts per SIMD hide each other's waits better than deeper prefetch does (a ring of four,
// or three, at two workgroups per CU was 5-9% slower).  Q4_1's kernels run four (their ring
// fits four times in LDS): gate/up fits 128 VGPRs when each column tile's MFMAs and
// convert + fma run in turn (measured 3% faster at T = 8,192), down when each wavefront takes
// one column tile of both row tiles (below).  The raw block-dot epilogue and the per-group
// kernel stay at two workgroups per CU (they would spill at three).
constexpr int kWgPerCu = 3;
template <int WT, int EPI>
constexpr int wg_per_cu() {
  return EPI == 2 ? 2 : (WT == 1 ? 4 : kWgPerCu);
}

// The fp32-output (down) kernel's workgroup sweeps up to kSweep consecutive n-tiles of its m-tile
// through one ring: its short reduction (k_in = F, a few stages) would otherwise pay a ring fill
// and an output drain per n-tile (measured at T = 8,192 / 32,768: down -4% / -9%).
constexpr int kSweep = 4;

template <int WT>
struct Ring {
  StageBuf<WT> buf[2];
};

// s_waitcnt immediate for vmcnt(n) (0 <= n < 64) with the other counters left alone
constexpr int vm_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Each lane's byte offsets of its DMA pieces, relative to the stage's first byte in global
// memory; fixed for a tile, the stage advance is added to the (uniform) base pointer.
template <int WT>
struct DmaPlan {
  uint32_t a[3];
  uint32_t b[Geo<WT>::kBPerWave];
};

__device__ __forceinline__ int wave_id() {  // uniform across the wavefront, kept in an SGPR
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// tile0 / tile1: byte offsets (from the weight pointer) of the two 64-row tiles whose stage 0
// fills LDS rows 0..63 and 64..127; stage t adds t * 64 * kBRow to both.
template <int WT>
__device__ __forceinline__ void plan_dma(DmaPlan<WT>& d, size_t act_row_bytes, int nrows,
                                         size_t tile0, size_t tile1) {
  const int lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int c = 64 * (wave + 4 * j) + lane;  // 16-byte piece of the 64 x 144-byte slice
    const int row = min(c / 9, nrows - 1);     // rows past the expert repeat its last row
    d.a[j] = (uint32_t)(row * act_row_bytes + (c % 9) * 16);
  }
#pragma unroll
  for (int j = 0; j < Geo<WT>::kBPerWave; ++j) {
    const int c = min(64 * (wave + 4 * j) + lane, 2 * Geo<WT>::kTilePieces - 1);
    const int k = Geo<WT>::kTilePieces;
    d.b[j] = (uint32_t)(c < k ? tile0 + 16 * c : tile1 + 16 * (c - k));
  }
}

// One direct global->LDS load: lane i's 16 (or 4) bytes land at lds + 16*i (4*i), lds
// wave-uniform (it is passed in M0).  Written as inline assembly so that the compiler's wait-count
// pass does not treat every later LDS read as possibly overlapping it (it cannot tell the ring
// buffers apart and would drain the loads in flight); the kernel orders these loads itself with
// explicit vmcnt waits and barriers.  Every other VMEM operation of the kernel retires in issue
// order with these, so the compiler's own waits stay correct (they can only wait longer).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// M0 is an input operand (the compiler writes it); the s_nop covers the one wait state an LDS
// DMA needs after an M0 write.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "{m0}"(lds), "v"(g) : "memory");
}

// Wavefront W of the workgroup issues pieces W, W + 4, ... of the stage: with W a template
// argument every piece's presence and LDS address are compile-time, so the issue is straight-line
// code (a runtime wavefront index cost a compare and a branch per piece).
template <int WT, int W>
__device__ __forceinline__ void issue_stage_w(uint32_t la, uint32_t lb, const DmaPlan<WT>& d,
                                              const uint8_t* abase, const uint8_t* wbase) {
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = W + 4 * j;
    if (i < kAInstr) dma16(abase + d.a[j], la + i * 1024);
  }
#pragma unroll
  for (int j = 0; j < Geo<WT>::kBPerWave; ++j) {
    const int i = W + 4 * j;
    if (i < Geo<WT>::kBInstr) dma16(wbase + d.b[j], lb + i * 64 * 16);
  }
}

template <int WT>
__device__ __forceinline__ void issue_stage(StageBuf<WT>& S, const DmaPlan<WT>& d,
                                            const uint8_t* abase, const uint8_t* wbase) {
  // the buffers' LDS addresses as opaque values (folded into constants, the generic-to-LDS
  // pointer conversion miscompiled)
  uint32_t la = lds_address(S.a), lb = lds_address(S.b);
  asm volatile("" : "+s"(la), "+s"(lb));
  switch (wave_id()) {
    case 0: issue_stage_w<WT, 0>(la, lb, d, abase, wbase); break;
    case 1: issue_stage_w<WT, 1>(la, lb, d, abase, wbase); break;
    case 2: issue_stage_w<WT, 2>(la, lb, d, abase, wbase); break;
    default: issue_stage_w<WT, 3>(la, lb, d, abase, wbase); break;
  }
}

// int8 MFMA operands of block b: lane half h takes elements 16h..16h+15 of both operands.
template <int WT>
__device__ __forceinline__ v4i a_frag(const uint8_t* arow, int b, int half) {
  return *reinterpret_cast<const v4i*>(arow + 16 + 32 * b + 16 * half);
}

// Weight operand of block b from a row's stage bytes (headers first).  Q4_1: the block's packed
// half h, low nibbles = elements 16h..16h+7, high nibbles = 16h+8..16h+15.
template <int WT>
__device__ __forceinline__ v4i b_frag(const uint8_t* brow, int b, int half) {
  if (WT == 1) {
    const uint2 x = *reinterpret_cast<const uint2*>(brow + 16 + 16 * b + 8 * half);
    const uint32_t m = 0x0f0f0f0fu;
    return (v4i){(int)(x.x & m), (int)(x.y & m), (int)((x.x >> 4) & m), (int)((x.y >> 4) & m)};
  }
  const uint8_t* q = brow + 8 + 32 * b + 16 * half;  // 8-byte aligned
  const uint2 lo = *reinterpret_cast<const uint2*>(q);
  const uint2 hi = *reinterpret_cast<const uint2*>(q + 8);
  return (v4i){(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
}

// The same operand in two steps, so that the LDS read can run ahead: the raw bytes (Q4_1: the
// 8 packed bytes in the low two words), then the int8 operand.
template <int WT>
__device__ __forceinline__ v4i b_raw(const uint8_t* brow, int b, int half) {
  if (WT == 1) {
    const uint2 x = *reinterpret_cast<const uint2*>(brow + 16 + 16 * b + 8 * half);
    return (v4i){(int)x.x, (int)x.y, 0, 0};
  }
  return b_frag<WT>(brow, b, half);
}

template <int WT>
__device__ __forceinline__ v4i b_unpack(const v4i& r) {
  if (WT != 1) return r;
  const uint32_t m = 0x0f0f0f0fu, x0 = (uint32_t)r[0], x1 = (uint32_t)r[1];
  return (v4i){(int)(x0 & m), (int)(x1 & m), (int)((x0 >> 4) & m), (int)((x1 >> 4) & m)};
}

// A row's weight headers as four dwords of fp16 pairs, the scale MFMAs' weight operands taken a
// dword pair at a time: Q4_1 (d_b, m_b) in dword b; Q8_0 d_0..d_3 in dwords 0 and 1 (2 and 3
// unused); Q8_0 read with D4 activations (d_b, d_b) in dword b (they meet the two fp16 halves of
// the activation's fp32 d).
template <int WT>
__device__ __forceinline__ v4i b_header(const uint8_t* brow) {
  if (WT == 1) return *reinterpret_cast<const v4i*>(brow);
  const uint2 d = *reinterpret_cast<const uint2*>(brow);
  if (WT == kWtQ8_0D4)
    return (v4i){(int)((d.x & 0xffffu) | (d.x << 16)), (int)((d.x >> 16) | (d.x & 0xffff0000u)),
                 (int)((d.y & 0xffffu) | (d.y << 16)), (int)((d.y >> 16) | (d.y & 0xffff0000u))};
  return (v4i){(int)d.x, (int)d.y, 0, 0};
}

// Wavefront roles.  By default wavefront w computes row tile w / 2 against two column tiles.
// Q4_1's fp32-output (down) kernel instead gives wavefront w column tile w of both row tiles:
// each weight fragment's nibbles are then split once per workgroup instead of twice (six VALU
// instructions per tile and block), and the kernel fits 128 VGPRs, so four workgroups share a
// CU (measured down -9.5% at T = 8,192, -6.8% on the Zipf workload; outputs bit-identical).  The
// SwiGLU kernel keeps the default: it needs gate and up of one feature in one wavefront.  NG
// and NG1 are the live 8-row groups of the wavefront's (first) and second row tile; NG1 = 0
// means row tile 1 holds none of the expert's rows.
template <int WT, int EPI, int NG = 4, int NG1 = 4>
__device__ __forceinline__ void mmq_tile(StageBuf<WT>& L0, StageBuf<WT>& L1,
                                         const MmqProblem& p, const uint8_t* W, int row0,
                                         int nrows, int ntile, int nsweep = 1) {
  constexpr bool kByColumn = WT == 1 && EPI == 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int nblk = p.k_in / kQK;
  const size_t act_row_bytes = (size_t)(p.k_in / kDs4Vals) * kDs4Bytes;
  const size_t tile_bytes = (size_t)(nblk / kKB) * 64 * Geo<WT>::kBRow;  // one 64-row tile
  const int n0 = EPI == 1 ? ntile * 64 : ntile * kRowsN;
  // the wavefront's two column tiles (32 LDS weight rows each)
  const int ct0 = EPI == 1 ? wc : 2 * wc;
  const int ct1 = EPI == 1 ? 2 + wc : 2 * wc + 1;
  const bool live = kByColumn || 32 * wr < nrows;  // a row tile past the expert's rows: no math
  const int nstages = p.k_in / kDs4Vals;
  const uint8_t* abase = p.act + (size_t)row0 * act_row_bytes;

  // SwiGLU: gate tile ntile and the up matrix's tile ntile; otherwise tiles 2*ntile, 2*ntile+1
  const size_t up_offset = (size_t)p.n_out * nblk * block_bytes(WT);
  const size_t tile0 = EPI == 1 ? ntile * tile_bytes : 2 * ntile * tile_bytes;
  const size_t tile1 = EPI == 1 ? up_offset + ntile * tile_bytes : tile0 + tile_bytes;
  DmaPlan<WT> plan;
  plan_dma<WT>(plan, act_row_bytes, nrows, tile0, tile1);

  v16f acc0, acc1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc0[i] = 0.0f;
    acc1[i] = 0.0f;
  }
  const v16i izero = {0};
  const v16f fzero = {0.0f};

  // The scale operand's selectors: the fp16 kept in the low half of a dword, or moved to the high
  // half (v_perm selector byte 0x0c is a zero byte); in the fp32-output kernel, lane half 1
  // contributes zeros.
  constexpr bool kOnce = EPI == 0;
  const bool zero_half = kOnce && half != 0;
  const uint32_t keep_lo = zero_half ? 0u : 0xffffu, keep_hi = keep_lo << 16;
  const uint32_t to_hi = zero_half ? 0x0c0c0c0cu : 0x01000c0cu;
  const uint32_t sel_s = zero_half ? 0x0c0c0c0cu : 0x07060302u;

  // stage t of the sweep's n-tile j (EPI 0: n-tile j's weights start 2j 64-row tiles later)
  auto issue = [&](StageBuf<WT>& buf, int j, int t) {
    issue_stage<WT>(buf, plan, abase + (size_t)t * kARow,
                    W + (size_t)j * 2 * tile_bytes + (size_t)t * 64 * Geo<WT>::kBRow);
  };

  // The MFMAs of stage s from LDS buffer `cur` into the accumulators.
  auto math = [&](int s, const StageBuf<WT>& cur) {
    const uint8_t* arow = cur.a + (32 * wr + l32) * kARow;
    const uint8_t* brow0 = cur.b + (32 * ct0 + l32) * Geo<WT>::kBRow;
    const uint8_t* brow1 = cur.b + (32 * ct1 + l32) * Geo<WT>::kBRow;
    if (EPI == 2) {
      int32_t* out = reinterpret_cast<int32_t*>(p.out);
#pragma unroll
      for (int b = 0; b < kKB; ++b) {
        const v4i a = a_frag<WT>(arow, b, half);
        const v16i I0 =
            __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b_frag<WT>(brow0, b, half), izero, 0, 0, 0);
        const v16i I1 =
            __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b_frag<WT>(brow1, b, half), izero, 0, 0, 0);
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
      return;
    }
    if (kByColumn) {  // column tile `wave` of row tiles 0 and 1
      const uint8_t* arow0 = cur.a + l32 * kARow;
      const uint8_t* arow1 = cur.a + (32 + l32) * kARow;
      const uint8_t* brow = cur.b + (32 * wave + l32) * Geo<WT>::kBRow;
      const v4i hx0 = *reinterpret_cast<const v4i*>(arow0);
      const v4i hw = b_header<WT>(brow);
      // the min term as in the default roles, for each row tile
      const v4h m = __builtin_bit_cast(
          v4h, (v2i){(int)__builtin_amdgcn_perm((uint32_t)hw[1], (uint32_t)hw[0], 0x07060302u),
                     (int)__builtin_amdgcn_perm((uint32_t)hw[3], (uint32_t)hw[2], 0x07060302u)});
      const v4h ss0 = __builtin_bit_cast(
          v4h, (v2i){(int)__builtin_amdgcn_perm((uint32_t)hx0[1], (uint32_t)hx0[0], sel_s),
                     (int)__builtin_amdgcn_perm((uint32_t)hx0[3], (uint32_t)hx0[2], sel_s)});
      acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(ss0, m, acc0, 0, 0, 0);
      v4i hx1 = hx0;
      if (NG1 > 0) {
        hx1 = *reinterpret_cast<const v4i*>(arow1);
        const v4h ss1 = __builtin_bit_cast(
            v4h, (v2i){(int)__builtin_amdgcn_perm((uint32_t)hx1[1], (uint32_t)hx1[0], sel_s),
                       (int)__builtin_amdgcn_perm((uint32_t)hx1[3], (uint32_t)hx1[2], sel_s)});
        acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(ss1, m, acc1, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < kKB; ++b) {
        const v4i xb = b_unpack<WT>(b_raw<WT>(brow, b, half));  // split once, used twice
        const v4h w =
            __builtin_bit_cast(v4h, (b >> 1) ? (v2i){hw[2], hw[3]} : (v2i){hw[0], hw[1]});
        {
          const uint32_t sv = (uint32_t)hx0[b] & keep_lo;
          const v4h sx = __builtin_bit_cast(v4h, (b & 1) ? (v2i){0, (int)sv} : (v2i){(int)sv, 0});
          const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_frag<WT>(arow0, b, half), xb,
                                                                izero, 0, 0, 0);
          const v16f S0 = __builtin_amdgcn_mfma_f32_32x32x8f16(sx, w, fzero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4 * NG; ++i) acc0[i] = fmaf((float)I0[i], S0[i], acc0[i]);
        }
        if (NG1 > 0) {
          __builtin_amdgcn_sched_barrier(0);
          const uint32_t sv = (uint32_t)hx1[b] & keep_lo;
          const v4h sx = __builtin_bit_cast(v4h, (b & 1) ? (v2i){0, (int)sv} : (v2i){(int)sv, 0});
          const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_frag<WT>(arow1, b, half), xb,
                                                                izero, 0, 0, 0);
          const v16f S1 = __builtin_amdgcn_mfma_f32_32x32x8f16(sx, w, fzero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4 * NG1; ++i) acc1[i] = fmaf((float)I1[i], S1[i], acc1[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    // activation headers (d_b, s_b) of the row, weight headers of the two column tiles
    const v4i hx = *reinterpret_cast<const v4i*>(arow);
    const v4i hw0 = b_header<WT>(brow0);
    const v4i hw1 = b_header<WT>(brow1);
    if (WT == 1) {
      // sum over the stage's blocks of sx_b * mw_b, added first so that its operands die before
      // the block loop: (s_0, s_1, s_2, s_3) against (m_0, m_1, m_2, m_3), both gathered from
      // the headers' high halves; zeros in lane half 1 of the fp32-output kernel
      const v4h ss = __builtin_bit_cast(
          v4h, (v2i){(int)__builtin_amdgcn_perm((uint32_t)hx[1], (uint32_t)hx[0], sel_s),
                     (int)__builtin_amdgcn_perm((uint32_t)hx[3], (uint32_t)hx[2], sel_s)});
      const v4h m0 = __builtin_bit_cast(
          v4h, (v2i){(int)__builtin_amdgcn_perm((uint32_t)hw0[1], (uint32_t)hw0[0], 0x07060302u),
                     (int)__builtin_amdgcn_perm((uint32_t)hw0[3], (uint32_t)hw0[2], 0x07060302u)});
      const v4h m1 = __builtin_bit_cast(
          v4h, (v2i){(int)__builtin_amdgcn_perm((uint32_t)hw1[1], (uint32_t)hw1[0], 0x07060302u),
                     (int)__builtin_amdgcn_perm((uint32_t)hw1[3], (uint32_t)hw1[2], 0x07060302u)});
      acc0 = __builtin_amdgcn_mfma_f32_32x32x8f16(ss, m0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x8f16(ss, m1, acc1, 0, 0, 0);
    }
    // Q4_1: the LDS reads of each block's operands are issued one block ahead of its MFMAs
    v4i fa = a_frag<WT>(arow, 0, half), f0 = b_raw<WT>(brow0, 0, half),
        f1 = b_raw<WT>(brow1, 0, half);
#pragma unroll
    for (int b = 0; b < kKB; ++b) {
      // Q8_0 reads each block's operands where it uses them: its 4-VGPR weight fragments held
      // one block ahead would not fit three workgroups' registers
      const v4i a = WT == 1 ? fa : a_frag<WT>(arow, b, half);
      const v4i x0 = WT == 1 ? f0 : b_raw<WT>(brow0, b, half);
      const v4i x1 = WT == 1 ? f1 : b_raw<WT>(brow1, b, half);
      if (WT == 1 && b + 1 < kKB) {
        fa = a_frag<WT>(arow, b + 1, half);
        f0 = b_raw<WT>(brow0, b + 1, half);
        f1 = b_raw<WT>(brow1, b + 1, half);
      }
      // S_b = dx_b * dw_b from v_mfma_f32_32x32x8_f16: a lane half supplies four fp16 K-slots
      // (two dwords); the weight operand is one dword pair of the header, the activation operand
      // holds dx_b in the slot facing dw_b and zeros elsewhere.  Q4_1 and D4: header dword b
      // holds block b's two weight fp16, the pair (2 (b / 2), 2 (b / 2) + 1); Q8_0: d_0..d_3 in
      // slots 0..3 of the pair (0, 1).  D4's fp32 dx_b goes in as two fp16 (hi = fp16(dx),
      // lo = fp16(dx - hi)) in both slots of its dword, both facing dw_b: the MFMA adds
      // hi*dw + lo*dw, each product exact in fp32.  Lane half 1 holds zeros in the fp32-output
      // kernel and the same values in the SwiGLU kernel.
      uint32_t sv;
      if (WT == kWtQ8_0D4) {
        const float dx = __int_as_float(hx[b]);
        const _Float16 hi = (_Float16)dx;
        const _Float16 lo = (_Float16)(dx - (float)hi);
        sv = ((uint32_t)__builtin_bit_cast(uint16_t, hi) |
              ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16)) &
             (keep_lo | keep_hi);
      } else if (WT == 1 || (b & 1) == 0) {
        sv = (uint32_t)hx[b] & keep_lo;
      } else {
        sv = __builtin_amdgcn_perm(0u, (uint32_t)hx[b], to_hi);
      }
      const int dsel = WT == 0 ? (b >> 1) : (b & 1);   // the dword of the pair dx_b goes in
      const v4h sx = __builtin_bit_cast(v4h, dsel ? (v2i){0, (int)sv} : (v2i){(int)sv, 0});
      const int pair = WT == 0 ? 0 : (b >> 1);
      const v4h w0 = __builtin_bit_cast(v4h, pair ? (v2i){hw0[2], hw0[3]} : (v2i){hw0[0], hw0[1]});
      const v4h w1 = __builtin_bit_cast(v4h, pair ? (v2i){hw1[2], hw1[3]} : (v2i){hw1[0], hw1[1]});
      if (WT == 1 && EPI == 1) {  // one column tile after the other (fits 128 VGPRs)
        {
          const v16i I0 =
              __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b_unpack<WT>(x0), izero, 0, 0, 0);
          const v16f S0 = __builtin_amdgcn_mfma_f32_32x32x8f16(sx, w0, fzero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4 * NG; ++i) acc0[i] = fmaf((float)I0[i], S0[i], acc0[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          const v16i I1 =
              __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b_unpack<WT>(x1), izero, 0, 0, 0);
          const v16f S1 = __builtin_amdgcn_mfma_f32_32x32x8f16(sx, w1, fzero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4 * NG; ++i) acc1[i] = fmaf((float)I1[i], S1[i], acc1[i]);
        }
        continue;
      }
      const v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b_unpack<WT>(x0), izero, 0, 0, 0);
      const v16f S0 = __builtin_amdgcn_mfma_f32_32x32x8f16(sx, w0, fzero, 0, 0, 0);
      const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b_unpack<WT>(x1), izero, 0, 0, 0);
      const v16f S1 = __builtin_amdgcn_mfma_f32_32x32x8f16(sx, w1, fzero, 0, 0, 0);
      // each tile's int and scale MFMAs back to back, so tile 0's convert + fma wait on two
      // MFMAs rather than four; in the fp32-output kernel a scheduling barrier also keeps the
      // compiler from moving them (measured: t32k down -4%, t2k -2.7%; the SwiGLU kernel is
      // faster without it)
      if (EPI == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4 * NG; ++i)  // registers 4g..4g+3 hold rows 8g..8g+7
        acc0[i] = fmaf((float)I0[i], S0[i], acc0[i]);
#pragma unroll
      for (int i = 0; i < 4 * NG; ++i)
        acc1[i] = fmaf((float)I1[i], S1[i], acc1[i]);
    }
  };

  // EPI 0: n-tile j's fp32 rows, then the accumulators cleared for the next n-tile.  The rows are
  // stored non-temporally, as nothing reads them before the combine, after the whole launch
  // (measured: down -0.5% / -1.1% and the combine that reads them -6% at T = 8,192 / 32,768).
  // In the default roles register i holds row 32 wr + 8 (i / 4) + 4 half + i % 4: its address
  // is a wavefront-uniform row base (scalar arithmetic) plus one 32-bit lane offset that does
  // not change with i (4 half rows and the lane's column; below 2^31 bytes as 64 rows x n_out
  // floats are); column tile ct1 lies 32 floats after ct0.
  auto store_f32 = [&](int j) {
    const int wu = wave_id();  // wr and ct0 as scalars
    if (kByColumn) {  // column tile wu of row tiles 0 and 1 (32 rows further down)
      const char* ob = reinterpret_cast<const char*>(p.out) +
                       ((size_t)row0 * p.n_out + n0 + j * kRowsN + 32 * wu) * 4;
      const uint32_t off = (uint32_t)((4 * half * p.n_out + l32) * 4);
      const size_t tile1 = (size_t)32 * p.n_out * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);
        const char* rb = ob + (size_t)(8 * (i >> 2) + (i & 3)) * p.n_out * 4 + off;
        if (row < nrows) __builtin_nontemporal_store(acc0[i], (float*)rb);
        if (NG1 > 0 && 32 + row < nrows)
          __builtin_nontemporal_store(acc1[i], (float*)(rb + tile1));
        acc0[i] = 0.0f;
        acc1[i] = 0.0f;
      }
      return;
    }
    const char* ob =
        reinterpret_cast<const char*>(p.out) +
        ((size_t)(row0 + 32 * (wu >> 1)) * p.n_out + n0 + j * kRowsN + 64 * (wu & 1)) * 4;
    const uint32_t off = (uint32_t)((4 * half * p.n_out + l32) * 4);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * wr + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < nrows) {
        float* dst = (float*)(ob + (size_t)(8 * (i >> 2) + (i & 3)) * p.n_out * 4 + off);
        __builtin_nontemporal_store(acc0[i], dst);
        __builtin_nontemporal_store(acc1[i], dst + 32);
      }
      acc0[i] = 0.0f;
      acc1[i] = 0.0f;
    }
  };

  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the previous tile
  __builtin_amdgcn_s_barrier();        // ... and every other wave's, before the ring refills
  issue(L0, 0, 0);
  if (EPI == 0) {
    // Sweep: the step computing stage cs of n-tile cj.  Each step waits until this wavefront's
    // loads of its stage are done and, at the barrier, every wavefront's (which also means every
    // wavefront is done with the previous stage, whose buffer `fill` then receives the next),
    // then its MFMAs.  An n-tile finished by the previous step is stored first, before this
    // step's loads are issued: the next wait (vector memory counts stores and loads alike) then
    // finds the stores done as well, after a whole stage of MFMAs.
    int cj = 0, cs = 0;
    auto step = [&](const StageBuf<WT>& cur, StageBuf<WT>& fill) {
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
      __builtin_amdgcn_s_barrier();
      if (cs == 0 && cj > 0 && live) store_f32(cj - 1);
      const int s = cs;
      int nj = cj, ns = cs + 1;
      if (ns == nstages) {
        ns = 0;
        ++nj;
      }
      if (nj < nsweep) issue(fill, nj, ns);
      cj = nj;
      cs = ns;
      if (live) math(s, cur);
    };
    const int total = nstages * nsweep;
    for (int t = 0; t < total; t += 2) {  // stage t + 1 goes into the other buffer
      step(L0, L1);
      if (t + 1 < total) step(L1, L0);
    }
    if (live) store_f32(nsweep - 1);
    return;
  }
  // One n-tile: the same steps without the sweep's bookkeeping.  The two buffers are distinct
  // LDS objects used with fixed roles per unrolled step, so the compiler can tell the reads of
  // one from the loads into the other and keeps the loads in flight.
  auto step = [&](int s, const StageBuf<WT>& cur, StageBuf<WT>& fill) {
    __builtin_amdgcn_s_waitcnt(vm_imm(0));
    __builtin_amdgcn_s_barrier();
    if (s + 1 < nstages) issue(fill, 0, s + 1);
    if (live) math(s, cur);
  };
  for (int s0 = 0; s0 < nstages; s0 += 2) {
    step(s0, L0, L1);
    if (s0 + 1 < nstages) step(s0 + 1, L1, L0);
  }
  if (EPI == 2) return;
  // EPI 1: every wavefront is past its last stage: the ring becomes scratch
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  if (!live) return;

  // EPI == 1: h = silu(g) * u, then q8_1 along F.  A lane holds one feature of 16 rows; the
  // wavefront's 32 x 32 block of h goes through LDS so that two lanes own one row's block of 32
  // features (16 each): the block's max and sum then take one exchange between the two lanes,
  // and each lane stores its 16 q bytes with one 16-byte write.  silu uses the hardware exp and
  // reciprocal (h only has to be accurate); the quantisation of h is the exact q8_1 arithmetic.
  float* xs = reinterpret_cast<float*>(&L0) + wave * 32 * 32;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // the accumulators hold 2g and 2u (the doubled scale products): the halving goes into the
    // exponent's argument and one final quarter, each exact, so h = silu(g) * u as if halved
    // first
    const float g2 = acc0[i], u2 = acc1[i];
    xs[(8 * (i >> 2) + 4 * half + (i & 3)) * 32 + l32] =
        g2 * __builtin_amdgcn_rcpf(1.0f + __expf(-0.5f * g2)) * u2 * 0.25f;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  const int rr = lane & 31, part = lane >> 5;  // row of the wavefront's 32, 16-feature half
  float v[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 t = *reinterpret_cast<const float4*>(xs + rr * 32 + 16 * part + 4 * k);
    v[4 * k] = t.x, v[4 * k + 1] = t.y, v[4 * k + 2] = t.z, v[4 * k + 3] = t.w;
  }
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) am = fmaxf(am, fabsf(v[k]));
  am = fmaxf(am, __shfl_xor(am, 32));
  const bool nz = am > 0.0f;
  const float d = am / 127.0f;
  uint32_t qw[4];
  int S = q8_pack16(v, d, nz, qw);
  S += __shfl_xor(S, 32);
  const int row = 32 * wr + rr;
  if (row < nrows) {
    const int fb = (n0 + 32 * wc) / kQK;  // block index along F
    const size_t h_row_bytes = (size_t)(p.n_out / kDs4Vals) * kDs4Bytes;
    const size_t hoff = (size_t)(fb >> 2) * kDs4Bytes;
    uint8_t* dst = reinterpret_cast<uint8_t*>(p.out) + (size_t)(row0 + row) * h_row_bytes;
    *reinterpret_cast<uint4*>(dst + hoff + 16 + (fb & 3) * 32 + 16 * part) =
        make_uint4(qw[0], qw[1], qw[2], qw[3]);
    if (part == 0) {
      const uint32_t hdr =
          !nz                ? 0u
          : WT == kWtQ8_0D4 ? __float_as_uint(d)
                            : (f2h(d) | (q8_1_scale_bits(d, S) << 16));
      *reinterpret_cast<uint32_t*>(dst + hoff + (fb & 3) * 4) = hdr;
    }
    if (p.debug_h != nullptr) {
      float* dh = p.debug_h + (size_t)(row0 + row) * p.n_out + n0 + 32 * wc + 16 * part;
#pragma unroll
      for (int k = 0; k < 16; ++k) dh[k] = v[k];
    }
  }
}

// The dispatcher hands workgroups to the 8 XCDs round-robin in launch order, and each XCD has
// its own L2.  The live (m-tile, n-tile) pairs are therefore renumbered so that XCD x receives
// one contiguous run of them, m-tile major: the n-tiles of an m-tile share its activation rows
// in one L2, and consecutive m-tiles of an expert share its weights there.
constexpr int kXcds = 8;

// The launch is one-dimensional (the host keeps n-tiles x m-tiles within the grid's x limit).
template <int WT, int EPI>
__global__ __launch_bounds__(256, (wg_per_cu<WT, EPI>())) void mmq_layer_kernel(MmqProblem p) {
  __shared__ Ring<WT> ring;
  const int ntl = p.n_tiles_n;
  const int live = ntl * (p.tile_count > 0 ? p.tile_count : *p.n_tiles);
  const int id = blockIdx.x;
  if (id >= live) return;
  const int xcd = id % kXcds;
  const int work = xcd * (live / kXcds) + min(xcd, live % kXcds) + id / kXcds;
  const int mt = work / ntl;
  const MTile t = p.tiles[mt];
  if (p.skip != nullptr && p.skip[t.expert] != 0) return;  // the host computes this expert
  const uint8_t* W = p.mat_offset + (p.w_off != nullptr
                                         ? p.wbase + p.w_off[t.expert]
                                         : p.wbase + (size_t)t.ordinal * p.pos_stride);
  // The direct-to-LDS loads need 16-byte aligned weights.  Group positions always are; a packed
  // pool's expert offset may not be (a caller error): the tile is then skipped and counted in
  // the status word the caller can read.
  if (((uintptr_t)W & 15) != 0) {
    if (threadIdx.x == 0 && p.misaligned != nullptr) atomicAdd(p.misaligned, 1);
    return;
  }
  // the wavefront's live 8-row groups: an expert's last tile skips the epilogue of its
  // padding rows (the MFMAs still cover all 32)
  const int nh = t.nrows - 32 * (wave_id() >> 1);
  const int ng = (EPI == 2 || nh <= 0 || nh >= 32) ? 4 : (nh + 7) / 8;
  // EPI 0: the workgroup's n-tiles kSweep * (work % ntl) onwards, at most kSweep of them
  const int nt0 = EPI == 0 ? (work % ntl) * kSweep : work % ntl;
  const int nsw = EPI == 0 ? min(kSweep, p.n_out / kRowsN - nt0) : 1;
  if (WT == 1 && EPI == 0) {  // by column: the live 8-row groups of both row tiles
    const int nr = t.nrows;
    if (nr > 56)
      mmq_tile<WT, EPI, 4, 4>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else if (nr > 48)
      mmq_tile<WT, EPI, 4, 3>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else if (nr > 40)
      mmq_tile<WT, EPI, 4, 2>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else if (nr > 32)
      mmq_tile<WT, EPI, 4, 1>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else if (nr > 24)
      mmq_tile<WT, EPI, 4, 0>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else if (nr > 16)
      mmq_tile<WT, EPI, 3, 0>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else if (nr > 8)
      mmq_tile<WT, EPI, 2, 0>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    else
      mmq_tile<WT, EPI, 1, 0>(ring.buf[0], ring.buf[1], p, W, t.row0, nr, nt0, nsw);
    return;
  }
  if (ng == 4)
    mmq_tile<WT, EPI, 4>(ring.buf[0], ring.buf[1], p, W, t.row0, t.nrows, nt0, nsw);
  else if (ng == 3)
    mmq_tile<WT, EPI, 3>(ring.buf[0], ring.buf[1], p, W, t.row0, t.nrows, nt0, nsw);
  else if (ng == 2)
    mmq_tile<WT, EPI, 2>(ring.buf[0], ring.buf[1], p, W, t.row0, t.nrows, nt0, nsw);
  else
    mmq_tile<WT, EPI, 1>(ring.buf[0], ring.buf[1], p, W, t.row0, t.nrows, nt0, nsw);
}

template <int WT, int EPI>
__global__ __launch_bounds__(256, 2) void mmq_group_kernel(MmqProblem p) {
  __shared__ Ring<WT> ring;
  const int j = blockIdx.z;
  const int e = p.experts[j];
  const int r0 = p.offsets[e], cnt = p.offsets[e + 1] - r0;
  const uint8_t* W = p.wbase + (size_t)j * p.pos_stride + p.mat_offset;
  for (int m = blockIdx.y; m * kRowsM < cnt; m += gridDim.y)
    mmq_tile<WT, EPI>(ring.buf[0], ring.buf[1], p, W,
                      r0 + m * kRowsM, min(kRowsM, cnt - m * kRowsM), blockIdx.x);
}

template <int WT, int EPI>
hipError_t launch_typed(const MmqProblem& p, hipStream_t s) {
  const int ntiles = EPI == 1 ? p.n_out / 64 : p.n_out / kRowsN;
  if (p.tiles != nullptr) {
    MmqProblem q = p;
    q.n_tiles_n = EPI == 0 ? (ntiles + kSweep - 1) / kSweep : ntiles;  // workgroups per m-tile
    const long long n = (long long)q.n_tiles_n * (p.tile_count > 0 ? p.tile_count : p.max_tiles);
    if (n > kMaxGridX) return hipErrorInvalidConfiguration;   // refused by the ABI's checks
    mmq_layer_kernel<WT, EPI><<<dim3((unsigned)n), 256, 0, s>>>(q);
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
  if (p.wtype == kWtQ8_0D4) {
    if (p.epilogue == 0) return launch_typed<kWtQ8_0D4, 0>(p, s);
    if (p.epilogue == 1) return launch_typed<kWtQ8_0D4, 1>(p, s);
    return launch_typed<kWtQ8_0D4, 2>(p, s);
  }
  if (p.epilogue == 0) return launch_typed<1, 0>(p, s);
  if (p.epilogue == 1) return launch_typed<1, 1>(p, s);
  return launch_typed<1, 2>(p, s);
}

}  // namespace moe
