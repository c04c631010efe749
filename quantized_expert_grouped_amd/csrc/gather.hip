// a3  The group gather.  "#439 prefill: a group's expert gathers in one launch", "What": one
// launch copies up to 16 experts into the MMQ group buffer (blockIdx.y = expert), and the buffer
// ends up byte for byte as one copy per expert leaves it; the page's test checks batches of 1 to
// 16, positions starting mid-group and the unaligned / odd-size fallback.  "Prompt path: an MMQ
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
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kGatherThreads = 512;
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

// ---- the MMQ layout -------------------------------------------------------------------------
// The grouped matmul stages its weights as tiles of 64 rows by 128 values (4 blocks), so the
// group buffer holds every matrix as those tile-stages, each one contiguous: for tile j, stage
// t and row i < 64 (matrix row 64j+i), the row's blocks 4t..4t+3 sit at byte
// ((j * stages + t) * 64 + i) * G, G = 4 * block bytes, with the blocks' headers first:
//   Q4_1, G = 80 : (d, m) of the 4 blocks, then each block's 16 packed bytes in two halves:
//                  byte 8h + i holds element 16h + i (low nibble) and 16h + 8 + i (high), so
//                  elements 16h..16h+15 sit in one 8-byte half (raw byte j: elements j, j + 16)
//   Q8_0, G = 136: d of the 4 blocks, then their q[32]
// The expert keeps its order (gate | up | down) and its size.  A 64-row tile is one contiguous
// run in the raw expert and one in the packed expert, so a workgroup moves a tile's rows for
// up to Pack<WT>::kStages stages: it reads the rows' bytes into LDS with wide coalesced loads
// and writes the tile-stages out, also coalesced, picking each output word from LDS.  Both the
// pool reads and the packed writes are non-temporal: each byte is moved once.  Q4_1 items span
// 8 stages (640 bytes of a row: whole 128-byte lines, so no line is fetched by two items);
// Q8_0 items span 4 (544 bytes; 8 would leave too few workgroups per CU).

constexpr int kLoadBatch = 8;  // loads a lane has in flight when it fills the LDS

template <int WT>
struct Pack {
  static constexpr int kG = WT == 1 ? 80 : 136;
  static constexpr int kStages = WT == 1 ? 8 : 4;
  static constexpr int kLds = 64 * kStages * kG;
};

// Q8_0: byte offset, within a row's 4-block group in the raw layout, of the low half of output
// word k of the packed group (the high half is 2 bytes further).  Every such offset is even.
__device__ __forceinline__ int q8_0_word_src(int k) {
  if (k < 2) return 68 * k;  // (d_{2k}, d_{2k+1}) live at 68k and 68k + 34
  return 34 * ((k - 2) >> 3) + 2 + 4 * ((k - 2) & 7);
}

__device__ __forceinline__ uint32_t q8_0_word(const uint8_t* grp, int k) {
  const int o = q8_0_word_src(k);
  const uint16_t* h = reinterpret_cast<const uint16_t*>(grp);
  const uint32_t lo = h[o >> 1];
  const uint32_t hi = h[(k < 2 ? o + 34 : o + 2) >> 1];
  return lo | (hi << 16);
}

// Q4_1: 16-byte piece c < 5 of a packed group from the raw group (4-byte aligned): c = 0 the
// blocks' (d, m), c >= 1 block c-1's packed bytes in the half order.  With the raw words
// x0..x3 (bytes 0-3, 4-7, 8-11, 12-15), the half-0 bytes take the low nibbles of x0 | x1 and,
// above them, those of x2 | x3; the half-1 bytes the high nibbles of the same words.
__device__ __forceinline__ v4u q4_1_piece(const uint8_t* grp, int c) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(grp);
  if (c == 0) return (v4u){w[0], w[5], w[10], w[15]};  // (d, m) of block u at byte 20u
  const uint32_t* x = w + 5 * (c - 1) + 1;             // qs of block c-1 at byte 20(c-1) + 4
  const uint32_t m = 0x0f0f0f0fu;
  return (v4u){(x[0] & m) | ((x[2] & m) << 4), (x[1] & m) | ((x[3] & m) << 4),
               ((x[0] >> 4) & m) | (x[2] & ~m), ((x[1] >> 4) & m) | (x[3] & ~m)};
}

// One work item: tile `tile` of matrix `mat` (0 gate, 1 up, 2 down), stages t0 .. t0+ns-1.
template <int WT>
__device__ __forceinline__ void pack_item(const uint8_t* __restrict__ src_e,
                                          uint8_t* __restrict__ dst_e, int H, int F, int item,
                                          uint8_t* lds) {
  constexpr int G = Pack<WT>::kG;
  const int sh = H / 128, sf = F / 128;
  constexpr int kPS = Pack<WT>::kStages;
  const int cg = (sh + kPS - 1) / kPS, cd = (sf + kPS - 1) / kPS;
  const int items_gu = (F / 64) * cg;
  int tile, chunk, nS;
  size_t mat_off;
  if (item < 2 * items_gu) {
    const int mat = item / items_gu, r = item % items_gu;
    tile = r / cg, chunk = r % cg, nS = sh;
    mat_off = (size_t)mat * F * sh * G;
  } else {
    const int r = item - 2 * items_gu;
    tile = r / cd, chunk = r % cd, nS = sf;
    mat_off = (size_t)2 * F * sh * G;
  }
  const size_t row_bytes = (size_t)nS * G;
  const int t0 = chunk * kPS, ns = min(kPS, nS - t0);
  const int seg = ns * G;  // bytes of one row in this item
  const uint8_t* s = src_e + mat_off + (size_t)tile * 64 * row_bytes + (size_t)t0 * G;
  uint8_t* d = dst_e + mat_off + ((size_t)tile * nS + t0) * 64 * G;
  const int tid = threadIdx.x;

  // rows -> LDS (row i at i * seg), in the widest pieces the alignment allows; each lane issues
  // up to kLoadBatch loads before it waits for the first, so that enough bytes are in flight
  // per CU to cover the HBM latency
  if (((uintptr_t)s & 15) == 0 && (row_bytes & 15) == 0 && (seg & 15) == 0) {
    const int per_row = seg / 16, total = 64 * per_row;
    for (int q0 = tid; q0 < total; q0 += kLoadBatch * kGatherThreads) {
      v4u r[kLoadBatch];
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int q = q0 + u * kGatherThreads;
        if (q < total)
          r[u] = __builtin_nontemporal_load(
              reinterpret_cast<const v4u*>(s + (q / per_row) * row_bytes + 16 * (q % per_row)));
      }
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int q = q0 + u * kGatherThreads;
        if (q < total) *reinterpret_cast<v4u*>(lds + 16 * q) = r[u];
      }
    }
  } else if (((uintptr_t)s & 7) == 0 && (row_bytes & 7) == 0) {
    const int per_row = seg / 8, total = 64 * per_row;
    for (int q0 = tid; q0 < total; q0 += kLoadBatch * kGatherThreads) {
      v2u r[kLoadBatch];
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int q = q0 + u * kGatherThreads;
        if (q < total)
          r[u] = __builtin_nontemporal_load(
              reinterpret_cast<const v2u*>(s + (q / per_row) * row_bytes + 8 * (q % per_row)));
      }
#pragma unroll
      for (int u = 0; u < kLoadBatch; ++u) {
        const int q = q0 + u * kGatherThreads;
        if (q < total) *reinterpret_cast<v2u*>(lds + 8 * q) = r[u];
      }
    }
  } else {
    for (int q = tid; q < 64 * seg; q += kGatherThreads) {
      const int i = q / seg, k = q % seg;
      lds[q] = s[i * row_bytes + k];
    }
  }
  __syncthreads();

  // LDS -> the ns tile-stages (one contiguous run of ns * 64 * G bytes), 16 bytes per lane
  constexpr int words = G / 4;  // per packed group
  const int total16 = ns * 64 * G / 16;
  const bool wide = ((uintptr_t)d & 15) == 0;
  for (int q = tid; q < total16; q += kGatherThreads) {
    uint32_t v[4];
    if (WT == 1) {  // a group is 5 whole pieces
      const int st = q / (64 * 5), qq = q % (64 * 5);
      const v4u p = q4_1_piece(lds + (qq / 5) * seg + st * G, qq % 5);
      v[0] = p[0], v[1] = p[1], v[2] = p[2], v[3] = p[3];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int w = 4 * q + u;                    // word of the run
        const int st = w / (64 * words), ww = w % (64 * words);
        const int i = ww / words, k = ww % words;   // row of the tile, word of its group
        v[u] = q8_0_word(lds + i * seg + st * G, k);
      }
    }
    if (wide) {
      __builtin_nontemporal_store((v4u){v[0], v[1], v[2], v[3]}, reinterpret_cast<v4u*>(d) + q);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int b = 0; b < 4; ++b) d[16 * q + 4 * u + b] = (uint8_t)(v[u] >> (8 * b));
    }
  }
  __syncthreads();  // the LDS is reused by the next item of this workgroup
}

int pack_items(int wtype, int H, int F) {
  const int sh = H / 128, sf = F / 128;
  const int ps = wtype == 1 ? Pack<1>::kStages : Pack<0>::kStages;
  return 2 * (F / 64) * ((sh + ps - 1) / ps) + (H / 64) * ((sf + ps - 1) / ps);
}

template <int WT>
__global__ __launch_bounds__(kGatherThreads) void gather_mmq_group_kernel(
    GatherPtrs p, int H, int F, uint8_t* __restrict__ dst, int first_pos, size_t pos_stride) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[Pack<WT>::kLds];
  const int j = blockIdx.y;
  pack_item<WT>(p.src[j], dst + (size_t)(first_pos + j) * pos_stride, H, F, blockIdx.x, lds);
}

template <int WT>
__global__ __launch_bounds__(kGatherThreads) void gather_mmq_all_kernel(
    const uint8_t* __restrict__ pool, const int64_t* __restrict__ expert_off,
    const int32_t* __restrict__ order, const int32_t* __restrict__ n_active, int H, int F,
    uint8_t* __restrict__ dst, size_t stride) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[Pack<WT>::kLds];
  // Workgroups reach the 8 XCDs round-robin; renumber the live ones so that each XCD moves a
  // contiguous run of (expert, item) pairs, keeping the neighbouring slices of a tile, which share
  // cache lines at their edges, in one L2.  The runs split the routed positions' items, not the
  // grid (sized for every expert): split over the grid, the XCDs whose runs fell past the routed
  // positions had nothing to move (skewed routing left half the chip idle).  (blockIdx.z = group
  // and blockIdx.y = position in it, as in one group's launch.)
  const int items = gridDim.x;
  const int live = *n_active * items;
  const int id = blockIdx.x + items * (blockIdx.y + gridDim.y * blockIdx.z);
  if (id >= live) return;
  const int xcd = id % 8;
  const int work = xcd * (live / 8) + min(xcd, live % 8) + id / 8;
  const int pos = work / items;
  pack_item<WT>(pool + expert_off[order[pos]], dst + (size_t)pos * stride, H, F, work % items,
                lds);
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

hipError_t launch_gather_group_mmq(const GatherPtrs& p, int n, int wtype, int H, int F,
                                   uint8_t* dst, int first_pos, size_t pos_stride,
                                   hipStream_t s) {
  const dim3 grid(pack_items(wtype, H, F), n);
  if (wtype == 1)
    gather_mmq_group_kernel<1><<<grid, kGatherThreads, 0, s>>>(p, H, F, dst, first_pos, pos_stride);
  else
    gather_mmq_group_kernel<0><<<grid, kGatherThreads, 0, s>>>(p, H, F, dst, first_pos, pos_stride);
  return hipGetLastError();
}

hipError_t launch_gather_all_mmq(const uint8_t* pool, const int64_t* expert_off,
                                 const int32_t* order, const int32_t* n_active, int max_slots,
                                 int group_size, int wtype, int H, int F, uint8_t* dst,
                                 size_t stride, hipStream_t s) {
  const int groups = (max_slots + group_size - 1) / group_size;
  const dim3 grid(pack_items(wtype, H, F), group_size, groups);
  if (wtype == 1)
    gather_mmq_all_kernel<1><<<grid, kGatherThreads, 0, s>>>(pool, expert_off, order, n_active, H,
                                                             F, dst, stride);
  else
    gather_mmq_all_kernel<0><<<grid, kGatherThreads, 0, s>>>(pool, expert_off, order, n_active, H,
                                                             F, dst, stride);
  return hipGetLastError();
}

}  // namespace moe
