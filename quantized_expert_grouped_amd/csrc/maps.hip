// a1  Token -> row maps.  "#1368 prefill: quantize each token's MoE input once and scatter it to
// its k rows", opening section: src_dev names each of the T*K rows' source, and token t's k-th row
// is slot[t*K+k], the inverse of src_dev.  Rows are grouped by expert id and keep ascending t*K+k
// inside an expert, so the result is unique: a stable counting sort.
//
// Three launches, no host synchronisation:
//   hist     one wavefront per chunk of kMapChunk entries: a per-chunk histogram in LDS.
//   scan     one workgroup: per-expert exclusive prefix over chunks, counts, offsets, the ring
//            order of the experts with rows and the m-tile list of the MMQ.
//   scatter  one wavefront per chunk, 64 entries at a time in index order: ballots over the bits
//            of the expert id give each lane its equal-id peers, mbcnt its rank among them, so
//            rows are placed in ascending t*K+k without atomics.
// An entry with an id outside [0, E) (a caller error) is counted as one more expert, E, that
// sorts after every real one: such entries take the rows offsets[E] .. T*K-1, in index order,
// with src = -1 for those rows and slot = -1 for the entries, so every later step can skip
// them (the quantiser writes no row for them, the combine adds nothing for them), and the scan
// stores their number in the status word at the front of the scratch buffer.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

// The scratch of moe_build_maps_noalloc: the status words and the per-chunk histograms for up to
// kNoAllocMaxRoutes routes of up to MOE_MAX_E experts, held by each GPU the library runs on until
// the process ends.  In host code this name is only a stand-in for the symbol: the device
// address is what hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[moe::kNoAllocScratchBytes];

namespace moe {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kMaxE = 2048;   // largest E the single-workgroup scan holds in LDS

__global__ __launch_bounds__(256) void maps_hist_kernel(const int32_t* __restrict__ idx, int R,
                                                         int E, int nchunks,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int32_t lds_hist[];  // [4][E+1]: bin E counts the out-of-range ids
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wave;
  const int NB = E + 1;
  int32_t* h = lds_hist + wave * NB;
  for (int e = lane; e < NB; e += 64) h[e] = 0;
  __syncthreads();
  if (chunk < nchunks) {
    // every step's ids are loaded before the first is counted: one load latency per chunk
    const int base = chunk * kMapChunk;
    int ids[kMapChunk / 64];
#pragma unroll
    for (int it = 0; it < kMapChunk / 64; ++it) {
      const int i = base + it * 64 + lane;
      ids[it] = i < R ? idx[i] : -1;
    }
#pragma unroll
    for (int it = 0; it < kMapChunk / 64; ++it) {
      const int e = ids[it];
      if (base + it * 64 + lane < R) atomicAdd(&h[(unsigned)e < (unsigned)E ? e : E], 1);
    }
  }
  __syncthreads();
  if (chunk < nchunks)
    for (int e = lane; e < NB; e += 64) hist[(size_t)chunk * NB + e] = h[e];
}

// Exclusive prefix of n ints (n <= 2 * kScanThreads) held as lds[0..n), in place; returns the
// total to every thread.
__device__ int block_exclusive_scan(int32_t* lds, int n, int32_t* wave_sums) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int a = i0 < n ? lds[i0] : 0;
  const int b = i1 < n ? lds[i1] : 0;
  int v = a + b;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int nw = kScanThreads / 64;
    int s = lane < nw ? wave_sums[lane] : 0;
    int si = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(si, off);
      if (lane >= off) si += o;
    }
    if (lane < nw) wave_sums[lane] = si - s;  // exclusive wave offsets
    if (lane == nw - 1) wave_sums[nw] = si;   // total
  }
  __syncthreads();
  const int excl = wave_sums[wave] + incl - v;
  const int total = wave_sums[kScanThreads / 64];
  if (i0 < n) lds[i0] = excl;
  if (i1 < n) lds[i1] = excl + a;
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kScanThreads) void maps_scan_kernel(
    int E, int nchunks, int ring_start, int32_t* __restrict__ hist, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ order, int32_t* __restrict__ n_active,
    MTile* __restrict__ tiles, int32_t* __restrict__ n_tiles, int tile_rows,
    int32_t* __restrict__ n_invalid, int32_t* __restrict__ mmq_skips) {
  __shared__ int32_t s_cnt[kMaxE];   // rows of expert e
  __shared__ int32_t s_off[kMaxE];   // first row of expert e
  __shared__ int32_t s_act[kMaxE];   // ring position j -> ordinal among the experts with rows
  __shared__ int32_t s_til[kMaxE];   // ring position j -> its first m-tile
  __shared__ int32_t s_wsum[kScanThreads / 64 + 1];
  const int tid = threadIdx.x;
  // per expert: exclusive prefix over chunks (in place), and the count; a batch of chunks'
  // loads is issued before any of them is used, so the chain waits once per batch
  // (bin E, the out-of-range ids, gets its prefix too: the scatter places them after the rest)
  constexpr int kBatch = 16;
  const int NB = E + 1;
  for (int e = tid; e < NB; e += kScanThreads) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = c0 + u < nchunks ? hist[(size_t)(c0 + u) * NB + e] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (c0 + u < nchunks) hist[(size_t)(c0 + u) * NB + e] = run;
        run += v[u];
      }
    }
    if (e == E) {  // the status words: out-of-range ids, and the MMQ's skip count cleared
      *n_invalid = run;
      if (mmq_skips != nullptr) *mmq_skips = 0;
      continue;
    }
    s_cnt[e] = run;
    s_off[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int R = block_exclusive_scan(s_off, E, s_wsum);
  for (int e = tid; e < E; e += kScanThreads) offsets[e] = s_off[e];
  if (tid == 0) offsets[E] = R;
  // ring order of the experts with rows, and their m-tiles
  for (int j = tid; j < E; j += kScanThreads) {
    const int c = s_cnt[(ring_start + j) % E];
    s_act[j] = c > 0 ? 1 : 0;
    s_til[j] = (c + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  const int nact = block_exclusive_scan(s_act, E, s_wsum);
  const int nt = block_exclusive_scan(s_til, E, s_wsum);
  for (int j = tid; j < E; j += kScanThreads) {
    const int e = (ring_start + j) % E;
    if (s_cnt[e] > 0) order[s_act[j]] = e;
  }
  // The m-tile list, every thread taking tiles t, t + 1024, ...: tile t belongs to the last ring
  // position j whose first tile s_til[j] is at most t (positions without rows own no tile and
  // share their successor's s_til, so that j holds rows).  One expert can own thousands of tiles
  // (skewed routing), so the tiles are spread over the threads rather than the experts.
  if (tiles != nullptr) {
    for (int t = tid; t < nt; t += kScanThreads) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_til[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      const int e = (ring_start + lo) % E;
      const int m = t - s_til[lo];
      MTile tl;
      tl.ordinal = s_act[lo];
      tl.expert = e;
      tl.row0 = s_off[e] + m * tile_rows;
      tl.nrows = min(tile_rows, s_cnt[e] - m * tile_rows);
      tiles[t] = tl;
    }
  }
  if (tid == 0) {
    *n_active = nact;
    if (n_tiles != nullptr) *n_tiles = nt;
  }
}

__global__ __launch_bounds__(256) void maps_scatter_kernel(const int32_t* __restrict__ idx, int R,
                                                            int E, int nbits, int nchunks,
                                                            const int32_t* __restrict__ hist,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ src,
                                                            int32_t* __restrict__ slot) {
  extern __shared__ int32_t lds_ctr[];  // [4][E+1]: each wavefront's next free row per expert
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wave;
  const bool live = chunk < nchunks;
  const int NB = E + 1;
  int32_t* ctr = lds_ctr + wave * NB;
  if (live)   // offsets[E] = the rows of real experts: bin E's rows follow them
    for (int e = lane; e < NB; e += 64) ctr[e] = offsets[e] + hist[(size_t)chunk * NB + e];
  __syncthreads();
  if (!live) return;
  // From here each wavefront touches only its own counters; LDS operations of one wavefront
  // complete in issue order, so no further barrier is needed.
  const int base = chunk * kMapChunk;
  int ids[kMapChunk / 64];  // every step's ids loaded up front: one load latency per chunk
#pragma unroll
  for (int it = 0; it < kMapChunk / 64; ++it) {
    const int i = base + it * 64 + lane;
    ids[it] = i < R ? idx[i] : -1;
  }
#pragma unroll
  for (int it = 0; it < kMapChunk / 64; ++it) {
    const int i = base + it * 64 + lane;
    const bool present = i < R;
    const bool valid = (unsigned)ids[it] < (unsigned)E;
    const int e = valid ? ids[it] : E;   // out-of-range ids: bin E (nbits covers it)
    uint64_t peers = ballot(present);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank = mbcnt(peers);   // equal-id lanes below this one
    const int cnt = __popcll(peers);
    if (present) {
      const int r = ctr[e] + rank;
      src[r] = valid ? i : -1;
      slot[i] = valid ? r : -1;
      if (rank == 0) ctr[e] = r + cnt;   // after every lane's read above (one instruction stream)
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_build_maps(const int32_t* idx, int T, int K, int E, int ring_start,
                             const MapsOut& o, hipStream_t s) {
  const int R = T * K;
  const int nchunks = map_chunks(R);
  const int blocks = (nchunks + 3) / 4;
  const size_t lds = (size_t)4 * (E + 1) * sizeof(int32_t);
  maps_hist_kernel<<<blocks, 256, lds, s>>>(idx, R, E, nchunks, o.hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  maps_scan_kernel<<<1, kScanThreads, 0, s>>>(E, nchunks, ring_start, o.hist, o.counts, o.offsets,
                                              o.order, o.n_active, o.tiles, o.n_tiles,
                                              o.tile_rows, o.n_invalid, o.mmq_skips);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  maps_scatter_kernel<<<blocks, 256, lds, s>>>(idx, R, E, nbits, nchunks, o.hist, o.offsets,
                                               o.src, o.slot);
  return hipGetLastError();
}

// This device's address of `scratch`, looked up once per device (with that device current) and
// kept; every later call on the device uses the kept address.
hipError_t noalloc_scratch(uint8_t** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = static_cast<uint8_t*>(ptr[dev]);
  return hipSuccess;
}

}  // namespace moe
