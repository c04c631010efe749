// Host-side launchers of the gfx950 kernels.  Each returns hipSuccess or the launch error; the
// C ABI in api.cpp validates arguments before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- a0 routing ----------------------------------------------------------------------------
hipError_t launch_route_topk(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                             hipStream_t s);

// ---- a1 maps (counting sort in chunks of kMapChunk entries, one wavefront per chunk) --------
constexpr int kMapChunk = 1024;
inline int map_chunks(int R) { return (R + kMapChunk - 1) / kMapChunk; }

// Tile list entry of the layer's MMQ: rows row0 .. row0+nrows-1 of active expert `ordinal`.
struct MTile {
  int32_t ordinal;
  int32_t expert;
  int32_t row0;
  int32_t nrows;
};

struct MapsOut {
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* src;       // [R]
  int32_t* slot;      // [R]
  int32_t* order;     // [E]
  int32_t* n_active;  // [1]
  int32_t* hist;      // [chunks x (E+1)] scratch
  MTile* tiles;       // [max tiles] or nullptr
  int32_t* n_tiles;   // [1] or nullptr
  int tile_rows;      // rows per m-tile
  int32_t* n_invalid; // [1]: routes whose expert id is outside [0, E)
  int32_t* mmq_skips; // [1] or nullptr: set to 0 (the layer's MMQ then counts skipped work)
};
// Scratch of moe_build_maps: the status words in the first 256 bytes, then hist.
constexpr size_t kMapsHistAt = 256;
inline size_t maps_hist_bytes(int R, int E) { return (size_t)map_chunks(R) * (E + 1) * 4; }

// moe_build_maps_noalloc: its scratch is a static device array of fixed size (maps.hip).
constexpr int kNoAllocMaxRoutes = 1 << 19;   // T*K
constexpr int kNoAllocMaxE = 2048;
constexpr size_t kNoAllocScratchBytes =
    kMapsHistAt + (((size_t)((kNoAllocMaxRoutes + kMapChunk - 1) / kMapChunk) * (kNoAllocMaxE + 1) *
                    4 + 255) / 256) * 256;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(uint8_t** out);
hipError_t launch_build_maps(const int32_t* idx, int T, int K, int E, int ring_start,
                             const MapsOut& o, hipStream_t s);
inline int max_mtiles(int R, int E, int tile_rows) { return R / tile_rows + (E < R ? E : R); }

// ---- a2 quantise ----------------------------------------------------------------------------
constexpr int kQuantPerRow = 1;  // mode bit: the per-row form (else scatter)
constexpr int kQuantD4 = 2;      // mode bit: the D4 layout (else DS4)
// The weight type that reads D4 activations (Q8_0 weights).
constexpr int kWtQ8_0D4 = 2;
inline int act_mode_bits(int wtype) { return wtype == kWtQ8_0D4 ? kQuantD4 : 0; }
hipError_t launch_quantize(const float* x, int T, int H, int K, const int32_t* slot,
                           const int32_t* src, int mode, uint8_t* q8, hipStream_t s);

// ---- a3 gather ------------------------------------------------------------------------------
struct GatherPtrs {
  const uint8_t* src[16];
};
hipError_t launch_gather_group(const GatherPtrs& p, int n, size_t bytes, uint8_t* dst,
                               int first_pos, size_t pos_stride, hipStream_t s);
// The same copy, each expert written in the MMQ layout the grouped matmul reads (64-row tiles of
// 4-block stages, headers first; the raw expert's size).
hipError_t launch_gather_group_mmq(const GatherPtrs& p, int n, int wtype, int H, int F,
                                   uint8_t* dst, int first_pos, size_t pos_stride,
                                   hipStream_t s);
// Every group of the layer in one launch: active expert i (ring order) -> dst + i*stride, in
// the MMQ layout.
hipError_t launch_gather_all_mmq(const uint8_t* pool, const int64_t* expert_off,
                                 const int32_t* order, const int32_t* n_active, int max_slots,
                                 int group_size, int wtype, int H, int F, uint8_t* dst,
                                 size_t stride, hipStream_t s);

// ---- a4..a6 MMQ -----------------------------------------------------------------------------
constexpr int kMmqRows = 64;  // rows per m-tile

struct MmqProblem {
  int wtype;
  int epilogue;           // 0 f32, 1 swiglu->q8_1, 2 int32 block dots
  const uint8_t* wbase;   // group buffer(s), or the packed pool when w_off is set
  size_t pos_stride;      // bytes between expert positions
  const int64_t* w_off;   // if set: expert e's MMQ-layout bytes at wbase + w_off[e]
  size_t mat_offset;      // bytes from an expert's start to the matrix
  int n_out;
  int k_in;
  const uint8_t* act;     // q8_1 rows of k_in values
  void* out;
  float* debug_h;
  // layer form: device tile list; tile_count > 0 takes that many tiles from `tiles` (a count
  // the host knows), otherwise *n_tiles of them with a grid sized for max_tiles
  const MTile* tiles;
  const int32_t* n_tiles;
  int max_tiles;
  int tile_count;
  int n_tiles_n;          // workgroups per m-tile (set by the launcher)
  int32_t* misaligned;    // layer form, packed pool: count of m-tiles skipped (or nullptr)
  const uint8_t* skip;    // layer form: skip[e] != 0 -> expert e's tiles are not computed
                          // (the host computes them), or nullptr
  // group form: positions j < n_group hold experts[j], rows from offsets
  const int32_t* offsets;
  int experts[16];
  int n_group;
};
hipError_t launch_mmq(const MmqProblem& p, hipStream_t s);
// The MMQ addresses a weight matrix's bytes by 32-bit offsets from the matrix's start (the gate
// and up matrices from the gate's): they must stay below 4 GiB.
inline bool mmq_offsets_fit(long long n_out, long long k_in, int wtype, bool gate_and_up) {
  const long long bb = wtype == 1 ? 20 : 34;
  return (gate_and_up ? 2 : 1) * n_out * (k_in / 32) * bb < (1LL << 32);
}
// The layer's MMQ launch is one-dimensional: n-tiles x m-tiles workgroups must fit in x.
constexpr long long kMaxGridX = 0x7fffffffLL;
inline long long mmq_layer_workgroups(int n_out_gu, int n_out_dn, int max_tiles) {
  const long long a = (long long)(n_out_gu / 64) * max_tiles;    // gate/up: 64 features a tile
  // down: 128 output columns a tile, up to 4 tiles a workgroup
  const long long b = (long long)((n_out_dn / 128 + 3) / 4) * max_tiles;
  return a > b ? a : b;
}

// ---- a7 combine -----------------------------------------------------------------------------
hipError_t launch_combine(const float* Dm, const int32_t* slot, const float* w, int T, int K,
                          int H, float* out, hipStream_t s);
// Dm[dst[j]] = rows[j] for j < n (fp32 rows of H values): the host's rows into their places.
hipError_t launch_scatter_rows(const float* rows, const int32_t* dst, int n, int H, float* Dm,
                               hipStream_t s);

}  // namespace moe
