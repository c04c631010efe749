// The layer's workspace layout and the small host helpers shared by the C ABI's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "internal.hpp"
#include "moe_prefill.h"

namespace moe {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }
inline bool valid_wtype(int wt) { return wt == MOE_Q8_0 || wt == MOE_Q4_1 || wt == MOE_Q8_0_D4; }
static_assert(MOE_Q8_0_D4 == kWtQ8_0D4 && MOE_QUANT_PER_ROW == kQuantPerRow &&
                  MOE_QUANT_D4 == kQuantD4,
              "the ABI's constants and the kernels' agree");

// Region offsets of the layer's workspace (each 256-byte aligned).
struct Layout {
  size_t status, hist, counts, offsets, src, slot, order, nactive, ntiles, tiles, q8x, groups, hq8, dm;
  size_t group_stride, total;
  int max_tiles;
};

inline bool make_layout(int T, int H, int F, int E, int K, int wt, Layout* L) {
  if (T < 1 || K < 1 || E < 1 || H < 128 || H % 128 != 0 || F < 128 || F % 128 != 0 ||
      !valid_wtype(wt))
    return false;
  const size_t R = (size_t)T * K;
  if (R > ((size_t)1 << 30)) return false;  // the row indices are int32
  const size_t eb = moe_expert_bytes(H, F, wt);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L->status = take(8);
  L->hist = take(maps_hist_bytes((int)R, E));
  L->counts = take((size_t)E * 4);
  L->offsets = take((size_t)(E + 1) * 4);
  L->src = take(R * 4);
  L->slot = take(R * 4);
  L->order = take((size_t)E * 4);
  L->nactive = take(4);
  L->ntiles = take(4);
  L->max_tiles = max_mtiles((int)R, E, kMmqRows);
  L->tiles = take((size_t)L->max_tiles * sizeof(MTile));
  L->q8x = take(R * moe_q8_1_row_bytes(H));
  L->group_stride = align_up(eb, 256);
  L->groups = take((size_t)E * L->group_stride);
  L->hq8 = take(R * moe_q8_1_row_bytes(F));
  L->dm = take(R * (size_t)H * 4);
  L->total = o;
  return true;
}

// The map outputs of the layer, in its workspace at `base`.
inline MapsOut layer_maps(uint8_t* base, const Layout& L) {
  auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
  return MapsOut{I32(L.counts), I32(L.offsets), I32(L.src), I32(L.slot), I32(L.order),
                 I32(L.nactive), I32(L.hist), reinterpret_cast<MTile*>(base + L.tiles),
                 I32(L.ntiles), kMmqRows, I32(L.status), I32(L.status) + 1};
}

// The layer's argument checks (moe_prefill_layer and its streamed form), in the order the
// statuses are documented; fills *L on MOE_OK.
inline int check_layer_args(const float* x, int T, int H, int F, int E, int K,
                            const int32_t* topk_idx, const float* topk_w, int wtype,
                            size_t expert_bytes, int group_size, int ring_start, const void* ws,
                            size_t ws_bytes, const float* out, Layout* L) {
  if (!x || !topk_idx || !topk_w || !ws || !out) return MOE_EINVAL;
  if (T < 1 || K < 1 || E < 1 || K > E || group_size < 1 || group_size > MOE_MAX_GROUP ||
      ring_start < 0 || ring_start >= E)
    return MOE_EINVAL;
  if (!valid_wtype(wtype)) return MOE_EUNSUPPORTED;
  if (H < 128 || H % 128 != 0 || F < 128 || F % 128 != 0 || E > MOE_MAX_E || K > MOE_MAX_K)
    return MOE_EUNSUPPORTED;
  if ((long long)T * K > (1LL << 30)) return MOE_EUNSUPPORTED;
  if (expert_bytes != moe_expert_bytes(H, F, wtype)) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 256)) return MOE_EINVAL;
  if (!make_layout(T, H, F, E, K, wtype, L)) return MOE_EINVAL;
  if (mmq_layer_workgroups(F, H, L->max_tiles) > kMaxGridX) return MOE_EUNSUPPORTED;
  if (!mmq_offsets_fit(F, H, wtype, true) || !mmq_offsets_fit(H, F, wtype, false))
    return MOE_EUNSUPPORTED;
  if (ws_bytes < L->total) return MOE_EWORKSPACE;
  return MOE_OK;
}

}  // namespace moe
