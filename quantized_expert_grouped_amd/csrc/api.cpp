// C ABI of libmoe_prefill.so: argument checks, the layer's workspace layout and its launch
// schedule.  Every compute step runs in the gfx950 kernels of this directory; nothing here
// computes on the host or synchronises with the device (the opt-in stage profiler aside).
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "internal.hpp"
#include "layout.hpp"
#include "moe_prefill.h"

namespace {

using namespace moe;

// ---- opt-in stage profiler -------------------------------------------------------------------
constexpr int kEvPerCall = MOE_N_STAGES + 1;
std::mutex g_prof_mu;
std::vector<hipEvent_t> g_prof_ev;
int g_prof_calls = 0;
int g_prof_done = 0;

void destroy_events() {
  for (hipEvent_t e : g_prof_ev) (void)hipEventDestroy(e);
  g_prof_ev.clear();
  g_prof_calls = g_prof_done = 0;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or type";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    case MOE_ENOMEM: return "host memory or threads could not be obtained";
    default: return "unknown status";
  }
}

size_t moe_block_bytes(int wtype) {
  return wtype == MOE_Q8_0 || wtype == MOE_Q8_0_D4 ? 34 : wtype == MOE_Q4_1 ? 20 : 0;
}

size_t moe_expert_bytes(int H, int F, int wtype) {
  if (H < 32 || F < 32 || !valid_wtype(wtype)) return 0;
  return ((size_t)2 * F * (H / 32) + (size_t)H * (F / 32)) * moe_block_bytes(wtype);
}

size_t moe_q8_1_row_bytes(int n) { return n > 0 ? (size_t)(n / 128) * 144 : 0; }

size_t moe_build_maps_workspace_size(int T, int K, int E) {
  if (T < 1 || K < 1 || E < 1 || (long long)T * K > (1LL << 30)) return 0;
  return kMapsHistAt + align_up(maps_hist_bytes(T * K, E), 256);
}

size_t moe_workspace_size(int T, int H, int F, int E, int K, int wtype, int group_size) {
  Layout L;
  if (group_size < 1 || group_size > MOE_MAX_GROUP) return 0;
  if (!make_layout(T, H, F, E, K, wtype, &L)) return 0;
  return L.total;
}

size_t moe_workspace_offset(int which, int T, int H, int F, int E, int K, int wtype,
                            int group_size) {
  Layout L;
  if (group_size < 1 || group_size > MOE_MAX_GROUP || !make_layout(T, H, F, E, K, wtype, &L))
    return (size_t)-1;
  switch (which) {
    case MOE_WS_COUNTS: return L.counts;
    case MOE_WS_OFFSETS: return L.offsets;
    case MOE_WS_SRC: return L.src;
    case MOE_WS_SLOT: return L.slot;
    case MOE_WS_ORDER: return L.order;
    case MOE_WS_NACTIVE: return L.nactive;
    case MOE_WS_Q8X: return L.q8x;
    case MOE_WS_GROUPS: return L.groups;
    case MOE_WS_HQ8: return L.hq8;
    case MOE_WS_DM: return L.dm;
    case MOE_WS_GROUP_STRIDE: return L.group_stride;
    case MOE_WS_STATUS: return L.status;
    default: return (size_t)-1;
  }
}

int moe_route_topk(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                   void* stream) {
  if (!logits || !idx || !w || T < 1 || E < 1 || K < 1 || K > E) return MOE_EINVAL;
  if (E > MOE_MAX_E || K > MOE_MAX_K) return MOE_EUNSUPPORTED;
  return status_of(launch_route_topk(logits, T, E, K, idx, w, as_stream(stream)));
}

int moe_build_maps(const int32_t* topk_idx, int T, int K, int E, int ring_start, int32_t* counts,
                   int32_t* offsets, int32_t* src, int32_t* slot, int32_t* order,
                   int32_t* n_active, void* ws, size_t ws_bytes, void* stream) {
  if (!topk_idx || !counts || !offsets || !src || !slot || !order || !n_active || !ws)
    return MOE_EINVAL;
  if (T < 1 || K < 1 || E < 1 || K > E || ring_start < 0 || ring_start >= E) return MOE_EINVAL;
  if ((long long)T * K > (1LL << 30)) return MOE_EUNSUPPORTED;
  if (E > MOE_MAX_E) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe_build_maps_workspace_size(T, K, E)) return MOE_EWORKSPACE;
  uint8_t* w = static_cast<uint8_t*>(ws);
  MapsOut o{counts, offsets, src, slot, order, n_active,
            reinterpret_cast<int32_t*>(w + kMapsHistAt), nullptr, nullptr, kMmqRows,
            reinterpret_cast<int32_t*>(w), nullptr};
  return status_of(launch_build_maps(topk_idx, T, K, E, ring_start, o, as_stream(stream)));
}

int moe_build_maps_noalloc(const int32_t* topk_idx, int T, int K, int E, int ring_start,
                           int32_t* counts, int32_t* offsets, int32_t* src, int32_t* slot,
                           int32_t* order, int32_t* n_active, int32_t* n_invalid, void* stream) {
  static_assert(MOE_NOALLOC_MAX_ROUTES == kNoAllocMaxRoutes && MOE_MAX_E == kNoAllocMaxE,
                "the header's limits are the scratch array's");
  static_assert(MOE_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "the stated scratch size");
  if (!topk_idx || !counts || !offsets || !src || !slot || !order || !n_active)
    return MOE_EINVAL;
  if (T < 1 || K < 1 || E < 1 || K > E || ring_start < 0 || ring_start >= E) return MOE_EINVAL;
  if ((long long)T * K > MOE_NOALLOC_MAX_ROUTES || E > MOE_MAX_E) return MOE_EUNSUPPORTED;
  uint8_t* sc = nullptr;
  if (noalloc_scratch(&sc) != hipSuccess) return MOE_EHIP;
  MapsOut o{counts, offsets, src, slot, order, n_active,
            reinterpret_cast<int32_t*>(sc + kMapsHistAt), nullptr, nullptr, kMmqRows,
            n_invalid != nullptr ? n_invalid : reinterpret_cast<int32_t*>(sc), nullptr};
  return status_of(launch_build_maps(topk_idx, T, K, E, ring_start, o, as_stream(stream)));
}

int moe_quantize_scatter_q8_1(const float* x, int T, int H, int K, const int32_t* slot,
                              const int32_t* src, int mode, void* q8, void* stream) {
  if (!x || !q8 || T < 1 || K < 1 || mode < 0 || mode > (MOE_QUANT_PER_ROW | MOE_QUANT_D4))
    return MOE_EINVAL;
  const bool per_row = (mode & MOE_QUANT_PER_ROW) != 0;
  if ((!per_row && !slot) || (per_row && !src)) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(q8, 16)) return MOE_EINVAL;
  if (H < 128 || H % 128 != 0 || K > MOE_MAX_K) return MOE_EUNSUPPORTED;
  if ((long long)T * K > (1LL << 30)) return MOE_EUNSUPPORTED;
  return status_of(launch_quantize(x, T, H, K, slot, src, mode, static_cast<uint8_t*>(q8),
                                   as_stream(stream)));
}

int moe_gather_group(const void* const* src_ptrs, int n, size_t expert_bytes, void* group_buf,
                     int first_pos, size_t pos_stride, void* stream) {
  if (!src_ptrs || !group_buf || n < 1 || n > MOE_MAX_GROUP || first_pos < 0 ||
      first_pos + n > MOE_MAX_GROUP || expert_bytes == 0)
    return MOE_EINVAL;
  if (n > 1 && pos_stride < expert_bytes) return MOE_EINVAL;
  GatherPtrs p{};
  for (int j = 0; j < n; ++j) {
    if (!src_ptrs[j]) return MOE_EINVAL;
    p.src[j] = static_cast<const uint8_t*>(src_ptrs[j]);
  }
  return status_of(launch_gather_group(p, n, expert_bytes, static_cast<uint8_t*>(group_buf),
                                       first_pos, pos_stride, as_stream(stream)));
}

int moe_gather_group_mmq(const void* const* src_ptrs, int n, int wtype, int H, int F,
                         void* group_buf, int first_pos, size_t pos_stride, void* stream) {
  if (!src_ptrs || !group_buf || n < 1 || n > MOE_MAX_GROUP || first_pos < 0 ||
      first_pos + n > MOE_MAX_GROUP)
    return MOE_EINVAL;
  if (!valid_wtype(wtype)) return MOE_EUNSUPPORTED;
  if (H < 128 || H % 128 != 0 || F < 128 || F % 128 != 0) return MOE_EUNSUPPORTED;
  if (n > 1 && pos_stride < moe_expert_bytes(H, F, wtype)) return MOE_EINVAL;
  GatherPtrs p{};
  for (int j = 0; j < n; ++j) {
    if (!src_ptrs[j]) return MOE_EINVAL;
    p.src[j] = static_cast<const uint8_t*>(src_ptrs[j]);
  }
  return status_of(launch_gather_group_mmq(p, n, wtype, H, F, static_cast<uint8_t*>(group_buf),
                                           first_pos, pos_stride, as_stream(stream)));
}

int moe_mmq_grouped(int wtype, const void* group_buf, size_t pos_stride, size_t mat_offset,
                    int n_out, int k_in, const int32_t* group_experts, int n_group,
                    const int32_t* offsets, int E, const void* act_q8, int epilogue, void* out,
                    float* debug_h, void* stream) {
  if (!group_buf || !group_experts || !offsets || !act_q8 || !out) return MOE_EINVAL;
  if (n_group < 1 || n_group > MOE_MAX_GROUP || E < 1) return MOE_EINVAL;
  if (epilogue < MOE_EPI_F32 || epilogue > MOE_EPI_I32_BLOCKDOTS) return MOE_EINVAL;
  if (!valid_wtype(wtype)) return MOE_EUNSUPPORTED;
  if (n_out < 128 || n_out % 128 != 0 || k_in < 128 || k_in % 128 != 0) return MOE_EUNSUPPORTED;
  if (!mmq_offsets_fit(n_out, k_in, wtype, epilogue == MOE_EPI_SWIGLU_Q8_1))
    return MOE_EUNSUPPORTED;
  if (!aligned(group_buf, 16) || pos_stride % 16 != 0 || mat_offset % 16 != 0 ||
      !aligned(act_q8, 16) || !aligned(out, 4) || !aligned(debug_h, 4))
    return MOE_EINVAL;
  MmqProblem p{};
  p.wtype = wtype;
  p.epilogue = epilogue;
  p.wbase = static_cast<const uint8_t*>(group_buf);
  p.pos_stride = pos_stride;
  p.mat_offset = mat_offset;
  p.n_out = n_out;
  p.k_in = k_in;
  p.act = static_cast<const uint8_t*>(act_q8);
  p.out = out;
  p.debug_h = debug_h;
  p.offsets = offsets;
  p.n_group = n_group;
  for (int j = 0; j < n_group; ++j) {
    if (group_experts[j] < 0 || group_experts[j] >= E) return MOE_EINVAL;
    p.experts[j] = group_experts[j];
  }
  return status_of(launch_mmq(p, as_stream(stream)));
}

int moe_combine(const float* Dm, const int32_t* slot, const float* topk_w, int T, int K, int H,
                float* out, void* stream) {
  if (!Dm || !slot || !topk_w || !out || T < 1 || K < 1 || H < 4) return MOE_EINVAL;
  if (!aligned(Dm, 16) || !aligned(out, 16)) return MOE_EINVAL;
  if (H % 4 != 0 || K > MOE_MAX_K) return MOE_EUNSUPPORTED;
  return status_of(launch_combine(Dm, slot, topk_w, T, K, H, out, as_stream(stream)));
}

int moe_prefill_layer(const float* x, int T, int H, int F, int E, int K, const int32_t* topk_idx,
                      const float* topk_w, int wtype, const void* pool, const int64_t* expert_off,
                      size_t expert_bytes, int group_size, int ring_start, void* ws,
                      size_t ws_bytes, float* out, void* stream) {
  if (!pool || !expert_off) return MOE_EINVAL;
  Layout L;
  const int rc = check_layer_args(x, T, H, F, E, K, topk_idx, topk_w, wtype, expert_bytes,
                                  group_size, ring_start, ws, ws_bytes, out, &L);
  if (rc != MOE_OK) return rc;

  hipStream_t s = as_stream(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  MapsOut mo = layer_maps(base, L);

  hipEvent_t* ev = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_done < g_prof_calls) ev = &g_prof_ev[(size_t)(g_prof_done++) * kEvPerCall];
  }
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], s);
  };

  hipError_t e;
  mark(0);
  if ((e = launch_build_maps(topk_idx, T, K, E, ring_start, mo, s)) != hipSuccess) return MOE_EHIP;
  mark(1);
  if ((e = launch_quantize(x, T, H, K, mo.slot, mo.src, act_mode_bits(wtype), base + L.q8x,
                           s)) != hipSuccess)
    return MOE_EHIP;
  mark(2);
  if ((e = launch_gather_all_mmq(static_cast<const uint8_t*>(pool), expert_off, mo.order,
                                 mo.n_active, E, group_size, wtype, H, F, base + L.groups,
                                 L.group_stride, s)) != hipSuccess)
    return MOE_EHIP;
  mark(3);
  MmqProblem gu{};
  gu.wtype = wtype;
  gu.epilogue = MOE_EPI_SWIGLU_Q8_1;
  gu.wbase = base + L.groups;
  gu.pos_stride = L.group_stride;
  gu.mat_offset = 0;
  gu.n_out = F;
  gu.k_in = H;
  gu.act = base + L.q8x;
  gu.out = base + L.hq8;
  gu.tiles = mo.tiles;
  gu.n_tiles = mo.n_tiles;
  gu.max_tiles = L.max_tiles;
  gu.misaligned = reinterpret_cast<int32_t*>(base + L.status) + 1;
  if ((e = launch_mmq(gu, s)) != hipSuccess) return MOE_EHIP;
  mark(4);
  MmqProblem dn = gu;
  dn.epilogue = MOE_EPI_F32;
  dn.mat_offset = (size_t)2 * F * (H / 32) * moe_block_bytes(wtype);
  dn.n_out = H;
  dn.k_in = F;
  dn.act = base + L.hq8;
  dn.out = base + L.dm;
  if ((e = launch_mmq(dn, s)) != hipSuccess) return MOE_EHIP;
  mark(5);
  if ((e = launch_combine(reinterpret_cast<const float*>(base + L.dm), mo.slot, topk_w, T, K, H,
                          out, s)) != hipSuccess)
    return MOE_EHIP;
  mark(6);
  return MOE_OK;
}

int moe_prefill_layer_packed(const float* x, int T, int H, int F, int E, int K,
                             const int32_t* topk_idx, const float* topk_w, int wtype,
                             const void* packed_pool, const int64_t* expert_off,
                             size_t expert_bytes, int ring_start, void* ws, size_t ws_bytes,
                             float* out, void* stream) {
  if (!packed_pool || !expert_off) return MOE_EINVAL;
  Layout L;
  const int rc = check_layer_args(x, T, H, F, E, K, topk_idx, topk_w, wtype, expert_bytes,
                                  MOE_MAX_GROUP, ring_start, ws, ws_bytes, out, &L);
  if (rc != MOE_OK) return rc;
  if (!aligned(packed_pool, 16)) return MOE_EINVAL;

  hipStream_t s = as_stream(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  MapsOut mo = layer_maps(base, L);
  if (launch_build_maps(topk_idx, T, K, E, ring_start, mo, s) != hipSuccess ||
      launch_quantize(x, T, H, K, mo.slot, mo.src, act_mode_bits(wtype), base + L.q8x, s) !=
          hipSuccess)
    return MOE_EHIP;
  MmqProblem gu{};
  gu.wtype = wtype;
  gu.epilogue = MOE_EPI_SWIGLU_Q8_1;
  gu.wbase = static_cast<const uint8_t*>(packed_pool);
  gu.w_off = expert_off;
  gu.mat_offset = 0;
  gu.n_out = F;
  gu.k_in = H;
  gu.act = base + L.q8x;
  gu.out = base + L.hq8;
  gu.tiles = mo.tiles;
  gu.n_tiles = mo.n_tiles;
  gu.max_tiles = L.max_tiles;
  gu.misaligned = reinterpret_cast<int32_t*>(base + L.status) + 1;
  MmqProblem dn = gu;
  dn.epilogue = MOE_EPI_F32;
  dn.mat_offset = (size_t)2 * F * (H / 32) * moe_block_bytes(wtype);
  dn.n_out = H;
  dn.k_in = F;
  dn.act = base + L.hq8;
  dn.out = base + L.dm;
  if (launch_mmq(gu, s) != hipSuccess || launch_mmq(dn, s) != hipSuccess ||
      launch_combine(reinterpret_cast<const float*>(base + L.dm), mo.slot, topk_w, T, K, H, out,
                     s) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

int moe_profile_begin(int n_calls) {
  if (n_calls < 1 || n_calls > 100000) return MOE_EINVAL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  destroy_events();
  try {
    g_prof_ev.assign((size_t)n_calls * kEvPerCall, nullptr);
  } catch (...) {
    return MOE_ENOMEM;
  }
  for (hipEvent_t& e : g_prof_ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      destroy_events();
      return MOE_EHIP;
    }
  }
  g_prof_calls = n_calls;
  g_prof_done = 0;
  return MOE_OK;
}

int moe_profile_end(float* ms, int max_calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int n = g_prof_done;
  int rc = n;
  if (n > 0) {
    if (hipEventSynchronize(g_prof_ev[(size_t)n * kEvPerCall - 1]) != hipSuccess) rc = MOE_EHIP;
    for (int c = 0; c < n && c < max_calls && rc >= 0 && ms; ++c)
      for (int st = 0; st < MOE_N_STAGES; ++st) {
        float v = 0.0f;
        if (hipEventElapsedTime(&v, g_prof_ev[(size_t)c * kEvPerCall + st],
                                g_prof_ev[(size_t)c * kEvPerCall + st + 1]) != hipSuccess)
          rc = MOE_EHIP;
        ms[(size_t)c * MOE_N_STAGES + st] = v;
      }
  }
  destroy_events();
  return rc;
}

}  // extern "C"
