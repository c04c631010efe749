// Streamed walk of the layer ([G2] "What changes"; the per-expert form it replaces is in its
// opening section): experts that are not resident in device memory are copied from a pinned host
// arena into a ring of device slots on a copy stream, while the compute stream gathers each batch
// of routed experts after one wait, releases the batch's slots with one event, and runs a group's
// MMQs once its last batch is gathered.
//
// The schedule is planned on the host after the routing sync (the routed experts and their row
// counts read back from the maps) and then enqueued in plan order, so every event a copy waits on
// has been recorded before that copy is enqueued, and every copy a batch waits for was enqueued
// on the (in-order) copy stream before the batch's wait.  That is the whole deadlock argument: a
// copy only ever waits on batches planned before it, and such a batch only waits on copies
// enqueued before it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <memory>
#include <new>
#include <thread>
#include <vector>

#include "cpu_share.hpp"
#include "internal.hpp"
#include "layout.hpp"
#include "moe_prefill.h"

using namespace moe;

namespace {

constexpr int kEvents = MOE_WALK_EVENTS;
constexpr int kMaxE = MOE_MAX_E;
enum { kOpCopy = 1, kOpGather = 2, kOpMmq = 3 };
enum { kWhyGroup = 0, kWhySkip = 1, kWhySlot = 2, kWhyOne = 3, kWhyHost = 4 };
enum { kResident = 0, kStreamed = 1, kHost = 2 };  // an expert's state in the plan
enum {
  kStCopies, kStBytes, kStBatches, kStWaits, kStCopyWaits, kStSkipFlush, kStSlotFlush, kStMmq,
  kStSyncs, kStTransfers, kStHostExperts, kStHostRows, kStHostUs, kStSharePpm, kStGpuNs,
  kStHostNs
};
static_assert(kStHostNs + 1 == MOE_WALK_NSTATS, "the header's counter list");

struct Op {
  int32_t v[6];
};

// The walk over ring entries ring_start, ring_start+1, ... (mod E).  A routed entry takes the
// next group position; a streamed one first takes the next ring slot (round robin) for its copy,
// which waits on the event of that slot's last reader.  The open batch is launched when its group
// is complete, at a skipped entry, when the next slot is one the open batch holds, or after every
// expert (one-expert mode); a group's MMQ record follows its last batch.  An expert the host
// computes (state kHost) keeps its position but is neither copied nor gathered: the open batch is
// launched before it, since a batch is a run of consecutive positions.
int plan(const int32_t* counts, const int32_t* order, int n_active, int E, int ring_start,
         const uint8_t* streamed, int G, int n_slots, int flags, int32_t* used_of,
         int32_t* cursor, int32_t* next_event, std::vector<Op>& ops) {
  if (!counts || !order || !streamed || !used_of || !cursor || !next_event) return MOE_EINVAL;
  if (E < 1 || E > kMaxE || ring_start < 0 || ring_start >= E || n_active < 0 || n_active > E ||
      G < 1 || G > MOE_MAX_GROUP || n_slots < 1 || *cursor < 0 || *cursor >= n_slots ||
      *next_event < 0 || *next_event >= kEvents ||
      (flags & ~(MOE_WALK_GATHER_ONE | MOE_WALK_NO_SKIP_FLUSH | MOE_WALK_MMQ_PER_GROUP)) != 0)
    return MOE_EINVAL;
  // order must be the routed entries in ring order
  int j = 0;
  for (int i = 0; i < E; ++i) {
    const int e = (ring_start + i) % E;
    if (counts[e] < 0) return MOE_EINVAL;
    if (counts[e] == 0) continue;
    if (j >= n_active || order[j] != e) return MOE_EINVAL;
    ++j;
  }
  if (j != n_active) return MOE_EINVAL;
  for (int s = 0; s < n_slots; ++s)
    if (used_of[s] < -1 || used_of[s] >= kEvents) return MOE_EINVAL;
  for (int e = 0; e < E; ++e)
    if (streamed[e] > kHost) return MOE_EINVAL;

  ops.clear();
  std::vector<char> held(n_slots, 0);  // the slot's copy belongs to the open batch
  std::vector<int> open_slots;
  int open_first = 0, open_n = 0, open_waits = 0;
  auto flush = [&](int why) {
    if (open_n == 0) return;
    const int ev = *next_event;
    ops.push_back({{kOpGather, open_first, open_n, open_waits, ev, why}});
    for (int s : open_slots) {
      used_of[s] = ev;
      held[s] = 0;
    }
    open_slots.clear();
    open_n = open_waits = 0;
    *next_event = (ev + 1) % kEvents;
  };
  const bool one = (flags & MOE_WALK_GATHER_ONE) != 0;
  int pos = 0, group_first = 0;
  for (int i = 0; i < E && pos < n_active; ++i) {
    const int e = (ring_start + i) % E;
    if (counts[e] == 0) {
      if (!(flags & MOE_WALK_NO_SKIP_FLUSH)) flush(kWhySkip);
      continue;
    }
    if (streamed[e] == kHost) {
      flush(kWhyHost);
      ++pos;
      if (pos % G == 0 || pos == n_active) {
        ops.push_back({{kOpMmq, (pos - 1) / G, group_first, pos - group_first, 0, 0}});
        group_first = pos;
      }
      continue;
    }
    if (streamed[e] == kStreamed) {
      const int s = *cursor;
      if (held[s]) flush(kWhySlot);
      ops.push_back({{kOpCopy, pos, e, s, used_of[s], 0}});
      held[s] = 1;
      open_slots.push_back(s);
      open_waits = 1;
      *cursor = (s + 1) % n_slots;
    }
    if (open_n == 0) open_first = pos;
    ++open_n;
    ++pos;
    if (pos % G == 0 || pos == n_active) {
      flush(one ? kWhyOne : kWhyGroup);
      ops.push_back({{kOpMmq, (pos - 1) / G, group_first, pos - group_first, 0, 0}});
      group_first = pos;
    } else if (one) {
      flush(kWhyOne);
    }
  }
  return (int)ops.size();
}

}  // namespace

namespace {

// The CPU share of a walk: what the host computes, the buffers it stages through, and the two
// per-expert rates the automatic share is set from.
struct HostShare {
  double share = 0;           // fixed share, or < 0: automatic
  double cur = 0.25;          // the share the next call hands the host
  int max_tokens = 0, T_max = 0, H = 0, rows_max = 0;
  std::unique_ptr<CpuPool> pool;
  std::vector<CpuScratch> scratch;
  float* h_x = nullptr;       // pinned [T_max x H]: the layer input
  int32_t* h_src = nullptr;   // pinned [T_max * MOE_MAX_K]: src
  float* h_rows = nullptr;    // pinned [rows_max x H]: the host's rows
  int32_t* h_dst = nullptr;   // pinned [rows_max]: each staged row's row in Dm
  uint8_t* h_skip = nullptr;  // pinned [MOE_MAX_E]: 1 = the host computes the expert
  float* d_rows = nullptr;    // device [rows_max x H]
  int32_t* d_dst = nullptr;   // device [rows_max]
  uint8_t* d_skip = nullptr;  // device [MOE_MAX_E]
  hipEvent_t t0 = nullptr, t1 = nullptr;  // around the GPU's expert work (timing)
  bool timed = false;         // t0/t1 were recorded by the previous call
  int timed_experts = 0;      // streamed experts the GPU computed in that call
  double gpu_ns = 0, host_ns = 0;  // measured time per expert, 0 = not yet
};

void free_host_share(HostShare* h) {
  if (!h) return;
  h->pool.reset();
  if (h->t0) (void)hipEventDestroy(h->t0);
  if (h->t1) (void)hipEventDestroy(h->t1);
  for (void* p : {(void*)h->h_x, (void*)h->h_src, (void*)h->h_rows, (void*)h->h_dst,
                  (void*)h->h_skip})
    if (p) (void)hipHostFree(p);
  for (void* p : {(void*)h->d_rows, (void*)h->d_dst, (void*)h->d_skip})
    if (p) (void)hipFree(p);
  h->h_x = h->h_rows = h->d_rows = nullptr;
  h->h_src = h->h_dst = h->d_dst = nullptr;
  h->h_skip = h->d_skip = nullptr;
  h->t0 = h->t1 = nullptr;
}

}  // namespace

struct moe_walk {
  uint8_t* ring = nullptr;
  int n_slots = 0;
  size_t stride = 0;
  hipStream_t copy = nullptr;
  hipEvent_t used[kEvents] = {};
  hipEvent_t copied = nullptr;  // recorded after a batch's last copy, waited on at once
  hipEvent_t routed = nullptr;  // the routing read-back has landed
  int32_t* host = nullptr;      // pinned: counts [kMaxE], order [kMaxE], n_active
  std::vector<int32_t> used_of;
  int32_t cursor = 0, next_event = 0;
  int64_t stats[MOE_WALK_NSTATS] = {};
  std::vector<Op> ops;
  std::vector<uint8_t> streamed;
  std::vector<int32_t> slot_of, tile_first;
  std::unique_ptr<HostShare> share;  // the CPU share, when configured
};

namespace {

void release(moe_walk* w) {
  // the copies, then every gather that read a ring slot (each batch's event follows its
  // gather), so that the caller may free the ring once this returns
  if (w->copy) (void)hipStreamSynchronize(w->copy);
  for (hipEvent_t& e : w->used)
    if (e) (void)hipEventSynchronize(e);
  for (hipEvent_t& e : w->used)
    if (e) (void)hipEventDestroy(e);
  if (w->copied) (void)hipEventDestroy(w->copied);
  if (w->routed) (void)hipEventDestroy(w->routed);
  if (w->copy) (void)hipStreamDestroy(w->copy);
  if (w->host) (void)hipHostFree(w->host);
  free_host_share(w->share.get());
  delete w;
}

}  // namespace

extern "C" {

int moe_walk_create(void* ring, int n_slots, size_t slot_stride, moe_walk** walk) {
  if (!ring || !walk || n_slots < 1 || slot_stride == 0 || slot_stride % 256 != 0 ||
      (uintptr_t)ring % 256 != 0)
    return MOE_EINVAL;
  moe_walk* w = new (std::nothrow) moe_walk;
  if (!w) return MOE_ENOMEM;
  w->ring = static_cast<uint8_t*>(ring);
  w->n_slots = n_slots;
  w->stride = slot_stride;
  try {  // host memory: no exception crosses the C boundary
    w->used_of.assign(n_slots, -1);
  } catch (...) {
    release(w);
    return MOE_ENOMEM;
  }
  bool ok = hipStreamCreateWithFlags(&w->copy, hipStreamNonBlocking) == hipSuccess;
  for (int i = 0; ok && i < kEvents; ++i)
    ok = hipEventCreateWithFlags(&w->used[i], hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&w->copied, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&w->routed, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&w->host), (2 * kMaxE + 1) * sizeof(int32_t),
                           hipHostMallocDefault) == hipSuccess;
  if (!ok) {
    release(w);
    return MOE_EHIP;
  }
  *walk = w;
  return MOE_OK;
}

int moe_walk_destroy(moe_walk* walk) {
  if (walk) release(walk);
  return MOE_OK;
}

int moe_walk_cpu_share(moe_walk* walk, double share, int max_tokens, int threads, int max_T,
                       int H, int max_rows) {
  if (!walk || !(share <= 1.0) || max_tokens < 0 || threads < 0) return MOE_EINVAL;
  if (share == 0.0) {
    free_host_share(walk->share.get());
    walk->share.reset();
    return MOE_OK;
  }
  if (max_T < 1 || H < 128 || H % 128 != 0 || max_rows < 1 ||
      (long long)max_T * MOE_MAX_K > (1LL << 30) || (long long)max_rows * H > (1LL << 40))
    return MOE_EINVAL;
  std::unique_ptr<HostShare> hs(new (std::nothrow) HostShare);
  if (!hs) return MOE_ENOMEM;
  hs->share = share < 0 ? -1.0 : share;
  hs->cur = share < 0 ? 0.25 : share;
  hs->max_tokens = max_tokens;
  hs->T_max = max_T;
  hs->H = H;
  hs->rows_max = max_rows;
  if (threads == 0) threads = std::max(1u, std::thread::hardware_concurrency());
  const size_t xb = (size_t)max_T * H * 4, rb = (size_t)max_rows * H * 4;
  bool ok = hipHostMalloc(reinterpret_cast<void**>(&hs->h_x), xb, hipHostMallocDefault) ==
                hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&hs->h_src), (size_t)max_T * MOE_MAX_K * 4,
                          hipHostMallocDefault) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&hs->h_rows), rb, hipHostMallocDefault) ==
                hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&hs->h_dst), (size_t)max_rows * 4,
                          hipHostMallocDefault) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&hs->h_skip), kMaxE, hipHostMallocDefault) ==
                hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&hs->d_rows), rb) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&hs->d_dst), (size_t)max_rows * 4) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&hs->d_skip), kMaxE) == hipSuccess &&
            hipEventCreate(&hs->t0) == hipSuccess && hipEventCreate(&hs->t1) == hipSuccess;
  if (!ok) {
    free_host_share(hs.get());
    return MOE_EHIP;
  }
  try {  // threads and their scratch (no exception crosses the C boundary)
    hs->pool.reset(new CpuPool(threads));
    hs->scratch.resize(threads);
  } catch (...) {
    free_host_share(hs.get());
    return MOE_ENOMEM;
  }
  free_host_share(walk->share.get());
  walk->share = std::move(hs);
  return MOE_OK;
}

int moe_walk_stats(const moe_walk* walk, int64_t* stats, int n) {
  if (!walk || !stats || n < 0) return MOE_EINVAL;
  for (int i = 0; i < n && i < MOE_WALK_NSTATS; ++i) stats[i] = walk->stats[i];
  return MOE_OK;
}

int moe_walk_plan(const int32_t* counts, const int32_t* order, int n_active, int E,
                  int ring_start, const uint8_t* streamed, int group_size, int n_slots, int flags,
                  int32_t* used_of, int32_t* cursor, int32_t* next_event, int32_t* ops,
                  int max_ops) {
  if (!ops || max_ops < 0) return MOE_EINVAL;
  try {
    std::vector<Op> v;
    const int n = plan(counts, order, n_active, E, ring_start, streamed, group_size, n_slots,
                       flags, used_of, cursor, next_event, v);
    if (n < 0) return n;
    if (n > max_ops) return MOE_EWORKSPACE;
    std::copy(v.begin(), v.end(), reinterpret_cast<Op*>(ops));
    return n;
  } catch (...) {  // host memory: no exception crosses the C boundary
    return MOE_ENOMEM;
  }
}

static int layer_streamed(moe_walk* walk, const float* x, int T, int H, int F, int E, int K,
                          const int32_t* topk_idx, const float* topk_w, int wtype,
                          const void* host_arena, size_t arena_bytes, const int64_t* host_off,
                          const void* const* resident, int group_size, int ring_start, int flags,
                          void* ws, size_t ws_bytes, float* out, void* stream) {
  if (!walk || !host_off || !resident) return MOE_EINVAL;
  if ((flags & ~(MOE_WALK_GATHER_ONE | MOE_WALK_NO_SKIP_FLUSH | MOE_WALK_MMQ_PER_GROUP)) != 0)
    return MOE_EINVAL;
  Layout L;
  const size_t eb = moe_expert_bytes(H, F, wtype);
  const int rc = check_layer_args(x, T, H, F, E, K, topk_idx, topk_w, wtype, eb, group_size,
                                  ring_start, ws, ws_bytes, out, &L);
  if (rc != MOE_OK) return rc;
  if (walk->stride < eb) return MOE_EINVAL;
  moe_walk& w = *walk;
  HostShare* hs = w.share.get();
  if (hs && (T > hs->T_max || H != hs->H)) return MOE_EINVAL;
  w.streamed.assign(E, 0);
  for (int e = 0; e < E; ++e) {
    if (resident[e] != nullptr) continue;
    if (!host_arena || host_off[e] < 0 || (size_t)host_off[e] > arena_bytes ||
        arena_bytes - (size_t)host_off[e] < eb)
      return MOE_EINVAL;
    w.streamed[e] = 1;
  }

  hipStream_t s = as_stream(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  MapsOut mo = layer_maps(base, L);
  auto ok = [](hipError_t e) { return e == hipSuccess; };

  // maps, the routing read-back, then the quantiser runs while the host plans the walk
  int32_t* h_counts = w.host;
  int32_t* h_order = w.host + kMaxE;
  int32_t* h_nact = w.host + 2 * kMaxE;
  if (!ok(launch_build_maps(topk_idx, T, K, E, ring_start, mo, s)) ||
      !ok(hipMemcpyAsync(h_counts, mo.counts, (size_t)E * 4, hipMemcpyDeviceToHost, s)) ||
      !ok(hipMemcpyAsync(h_order, mo.order, (size_t)E * 4, hipMemcpyDeviceToHost, s)) ||
      !ok(hipMemcpyAsync(h_nact, mo.n_active, 4, hipMemcpyDeviceToHost, s)) ||
      (hs && !ok(hipMemcpyAsync(hs->h_x, x, (size_t)T * H * 4, hipMemcpyDeviceToHost, s))) ||
      (hs && !ok(hipMemcpyAsync(hs->h_src, mo.src, (size_t)T * K * 4, hipMemcpyDeviceToHost,
                                s))) ||
      !ok(hipEventRecord(w.routed, s)) ||
      !ok(launch_quantize(x, T, H, K, mo.slot, mo.src, act_mode_bits(wtype), base + L.q8x, s)) ||
      !ok(hipEventSynchronize(w.routed)))
    return MOE_EHIP;
  ++w.stats[kStSyncs];
  const int n_active = *h_nact;

  // The host's share ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto ...", "What it does"): the
  // streamed experts routed by at most max_tokens tokens, fewest first, share x the streamed
  // experts of this call; automatic: share = g / (c + g) from the last measured GPU time per
  // streamed expert (g, events of the previous call, complete by this sync) and host time per
  // expert (c), where both sides end together.
  std::vector<int> host_experts;
  std::vector<int64_t> off;           // expert e's first row (the maps' offsets, on the host)
  int host_rows = 0, n_streamed = 0;
  double share_now = 0;
  if (hs) {
    if (hs->timed && hs->timed_experts > 0) {
      float ms = 0;
      if (hipEventElapsedTime(&ms, hs->t0, hs->t1) == hipSuccess && ms > 0)
        hs->gpu_ns = ms * 1e6 / hs->timed_experts;
    }
    hs->timed = false;
    if (hs->share < 0 && hs->gpu_ns > 0 && hs->host_ns > 0)
      hs->cur = hs->gpu_ns / (hs->gpu_ns + hs->host_ns);
    share_now = hs->share < 0 ? hs->cur : hs->share;
    std::vector<int> cand;
    for (int j = 0; j < n_active; ++j) {
      const int e = h_order[j];
      if (e < 0 || e >= E) return MOE_EHIP;  // inconsistent device maps
      if (w.streamed[e] != kStreamed) continue;
      ++n_streamed;
      if (hs->max_tokens <= 0 || h_counts[e] <= hs->max_tokens) cand.push_back(e);
    }
    std::sort(cand.begin(), cand.end(), [&](int a, int b) {
      return h_counts[a] != h_counts[b] ? h_counts[a] < h_counts[b] : a < b;
    });
    const int want = (int)(share_now * n_streamed + 0.5);
    for (int e : cand) {
      if ((int)host_experts.size() >= want) break;
      if (host_rows + h_counts[e] > hs->rows_max) break;
      w.streamed[e] = kHost;
      host_experts.push_back(e);
      host_rows += h_counts[e];
    }
    off.assign(E, 0);
    for (int e = 1; e < E; ++e) off[e] = off[e - 1] + h_counts[e - 1];
  }
  const int n_host = (int)host_experts.size();

  const int n = plan(h_counts, h_order, n_active, E, ring_start, w.streamed.data(), group_size,
                     w.n_slots, flags, w.used_of.data(), &w.cursor, &w.next_event, w.ops);
  if (n < 0) return MOE_EHIP;  // the device maps are inconsistent: not a caller error

  // first m-tile of each routed position (the maps list them in ring order, 64 rows a tile)
  w.tile_first.assign(n_active + 1, 0);
  for (int j = 0; j < n_active; ++j)
    w.tile_first[j + 1] = w.tile_first[j] + (h_counts[h_order[j]] + kMmqRows - 1) / kMmqRows;
  w.slot_of.assign(n_active, -1);

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
  gu.n_tiles = mo.n_tiles;
  gu.max_tiles = L.max_tiles;
  gu.misaligned = mo.mmq_skips;
  MmqProblem dn = gu;
  dn.epilogue = MOE_EPI_F32;
  dn.mat_offset = (size_t)2 * F * (H / 32) * moe_block_bytes(wtype);
  dn.n_out = H;
  dn.k_in = F;
  dn.act = base + L.hq8;
  dn.out = base + L.dm;

  const uint8_t* arena = static_cast<const uint8_t*>(host_arena);
  // the host's experts: the MMQs skip their tiles; the pool computes their rows meanwhile
  std::vector<int> stage_first(n_host + 1, 0);  // the expert's first staged row
  std::atomic<bool> host_failed{false};
  std::chrono::steady_clock::time_point host_t0;
  // The pool's jobs read the arena, the staging buffers and the locals above: on any exit the
  // pool is joined first (this object is destroyed before everything declared earlier).
  struct PoolJoin {
    CpuPool* pool = nullptr;
    ~PoolJoin() {
      if (pool) pool->wait();
    }
  } join;
  if (hs) {
    for (int e = 0; e < E; ++e) hs->h_skip[e] = w.streamed[e] == kHost ? 1 : 0;
    if (!ok(hipMemcpyAsync(hs->d_skip, hs->h_skip, (size_t)E, hipMemcpyHostToDevice, s)) ||
        !ok(hipEventRecord(hs->t0, s)))
      return MOE_EHIP;
    gu.skip = dn.skip = hs->d_skip;
    for (int j = 0; j < n_host; ++j) stage_first[j + 1] = stage_first[j] + h_counts[host_experts[j]];
    if (n_host > 0) {
      host_t0 = std::chrono::steady_clock::now();
      hs->pool->start(n_host, [&, hs](int j, int worker) {
        try {  // a worker's exception would end the process: flag it instead
          const int e = host_experts[j];
          const int cnt = h_counts[e], first = stage_first[j];
          std::vector<const float*> xr(cnt);
          for (int i = 0; i < cnt; ++i) {
            const int32_t r = (int32_t)(off[e] + i);
            xr[i] = hs->h_x + (size_t)(hs->h_src[r] / K) * H;
            hs->h_dst[first + i] = r;
          }
          cpu_expert_rows(wtype, H, F, arena + host_off[e], xr.data(), cnt,
                          hs->h_rows + (size_t)first * H, hs->scratch[worker]);
        } catch (...) {
          host_failed.store(true);
        }
      });
      join.pool = hs->pool.get();
    }
  }
  // The MMQs of consecutive groups are deferred and launched together until a batch must wait
  // for copies (a deferred launch then goes first, so it still overlaps those copies): a
  // batch that needs no wait runs at once on the compute stream, so launching the earlier
  // group's MMQ after it delays nothing.  The slots a batch reads are released by its own
  // event, and the MMQs read only group positions, so the order is free.
  const bool per_group = (flags & MOE_WALK_MMQ_PER_GROUP) != 0;
  int mmq_p0 = -1, mmq_p1 = -1;  // the deferred MMQs' positions [p0, p1)
  auto flush_mmq = [&]() -> bool {
    if (mmq_p0 < 0) return true;
    const int t0 = w.tile_first[mmq_p0], t1 = w.tile_first[mmq_p1];
    mmq_p0 = mmq_p1 = -1;
    if (t1 <= t0) return true;  // cannot happen: a routed expert has at least one m-tile
    gu.tiles = dn.tiles = mo.tiles + t0;
    gu.tile_count = dn.tile_count = t1 - t0;
    if (!ok(launch_mmq(gu, s)) || !ok(launch_mmq(dn, s))) return false;
    w.stats[kStMmq] += 2;
    return true;
  };
  const size_t nops = w.ops.size();
  for (size_t k = 0; k < nops; ++k) {
    const int32_t* v = w.ops[k].v;
    if (v[0] == kOpCopy) {
      // Consecutive copies (always of one batch: a gather record separates batches) whose
      // experts lie slot_stride apart in the arena and whose slots follow each other go out as
      // one transfer: the copy engine's cost per transfer is then paid once per run.
      size_t r = k;
      while (r + 1 < nops && w.ops[r + 1].v[0] == kOpCopy &&
             w.ops[r + 1].v[3] == w.ops[r].v[3] + 1 &&
             host_off[w.ops[r + 1].v[2]] == host_off[w.ops[r].v[2]] + (int64_t)w.stride)
        ++r;
      uint64_t waited = 0;  // events this run already waits on (a batch releases many slots)
      static_assert(kEvents <= 64, "one bit per event");
      for (size_t q = k; q <= r; ++q) {
        const int32_t* u = w.ops[q].v;
        // a reader batch that has already finished needs no stream wait
        if (u[4] >= 0 && !((waited >> u[4]) & 1) && hipEventQuery(w.used[u[4]]) != hipSuccess) {
          if (!ok(hipStreamWaitEvent(w.copy, w.used[u[4]], 0))) return MOE_EHIP;
          waited |= uint64_t{1} << u[4];
          ++w.stats[kStCopyWaits];
        }
        w.slot_of[u[1]] = u[3];
        ++w.stats[kStCopies];
        w.stats[kStBytes] += (int64_t)eb;
      }
      const size_t bytes = (r - k) * w.stride + eb;
      if (!ok(hipMemcpyAsync(w.ring + (size_t)v[3] * w.stride, arena + host_off[v[2]], bytes,
                             hipMemcpyHostToDevice, w.copy)))
        return MOE_EHIP;
      ++w.stats[kStTransfers];
      k = r;
    } else if (v[0] == kOpGather) {
      if (v[3]) {
        if (!flush_mmq() || !ok(hipEventRecord(w.copied, w.copy)) ||
            !ok(hipStreamWaitEvent(s, w.copied, 0)))
          return MOE_EHIP;
        ++w.stats[kStWaits];
      }
      GatherPtrs gp{};
      for (int j = 0; j < v[2]; ++j) {
        const int pos = v[1] + j;
        gp.src[j] = w.slot_of[pos] >= 0
                        ? w.ring + (size_t)w.slot_of[pos] * w.stride
                        : static_cast<const uint8_t*>(resident[h_order[pos]]);
      }
      if (!ok(launch_gather_group_mmq(gp, v[2], wtype, H, F, base + L.groups, v[1],
                                      L.group_stride, s)) ||
          !ok(hipEventRecord(w.used[v[4]], s)))
        return MOE_EHIP;
      ++w.stats[kStBatches];
      if (v[5] == kWhySkip) ++w.stats[kStSkipFlush];
      if (v[5] == kWhySlot) ++w.stats[kStSlotFlush];
    } else {
      if (mmq_p0 >= 0 && mmq_p1 == v[2]) {
        mmq_p1 = v[2] + v[3];  // the next group: one launch over both
      } else {
        if (!flush_mmq()) return MOE_EHIP;
        mmq_p0 = v[2];
        mmq_p1 = v[2] + v[3];
      }
      if (per_group && !flush_mmq()) return MOE_EHIP;
    }
  }
  if (!flush_mmq()) return MOE_EHIP;
  if (hs) {
    if (!ok(hipEventRecord(hs->t1, s))) return MOE_EHIP;
    hs->timed_experts = n_streamed - n_host;
    hs->timed = hs->timed_experts > 0;
    if (n_host > 0) {
      join.pool = nullptr;
      hs->pool->wait();
      if (host_failed.load()) return MOE_ENOMEM;
      const double ns = std::chrono::duration<double, std::nano>(
                            std::chrono::steady_clock::now() - host_t0).count();
      hs->host_ns = ns / n_host;
      w.stats[kStHostUs] += (int64_t)(ns / 1e3);
      if (!ok(hipMemcpyAsync(hs->d_rows, hs->h_rows, (size_t)host_rows * H * 4,
                             hipMemcpyHostToDevice, s)) ||
          !ok(hipMemcpyAsync(hs->d_dst, hs->h_dst, (size_t)host_rows * 4, hipMemcpyHostToDevice,
                             s)) ||
          !ok(launch_scatter_rows(hs->d_rows, hs->d_dst, host_rows, H,
                                  reinterpret_cast<float*>(base + L.dm), s)))
        return MOE_EHIP;
    }
    w.stats[kStHostExperts] += n_host;
    w.stats[kStHostRows] += host_rows;
    w.stats[kStSharePpm] = (int64_t)(share_now * 1e6 + 0.5);
    w.stats[kStGpuNs] = (int64_t)hs->gpu_ns;
    w.stats[kStHostNs] = (int64_t)hs->host_ns;
  }
  if (!ok(launch_combine(reinterpret_cast<const float*>(base + L.dm), mo.slot, topk_w, T, K, H,
                         out, s)))
    return MOE_EHIP;
  return MOE_OK;
}

int moe_prefill_layer_streamed(moe_walk* walk, const float* x, int T, int H, int F, int E, int K,
                               const int32_t* topk_idx, const float* topk_w, int wtype,
                               const void* host_arena, size_t arena_bytes,
                               const int64_t* host_off, const void* const* resident,
                               int group_size, int ring_start, int flags, void* ws,
                               size_t ws_bytes, float* out, void* stream) {
  try {  // the walk's host vectors: no exception crosses the C boundary
    return layer_streamed(walk, x, T, H, F, E, K, topk_idx, topk_w, wtype, host_arena,
                          arena_bytes, host_off, resident, group_size, ring_start, flags, ws,
                          ws_bytes, out, stream);
  } catch (...) {
    return MOE_ENOMEM;
  }
}

int moe_cpu_expert_rows(int wtype, int H, int F, const void* expert, const float* x, int n_rows,
                        float* out) {
  if (!expert || !x || !out || n_rows < 1) return MOE_EINVAL;
  if (!valid_wtype(wtype)) return MOE_EUNSUPPORTED;
  if (H < 128 || H % 128 != 0 || F < 128 || F % 128 != 0) return MOE_EUNSUPPORTED;
  try {
    std::vector<const float*> xr(n_rows);
    for (int r = 0; r < n_rows; ++r) xr[r] = x + (size_t)r * H;
    CpuScratch sc;
    cpu_expert_rows(wtype, H, F, static_cast<const uint8_t*>(expert), xr.data(), n_rows, out, sc);
  } catch (...) {
    return MOE_ENOMEM;
  }
  return MOE_OK;
}

const char* moe_cpu_share_isa(void) { return cpu_share_isa(); }

}  // extern "C"
