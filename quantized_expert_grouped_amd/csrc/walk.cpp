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
#include <new>
#include <vector>

#include "internal.hpp"
#include "layout.hpp"
#include "moe_prefill.h"

using namespace moe;

namespace {

constexpr int kEvents = MOE_WALK_EVENTS;
constexpr int kMaxE = MOE_MAX_E;
enum { kOpCopy = 1, kOpGather = 2, kOpMmq = 3 };
enum { kWhyGroup = 0, kWhySkip = 1, kWhySlot = 2, kWhyOne = 3 };
enum {
  kStCopies, kStBytes, kStBatches, kStWaits, kStCopyWaits, kStSkipFlush, kStSlotFlush, kStMmq,
  kStSyncs, kStTransfers
};

struct Op {
  int32_t v[6];
};

// The walk over ring entries ring_start, ring_start+1, ... (mod E).  A routed entry takes the
// next group position; a streamed one first takes the next ring slot (round robin) for its copy,
// which waits on the event of that slot's last reader.  The open batch is launched when its group
// is complete, at a skipped entry, when the next slot is one the open batch holds, or after every
// expert (one-expert mode); a group's MMQ record follows its last batch.
int plan(const int32_t* counts, const int32_t* order, int n_active, int E, int ring_start,
         const uint8_t* streamed, int G, int n_slots, int flags, int32_t* used_of,
         int32_t* cursor, int32_t* next_event, std::vector<Op>& ops) {
  if (!counts || !order || !streamed || !used_of || !cursor || !next_event) return MOE_EINVAL;
  if (E < 1 || E > kMaxE || ring_start < 0 || ring_start >= E || n_active < 0 || n_active > E ||
      G < 1 || G > MOE_MAX_GROUP || n_slots < 1 || *cursor < 0 || *cursor >= n_slots ||
      *next_event < 0 || *next_event >= kEvents ||
      (flags & ~(MOE_WALK_GATHER_ONE | MOE_WALK_NO_SKIP_FLUSH)) != 0)
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
    if (streamed[e]) {
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
  delete w;
}

}  // namespace

extern "C" {

int moe_walk_create(void* ring, int n_slots, size_t slot_stride, moe_walk** walk) {
  if (!ring || !walk || n_slots < 1 || slot_stride == 0 || slot_stride % 256 != 0 ||
      (uintptr_t)ring % 256 != 0)
    return MOE_EINVAL;
  moe_walk* w = new (std::nothrow) moe_walk;
  if (!w) return MOE_EHIP;
  w->ring = static_cast<uint8_t*>(ring);
  w->n_slots = n_slots;
  w->stride = slot_stride;
  w->used_of.assign(n_slots, -1);
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
  std::vector<Op> v;
  const int n = plan(counts, order, n_active, E, ring_start, streamed, group_size, n_slots, flags,
                     used_of, cursor, next_event, v);
  if (n < 0) return n;
  if (n > max_ops) return MOE_EWORKSPACE;
  std::copy(v.begin(), v.end(), reinterpret_cast<Op*>(ops));
  return n;
}

int moe_prefill_layer_streamed(moe_walk* walk, const float* x, int T, int H, int F, int E, int K,
                               const int32_t* topk_idx, const float* topk_w, int wtype,
                               const void* host_arena, size_t arena_bytes,
                               const int64_t* host_off, const void* const* resident,
                               int group_size, int ring_start, int flags, void* ws,
                               size_t ws_bytes, float* out, void* stream) {
  if (!walk || !host_off || !resident) return MOE_EINVAL;
  if ((flags & ~(MOE_WALK_GATHER_ONE | MOE_WALK_NO_SKIP_FLUSH)) != 0) return MOE_EINVAL;
  Layout L;
  const size_t eb = moe_expert_bytes(H, F, wtype);
  const int rc = check_layer_args(x, T, H, F, E, K, topk_idx, topk_w, wtype, eb, group_size,
                                  ring_start, ws, ws_bytes, out, &L);
  if (rc != MOE_OK) return rc;
  if (walk->stride < eb) return MOE_EINVAL;
  moe_walk& w = *walk;
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
      !ok(hipEventRecord(w.routed, s)) ||
      !ok(launch_quantize(x, T, H, K, mo.slot, mo.src, act_mode_bits(wtype), base + L.q8x, s)) ||
      !ok(hipEventSynchronize(w.routed)))
    return MOE_EHIP;
  ++w.stats[kStSyncs];
  const int n_active = *h_nact;
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
        if (!ok(hipEventRecord(w.copied, w.copy)) || !ok(hipStreamWaitEvent(s, w.copied, 0)))
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
      const int t0 = w.tile_first[v[2]], t1 = w.tile_first[v[2] + v[3]];
      if (t1 <= t0) continue;  // cannot happen: a routed expert has at least one m-tile
      gu.tiles = dn.tiles = mo.tiles + t0;
      gu.tile_count = dn.tile_count = t1 - t0;
      if (!ok(launch_mmq(gu, s)) || !ok(launch_mmq(dn, s))) return MOE_EHIP;
      w.stats[kStMmq] += 2;
    }
  }
  if (!ok(launch_combine(reinterpret_cast<const float*>(base + L.dm), mo.slot, topk_w, T, K, H,
                         out, s)))
    return MOE_EHIP;
  return MOE_OK;
}

}  // extern "C"
