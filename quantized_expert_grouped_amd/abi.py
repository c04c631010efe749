"""Thin Python binding of libmoe_prefill.so (include/moe_prefill.h).

Argument marshalling only: every step runs in the library's HIP kernels.  Tensors are torch
tensors on the GPU; the stream defaults to torch's current stream.  Loading fails loudly when the
library has not been built (``python -m quantized_expert_grouped_amd.build``) -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_prefill.so")

Q8_0, Q4_1, Q8_0_D4 = 0, 1, 2
QUANT_PER_ROW, QUANT_D4 = 1, 2
EPI_F32, EPI_SWIGLU_Q8_1, EPI_I32_BLOCKDOTS = 0, 1, 2
WS_COUNTS, WS_OFFSETS, WS_SRC, WS_SLOT, WS_ORDER, WS_NACTIVE, WS_Q8X, WS_GROUPS, WS_HQ8, WS_DM, \
    WS_GROUP_STRIDE, WS_STATUS = range(12)
N_STAGES = 6
STAGES = ("maps", "quantize", "gather", "gate_up", "down", "combine")

WALK_EVENTS = 64
WALK_GATHER_ONE, WALK_NO_SKIP_FLUSH, WALK_MMQ_PER_GROUP = 1, 2, 4
WALK_NSTATS = 16
WALK_STATS = ("copies", "bytes", "batches", "waits", "copy_waits", "skip_flushes", "slot_flushes",
              "mmq_launches", "routing_syncs", "transfers", "host_experts", "host_rows",
              "host_us", "share_ppm", "gpu_ns_per_expert", "host_ns_per_expert")
OP_COPY, OP_GATHER, OP_MMQ = 1, 2, 3

STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED", -3: "MOE_EWORKSPACE",
          -4: "MOE_EHIP", -5: "MOE_ENOMEM"}

# name -> (restype, argtypes); the order of this table is the header's order
P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "moe_abi_version": (I, []),
    "moe_strerror": (ctypes.c_char_p, [I]),
    "moe_block_bytes": (SZ, [I]),
    "moe_expert_bytes": (SZ, [I, I, I]),
    "moe_q8_1_row_bytes": (SZ, [I]),
    "moe_build_maps_workspace_size": (SZ, [I, I, I]),
    "moe_workspace_size": (SZ, [I, I, I, I, I, I, I]),
    "moe_route_topk": (I, [P, I, I, I, P, P, P]),
    "moe_build_maps": (I, [P, I, I, I, I, P, P, P, P, P, P, P, SZ, P]),
    "moe_build_maps_noalloc": (I, [P, I, I, I, I, P, P, P, P, P, P, P, P]),
    "moe_quantize_scatter_q8_1": (I, [P, I, I, I, P, P, I, P, P]),
    "moe_gather_group": (I, [P, I, SZ, P, I, SZ, P]),
    "moe_gather_group_mmq": (I, [P, I, I, I, I, P, I, SZ, P]),
    "moe_mmq_grouped": (I, [I, P, SZ, SZ, I, I, P, I, P, I, P, I, P, P, P]),
    "moe_combine": (I, [P, P, P, I, I, I, P, P]),
    "moe_prefill_layer": (I, [P, I, I, I, I, I, P, P, I, P, P, SZ, I, I, P, SZ, P, P]),
    "moe_prefill_layer_packed": (I, [P, I, I, I, I, I, P, P, I, P, P, SZ, I, P, SZ, P, P]),
    "moe_workspace_offset": (SZ, [I, I, I, I, I, I, I, I]),
    "moe_walk_create": (I, [P, I, SZ, P]),
    "moe_walk_destroy": (I, [P]),
    "moe_prefill_layer_streamed": (I, [P, P, I, I, I, I, I, P, P, I, P, SZ, P, P, I, I, I, P, SZ,
                                       P, P]),
    "moe_walk_stats": (I, [P, P, I]),
    "moe_walk_cpu_share": (I, [P, ctypes.c_double, I, I, I, I, I]),
    "moe_cpu_expert_rows": (I, [I, I, I, P, P, I, P]),
    "moe_cpu_share_isa": (ctypes.c_char_p, []),
    "moe_walk_plan": (I, [P, P, I, I, I, P, I, I, I, P, P, P, P, I]),
    "moe_profile_begin": (I, [I]),
    "moe_profile_end": (I, [P, I]),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_expert_grouped_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name: str, rc: int) -> None:
    if rc != 0:
        raise MoeError(name, rc)


# ---- sizes ----------------------------------------------------------------------------------
def abi_version() -> int:
    return lib().moe_abi_version()


def strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def block_bytes(wtype: int) -> int:
    return lib().moe_block_bytes(wtype)


def expert_bytes(H: int, F: int, wtype: int) -> int:
    return lib().moe_expert_bytes(H, F, wtype)


def q8_1_row_bytes(n: int) -> int:
    return lib().moe_q8_1_row_bytes(n)


def build_maps_workspace_size(T: int, K: int, E: int) -> int:
    return lib().moe_build_maps_workspace_size(T, K, E)


def workspace_size(T, H, F, E, K, wtype, group_size=16) -> int:
    return lib().moe_workspace_size(T, H, F, E, K, wtype, group_size)


def workspace_offset(which, T, H, F, E, K, wtype, group_size=16) -> int:
    return lib().moe_workspace_offset(which, T, H, F, E, K, wtype, group_size)


# ---- entry points (raise MoeError on a non-zero status; `raw_*` return the status) -------------
def route_topk(logits, K, idx, w, stream=None):
    T, E = logits.shape
    _check("moe_route_topk", lib().moe_route_topk(_ptr(logits), T, E, K, _ptr(idx), _ptr(w),
                                                  _stream(stream)))


def build_maps(topk_idx, E, ring_start, counts, offsets, src, slot, order, n_active, ws,
               stream=None):
    T, K = topk_idx.shape
    _check("moe_build_maps", lib().moe_build_maps(
        _ptr(topk_idx), T, K, E, ring_start, _ptr(counts), _ptr(offsets), _ptr(src), _ptr(slot),
        _ptr(order), _ptr(n_active), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def raw_build_maps_noalloc(topk_idx, E, ring_start, counts, offsets, src, slot, order,
                           n_active, n_invalid=None, stream=None):
    T, K = topk_idx.shape
    return lib().moe_build_maps_noalloc(
        _ptr(topk_idx), T, K, E, ring_start, _ptr(counts), _ptr(offsets), _ptr(src), _ptr(slot),
        _ptr(order), _ptr(n_active), _ptr(n_invalid), _stream(stream))


def build_maps_noalloc(*args, **kw):
    _check("moe_build_maps_noalloc", raw_build_maps_noalloc(*args, **kw))


def quantize_scatter_q8_1(x, K, slot, src, mode, q8, stream=None):
    T, H = x.shape
    _check("moe_quantize_scatter_q8_1", lib().moe_quantize_scatter_q8_1(
        _ptr(x), T, H, K, _ptr(slot), _ptr(src), mode, _ptr(q8), _stream(stream)))


def raw_gather_group(src_ptrs, expert_bytes_, group_buf, first_pos, pos_stride, stream=None):
    n = len(src_ptrs)
    arr = (ctypes.c_void_p * max(n, 1))(*[int(p) for p in src_ptrs])
    return lib().moe_gather_group(ctypes.cast(arr, ctypes.c_void_p) if n else None, n,
                                  expert_bytes_, _ptr(group_buf), first_pos, pos_stride,
                                  _stream(stream))


def gather_group(src_ptrs, expert_bytes_, group_buf, first_pos, pos_stride, stream=None):
    _check("moe_gather_group", raw_gather_group(src_ptrs, expert_bytes_, group_buf, first_pos,
                                                pos_stride, stream))


def raw_gather_group_mmq(src_ptrs, wtype, H, F, group_buf, first_pos, pos_stride, stream=None):
    n = len(src_ptrs)
    arr = (ctypes.c_void_p * max(n, 1))(*[int(p) for p in src_ptrs])
    return lib().moe_gather_group_mmq(ctypes.cast(arr, ctypes.c_void_p) if n else None, n, wtype,
                                      H, F, _ptr(group_buf), first_pos, pos_stride,
                                      _stream(stream))


def gather_group_mmq(src_ptrs, wtype, H, F, group_buf, first_pos, pos_stride, stream=None):
    _check("moe_gather_group_mmq", raw_gather_group_mmq(src_ptrs, wtype, H, F, group_buf,
                                                        first_pos, pos_stride, stream))


def raw_mmq_grouped(wtype, group_buf, pos_stride, mat_offset, n_out, k_in, group_experts,
                    offsets, E, act_q8, epilogue, out, debug_h=None, stream=None):
    ge = np.ascontiguousarray(group_experts, dtype=np.int32)
    return lib().moe_mmq_grouped(
        wtype, _ptr(group_buf), pos_stride, mat_offset, n_out, k_in,
        ge.ctypes.data_as(ctypes.c_void_p), len(ge), _ptr(offsets), E, _ptr(act_q8), epilogue,
        _ptr(out), _ptr(debug_h), _stream(stream))


def mmq_grouped(*args, **kw):
    _check("moe_mmq_grouped", raw_mmq_grouped(*args, **kw))


def combine(Dm, slot, topk_w, out, stream=None):
    T, K = topk_w.shape
    H = Dm.shape[1]
    _check("moe_combine", lib().moe_combine(_ptr(Dm), _ptr(slot), _ptr(topk_w), T, K, H,
                                            _ptr(out), _stream(stream)))


def raw_prefill_layer(x, topk_idx, topk_w, wtype, pool, expert_off, F, E, group_size, ring_start,
                      ws, out, stream=None, ws_bytes=None):
    T, H = x.shape
    K = topk_idx.shape[1]
    eb = expert_bytes(H, F, wtype)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    return lib().moe_prefill_layer(_ptr(x), T, H, F, E, K, _ptr(topk_idx), _ptr(topk_w), wtype,
                                   _ptr(pool), _ptr(expert_off), eb, group_size, ring_start,
                                   _ptr(ws), nbytes, _ptr(out), _stream(stream))


def prefill_layer(*args, **kw):
    _check("moe_prefill_layer", raw_prefill_layer(*args, **kw))


def raw_prefill_layer_packed(x, topk_idx, topk_w, wtype, packed_pool, expert_off, F, E,
                             ring_start, ws, out, stream=None):
    T, H = x.shape
    K = topk_idx.shape[1]
    eb = expert_bytes(H, F, wtype)
    return lib().moe_prefill_layer_packed(_ptr(x), T, H, F, E, K, _ptr(topk_idx), _ptr(topk_w),
                                          wtype, _ptr(packed_pool), _ptr(expert_off), eb,
                                          ring_start, _ptr(ws), ws.numel() * ws.element_size(),
                                          _ptr(out), _stream(stream))


def prefill_layer_packed(*args, **kw):
    _check("moe_prefill_layer_packed", raw_prefill_layer_packed(*args, **kw))


def profile_begin(n_calls: int) -> None:
    _check("moe_profile_begin", lib().moe_profile_begin(n_calls))


def profile_end(max_calls: int) -> np.ndarray:
    ms = np.zeros((max_calls, N_STAGES), np.float32)
    n = lib().moe_profile_end(ms.ctypes.data_as(ctypes.c_void_p), max_calls)
    if n < 0:
        raise MoeError("moe_profile_end", n)
    return ms[:n]


# ---- streamed walk --------------------------------------------------------------------------
class Walk:
    """A walk's state (copy stream, events, slot map) over a caller-owned device ring of n_slots
    slots of slot_stride bytes (`ring`: a device tensor kept alive by this object)."""

    def __init__(self, ring, n_slots: int, slot_stride: int):
        self.ring = ring
        self.n_slots, self.slot_stride = n_slots, slot_stride
        h = ctypes.c_void_p()
        _check("moe_walk_create", lib().moe_walk_create(_ptr(ring), n_slots, slot_stride,
                                                        ctypes.byref(h)))
        self.handle = h.value

    def close(self) -> None:
        if self.handle:
            lib().moe_walk_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def cpu_share(self, share: float, max_tokens: int, threads: int, max_T: int, H: int,
                  max_rows: int) -> None:
        """The host's share of the walk (share < 0: automatic; 0: off)."""
        _check("moe_walk_cpu_share", lib().moe_walk_cpu_share(self.handle, float(share),
                                                              max_tokens, threads, max_T, H,
                                                              max_rows))

    def stats(self) -> dict:
        a = np.zeros(WALK_NSTATS, np.int64)
        _check("moe_walk_stats", lib().moe_walk_stats(self.handle,
                                                      a.ctypes.data_as(ctypes.c_void_p),
                                                      WALK_NSTATS))
        return dict(zip(WALK_STATS, (int(v) for v in a)))


def raw_prefill_layer_streamed(walk, x, topk_idx, topk_w, wtype, host_arena, host_off, resident,
                               F, E, group_size, ring_start, flags, ws, out, stream=None,
                               arena_bytes=None):
    """host_arena: a pinned host tensor (uint8); host_off: int64 [E]; resident: E device pointers
    (0 = stream the expert from the arena)."""
    T, H = x.shape
    K = topk_idx.shape[1]
    off = np.ascontiguousarray(host_off, dtype=np.int64)
    res = (ctypes.c_void_p * E)(*[int(p) if p else None for p in resident])
    nb = (host_arena.numel() * host_arena.element_size() if arena_bytes is None
          else arena_bytes) if host_arena is not None else 0
    return lib().moe_prefill_layer_streamed(
        walk.handle if isinstance(walk, Walk) else walk, _ptr(x), T, H, F, E, K, _ptr(topk_idx),
        _ptr(topk_w), wtype, _ptr(host_arena), nb, off.ctypes.data_as(ctypes.c_void_p),
        ctypes.cast(res, ctypes.c_void_p), group_size, ring_start, flags, _ptr(ws),
        ws.numel() * ws.element_size(), _ptr(out), _stream(stream))


def prefill_layer_streamed(*args, **kw):
    _check("moe_prefill_layer_streamed", raw_prefill_layer_streamed(*args, **kw))


def cpu_expert_rows(wtype, H, F, expert, x):
    """The host's computation of one expert's unweighted rows (numpy in, numpy out)."""
    expert = np.ascontiguousarray(expert, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty((x.shape[0], H), np.float32)
    vp = ctypes.c_void_p
    _check("moe_cpu_expert_rows", lib().moe_cpu_expert_rows(
        wtype, H, F, expert.ctypes.data_as(vp), x.ctypes.data_as(vp), x.shape[0],
        out.ctypes.data_as(vp)))
    return out


def cpu_share_isa() -> str:
    return lib().moe_cpu_share_isa().decode()


def walk_plan(counts, order, n_active, ring_start, streamed, group_size, n_slots, flags=0,
              state=None, max_ops=None):
    """The walk's schedule (host only).  state: dict with used_of / cursor / next_event, updated
    in place (a fresh one when None).  Returns (status_or_count, ops int32 [n x 6], state)."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    E = len(counts)
    order = np.ascontiguousarray(order, dtype=np.int32)
    if len(order) < E:
        order = np.concatenate([order, np.zeros(E - len(order), np.int32)])
    streamed = np.ascontiguousarray(streamed, dtype=np.uint8)
    if state is None:
        state = {"used_of": np.full(n_slots, -1, np.int32), "cursor": 0, "next_event": 0}
    used_of = state["used_of"]
    cur = ctypes.c_int32(state["cursor"])
    nev = ctypes.c_int32(state["next_event"])
    if max_ops is None:
        max_ops = 4 * E + 8
    ops = np.zeros((max(max_ops, 1), 6), np.int32)
    vp = ctypes.c_void_p
    n = lib().moe_walk_plan(counts.ctypes.data_as(vp), order.ctypes.data_as(vp), n_active, E,
                            ring_start, streamed.ctypes.data_as(vp), group_size, n_slots, flags,
                            used_of.ctypes.data_as(vp), ctypes.byref(cur), ctypes.byref(nev),
                            ops.ctypes.data_as(vp), max_ops)
    state["cursor"], state["next_event"] = cur.value, nev.value
    return n, (ops[:n] if n >= 0 else ops[:0]), state
