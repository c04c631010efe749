"""CPU oracle for the prefill MoE expert layer (TEST INFRASTRUCTURE).

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may import this
package.  The arithmetic lives in ``moe_oracle.c`` (plain C, fp64); this module only builds
it with gcc and marshals numpy arrays through ctypes.  Nothing here is shared with the HIP
library in ``quantized_expert_grouped_amd``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_0, Q4_1, Q8_0_D4 = 0, 1, 2      # Q8_0_D4: Q8_0 weights, D4 activations
DS4, D4 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (portable -O2, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        sz = ctypes.c_size_t
        sig = {
            "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_block_bytes": (sz, [i]),
            "orc_expert_bytes": (sz, [i, i, i]),
            "orc_q8_1_row_bytes": (sz, [i]),
            "orc_set_threads": (None, [i]),
            "orc_get_threads": (i, []),
            "orc_route_topk": (None, [P, i, i, i, P, P]),
            "orc_build_maps": (None, [P, i, i, i, i, P, P, P, P, P, P]),
            "orc_q8_1_block": (None, [P, P, P, P]),
            "orc_q8_1_row": (None, [P, i, P]),
            "orc_q8_1_row_d4": (None, [P, i, P]),
            "orc_quantize_gather": (None, [P, i, i, i, P, i, P]),
            "orc_quantize_scatter": (None, [P, i, i, i, P, i, P]),
            "orc_gather": (None, [P, P, P, i, sz, P, i, sz]),
            "orc_block_idot": (ctypes.c_int32, [i, P, P]),
            "orc_row_dot": (ctypes.c_double, [i, P, P, i]),
            "orc_block_dots": (None, [i, P, i, i, P, i, P]),
            "orc_matrix_rows": (None, [i, P, i, i, P, i, P]),
            "orc_expert_row": (None, [i, P, i, i, P, P, P, P]),
            "orc_combine": (None, [P, P, P, i, i, i, P]),
            "orc_prefill_layer": (i, [P, i, i, i, i, i, P, P, i, P, P, P, P, P, P, P]),
            "orc_token_out": (None, [P, i, i, i, P, P, i, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ---- formats -----------------------------------------------------------------------------
def f32_to_f16(f: float) -> int:
    return int(lib().orc_f32_to_f16(float(f)))


def f16_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(int(h)))


def block_bytes(wtype: int) -> int:
    return int(lib().orc_block_bytes(wtype))


def expert_bytes(H: int, F: int, wtype: int) -> int:
    return int(lib().orc_expert_bytes(H, F, wtype))


def q8_1_row_bytes(n: int) -> int:
    return int(lib().orc_q8_1_row_bytes(n))


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ---- a0 / a1 -----------------------------------------------------------------------------
def route_topk(logits, K: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    lib().orc_route_topk(_p(logits), T, E, K, _p(idx), _p(w))
    return idx, w


def build_maps(idx, E: int, ring_start: int = 0):
    idx = _c(idx, np.int32)
    T, K = idx.shape
    R = T * K
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    src = np.empty(R, np.int32)
    slot = np.empty(R, np.int32)
    order = np.empty(E, np.int32)
    n_active = np.zeros(1, np.int32)
    lib().orc_build_maps(_p(idx), T, K, E, int(ring_start), _p(counts), _p(offsets), _p(src),
                         _p(slot), _p(order), _p(n_active))
    n = int(n_active[0])
    return dict(counts=counts, offsets=offsets, src=src, slot=slot, order=order[:n].copy(),
                n_active=n)


# ---- a2 / a5 -----------------------------------------------------------------------------
def q8_1_block(v):
    v = _c(v, np.float32)
    assert v.shape == (32,)
    q = np.empty(32, np.int8)
    d = np.zeros(1, np.uint16)
    s = np.zeros(1, np.uint16)
    lib().orc_q8_1_block(_p(v), _p(q), _p(d), _p(s))
    return q, int(d[0]), int(s[0])


def q8_1_rows(v, layout: int = DS4):
    """Quantise every row of a [N x n] fp32 array to q8_1 bytes [N x n/128*144] (DS4 or D4)."""
    v = _c(v, np.float32)
    N, n = v.shape
    rb = q8_1_row_bytes(n)
    out = np.empty((N, rb), np.uint8)
    L = lib()
    fn = L.orc_q8_1_row_d4 if layout == D4 else L.orc_q8_1_row
    for r in range(N):
        fn(_p(v[r]), n, _p(out[r]))
    return out


def act_layout(wtype: int) -> int:
    """The q8_1 layout of a weight type's activations."""
    return D4 if wtype == Q8_0_D4 else DS4


def quantize_gather(x, K: int, src, layout: int = DS4):
    x = _c(x, np.float32)
    src = _c(src, np.int32)
    T, H = x.shape
    out = np.empty((T * K, q8_1_row_bytes(H)), np.uint8)
    lib().orc_quantize_gather(_p(x), T, H, K, _p(src), layout, _p(out))
    return out


def quantize_scatter(x, K: int, slot, layout: int = DS4):
    x = _c(x, np.float32)
    slot = _c(slot, np.int32)
    T, H = x.shape
    out = np.empty((T * K, q8_1_row_bytes(H)), np.uint8)
    lib().orc_quantize_scatter(_p(x), T, H, K, _p(slot), layout, _p(out))
    return out


# ---- a3 ----------------------------------------------------------------------------------
def gather(pool, expert_off, experts, expert_bytes_: int, group_buf, first_pos: int,
           pos_stride: int):
    pool = _c(pool, np.uint8)
    expert_off = _c(expert_off, np.int64)
    experts = _c(experts, np.int32)
    assert group_buf.dtype == np.uint8 and group_buf.flags.c_contiguous
    assert (first_pos + len(experts) - 1) * pos_stride + expert_bytes_ <= group_buf.size
    lib().orc_gather(_p(pool), _p(expert_off), _p(experts), len(experts), expert_bytes_,
                     _p(group_buf), int(first_pos), int(pos_stride))
    return group_buf


# ---- a4 / a6 -----------------------------------------------------------------------------
def block_idot(wtype: int, wblock, xq) -> int:
    wblock = _c(wblock, np.uint8)
    xq = _c(xq, np.int8)
    return int(lib().orc_block_idot(wtype, _p(wblock), _p(xq)))


def row_dot(wtype: int, wrow, xrow_q8, k_in: int) -> float:
    wrow = _c(wrow, np.uint8)
    xrow_q8 = _c(xrow_q8, np.uint8)
    return float(lib().orc_row_dot(wtype, _p(wrow), _p(xrow_q8), k_in))


def block_dots(wtype: int, wmat, n_out: int, k_in: int, act_q8):
    wmat = _c(wmat, np.uint8)
    act_q8 = _c(act_q8, np.uint8)
    n_rows = act_q8.shape[0]
    out = np.empty((n_rows, n_out, k_in // 32), np.int32)
    lib().orc_block_dots(wtype, _p(wmat), n_out, k_in, _p(act_q8), n_rows, _p(out))
    return out


def matrix_rows(wtype: int, wmat, n_out: int, k_in: int, act_q8):
    """fp64 products [n_rows x n_out] of activation rows with a weight matrix's rows."""
    wmat = _c(wmat, np.uint8)
    act_q8 = _c(act_q8, np.uint8)
    n_rows = act_q8.shape[0]
    out = np.empty((n_rows, n_out), np.float64)
    lib().orc_matrix_rows(wtype, _p(wmat), n_out, k_in, _p(act_q8), n_rows, _p(out))
    return out


def expert_row(wtype: int, expert, H: int, F: int, xrow_q8):
    expert = _c(expert, np.uint8)
    xrow_q8 = _c(xrow_q8, np.uint8)
    h = np.empty(F, np.float32)
    hq = np.empty(q8_1_row_bytes(F), np.uint8)
    dm = np.empty(H, np.float64)
    lib().orc_expert_row(wtype, _p(expert), H, F, _p(xrow_q8), _p(h), _p(hq), _p(dm))
    return h, hq, dm


# ---- a7 / layer --------------------------------------------------------------------------
def combine(Dm, slot, w):
    Dm = _c(Dm, np.float64)
    slot = _c(slot, np.int32)
    w = _c(w, np.float32)
    T, K = w.shape
    H = Dm.shape[1]
    out = np.empty((T, H), np.float32)
    lib().orc_combine(_p(Dm), _p(slot), _p(w), T, K, H, _p(out))
    return out


def prefill_layer(x, idx, w, wtype: int, pool, expert_off, F: int, E: int, debug: bool = False):
    x = _c(x, np.float32)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    pool = _c(pool, np.uint8)
    expert_off = _c(expert_off, np.int64)
    T, H = x.shape
    K = idx.shape[1]
    R = T * K
    out = np.empty((T, H), np.float32)
    q8x = h = hq8 = Dm = None
    if debug:
        q8x = np.empty((R, q8_1_row_bytes(H)), np.uint8)
        h = np.empty((R, F), np.float32)
        hq8 = np.empty((R, q8_1_row_bytes(F)), np.uint8)
        Dm = np.empty((R, H), np.float64)
    rc = lib().orc_prefill_layer(_p(x), T, H, F, E, K, _p(idx), _p(w), wtype, _p(pool),
                                 _p(expert_off), _p(out), _p(q8x), _p(h), _p(hq8), _p(Dm))
    if rc != 0:
        raise ValueError(f"orc_prefill_layer rejected the arguments (rc={rc})")
    if debug:
        return out, dict(q8x=q8x, h=h, hq8=hq8, Dm=Dm)
    return out


def token_out(x_row, idx_row, w_row, wtype: int, pool, expert_off, F: int):
    x_row = _c(x_row, np.float32)
    idx_row = _c(idx_row, np.int32)
    w_row = _c(w_row, np.float32)
    H = x_row.shape[0]
    out = np.empty(H, np.float32)
    lib().orc_token_out(_p(x_row), H, F, len(idx_row), _p(idx_row), _p(w_row), wtype,
                        _p(_c(pool, np.uint8)), _p(_c(expert_off, np.int64)), _p(out))
    return out
