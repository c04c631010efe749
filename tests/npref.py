"""Independent numpy brute force used to pin the C oracle (tests only).

Written from the definitions, not from the oracle's code: numpy's own float16 for the fp16
conversions, vectorised quantisation, dequantise-then-matmul products, a stable library sort
for the maps.  It shares nothing with oracle/moe_oracle.c.
"""
from __future__ import annotations

import numpy as np

Q8_0, Q4_1, Q8_0_D4 = 0, 1, 2    # Q8_0_D4: Q8_0 weights, D4 activations


# ---- fp16 ------------------------------------------------------------------------------------
def f16_bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def f16_val(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# ---- q8_1 (DS4) -------------------------------------------------------------------------------
def q8_1_blocks(v: np.ndarray):
    """v float32 [..., 32] -> (q int8 [..., 32], d16 bits, s16 bits).

    d = amax/127 in fp32; q = round half away from zero of v/d (fp32 quotient, the rounding
    done in fp64 so that adding 0.5 is exact); s = fp16(d * S) with an fp32 product."""
    v = np.asarray(v, np.float32)
    amax = np.max(np.abs(v), axis=-1)
    zero = amax == 0
    d = (amax / np.float32(127.0)).astype(np.float32)
    dsafe = np.where(zero, np.float32(1.0), d).astype(np.float32)
    quot = (v / dsafe[..., None]).astype(np.float32).astype(np.float64)
    q = (np.sign(quot) * np.floor(np.abs(quot) + 0.5)).astype(np.int64)
    q[zero] = 0
    S = q.sum(axis=-1)
    s = (d * S.astype(np.float32)).astype(np.float32)
    d16 = f16_bits(d)
    s16 = f16_bits(s)
    d16[zero] = 0
    s16[zero] = 0
    return q.astype(np.int8), d16, s16


def q8_1_rows(v: np.ndarray) -> np.ndarray:
    """[N, n] fp32 -> [N, n/128*144] bytes in the DS4 layout."""
    v = np.asarray(v, np.float32)
    N, n = v.shape
    G = n // 128
    q, d16, s16 = q8_1_blocks(v.reshape(N, G, 4, 32))
    out = np.empty((N, G, 144), np.uint8)
    ds = np.stack([d16, s16], axis=-1).astype("<u2")           # [N, G, 4, 2]
    out[:, :, 0:16] = ds.view(np.uint8).reshape(N, G, 16)
    out[:, :, 16:] = q.view(np.uint8).reshape(N, G, 128)
    return out.reshape(N, G * 144)


def q8_1_rows_d4(v: np.ndarray) -> np.ndarray:
    """[N, n] fp32 -> [N, n/128*144] bytes in the D4 layout: per 128 values the 4 blocks' fp32
    d (amax/127, the value before any fp16 rounding), then their q (as in DS4)."""
    v = np.asarray(v, np.float32)
    N, n = v.shape
    G = n // 128
    blocks = v.reshape(N, G, 4, 32)
    q, _, _ = q8_1_blocks(blocks)
    d = (np.max(np.abs(blocks), axis=-1) / np.float32(127.0)).astype("<f4")   # 0 for zero blocks
    out = np.empty((N, G, 144), np.uint8)
    out[:, :, 0:16] = d.view(np.uint8).reshape(N, G, 16)
    out[:, :, 16:] = q.view(np.uint8).reshape(N, G, 128)
    return out.reshape(N, G * 144)


def q8_1_rows_for(v: np.ndarray, wtype: int) -> np.ndarray:
    return q8_1_rows_d4(v) if wtype == Q8_0_D4 else q8_1_rows(v)


def q8_1_decode_d4(rows: np.ndarray, n: int):
    """D4 bytes -> (q int [N, n], dx [N, n/32] fp64 of the fp32 d, sx zeros)."""
    rows = np.asarray(rows, np.uint8)
    N = rows.shape[0]
    G = n // 128
    g = rows.reshape(N, G, 144)
    d = g[:, :, 0:16].copy().view("<f4").reshape(N, G * 4).astype(np.float64)
    q = g[:, :, 16:].copy().view(np.int8).reshape(N, n).astype(np.int64)
    return q, d, np.zeros_like(d)


def q8_1_decode(rows: np.ndarray, n: int):
    """DS4 bytes -> (q int [N, n], dx [N, n/32], sx [N, n/32]) as fp64 values."""
    rows = np.asarray(rows, np.uint8)
    N = rows.shape[0]
    G = n // 128
    g = rows.reshape(N, G, 144)
    ds = g[:, :, 0:16].copy().view("<u2").reshape(N, G, 4, 2)
    q = g[:, :, 16:].copy().view(np.int8).reshape(N, n).astype(np.int64)
    dx = f16_val(ds[..., 0]).reshape(N, G * 4)
    sx = f16_val(ds[..., 1]).reshape(N, G * 4)
    return q, dx, sx


# ---- weights ----------------------------------------------------------------------------------
def unpack_matrix(raw: np.ndarray, n_rows: int, k_in: int, wtype: int):
    """Weight matrix bytes -> (q int [n_rows, k_in], d [n_rows, k_in/32], m or None)."""
    nb = k_in // 32
    bb = 20 if wtype == Q4_1 else 34
    blk = np.asarray(raw, np.uint8)[: n_rows * nb * bb].reshape(n_rows, nb, bb)
    d = f16_val(blk[:, :, 0:2].copy().view("<u2")[..., 0])
    if wtype != Q4_1:
        q = blk[:, :, 2:34].copy().view(np.int8).astype(np.int64).reshape(n_rows, k_in)
        return q, d, None
    m = f16_val(blk[:, :, 2:4].copy().view("<u2")[..., 0])
    qs = blk[:, :, 4:20].astype(np.int64)
    q = np.concatenate([qs & 15, qs >> 4], axis=-1).reshape(n_rows, k_in)
    return q, d, m


def dequant_matrix(raw, n_rows, k_in, wtype) -> np.ndarray:
    q, d, m = unpack_matrix(raw, n_rows, k_in, wtype)
    w = q.reshape(n_rows, k_in // 32, 32) * d[..., None]
    if m is not None:
        w = w + m[..., None]
    return w.reshape(n_rows, k_in)


def matrix_parts(raw, n_rows, k_in, wtype):
    """-> (A, M): A = d*q per weight [n_rows, k_in]; M = m per block [n_rows, k_in/32] or None."""
    q, d, m = unpack_matrix(raw, n_rows, k_in, wtype)
    A = (q.reshape(n_rows, k_in // 32, 32) * d[..., None]).reshape(n_rows, k_in)
    return A, m


def expert_mats(expert: np.ndarray, H: int, F: int, wtype: int):
    """(gate, up, down) as (A, M) pairs; gate is the first F rows, up the next F, then down."""
    bb = 20 if wtype == Q4_1 else 34
    gu = F * (H // 32) * bb
    gate = matrix_parts(expert[0:gu], F, H, wtype)
    up = matrix_parts(expert[gu:2 * gu], F, H, wtype)
    down = matrix_parts(expert[2 * gu:], H, F, wtype)
    return gate, up, down


def dequant_act(rows: np.ndarray, n: int, wtype: int = Q8_0) -> np.ndarray:
    q, dx, _ = (q8_1_decode_d4 if wtype == Q8_0_D4 else q8_1_decode)(rows, n)
    N = q.shape[0]
    return (q.reshape(N, n // 32, 32) * dx[..., None]).reshape(N, n)


def qproduct(parts, act_row: np.ndarray, n: int, wtype: int = Q8_0) -> np.ndarray:
    """Weight matrix times one q8_1 activation row, in matrix form: A @ (dx*q) plus, for Q4_1,
    M @ s -- the min term uses the s the DS4 layout stores for it."""
    A, M = parts
    q, dx, sx = (q8_1_decode_d4 if wtype == Q8_0_D4 else q8_1_decode)(act_row[None, :], n)
    xh = (q.reshape(n // 32, 32) * dx[0][:, None]).reshape(n)
    y = A @ xh
    if M is not None:
        y = y + M @ sx[0]
    return y


# ---- routing / maps --------------------------------------------------------------------------
def route(logits: np.ndarray, K: int):
    T, E = logits.shape
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    ids = np.arange(E)
    for t in range(T):
        o = np.lexsort((ids, -logits[t].astype(np.float64)))[:K]
        idx[t] = o
        z = logits[t, o].astype(np.float64)
        e = np.exp(z - z.max())
        w[t] = e / e.sum()
    return idx, w


def maps(idx: np.ndarray, E: int, ring_start: int):
    flat = np.asarray(idx, np.int64).reshape(-1)
    src = np.argsort(flat, kind="stable").astype(np.int32)
    slot = np.empty_like(src)
    slot[src] = np.arange(len(src), dtype=np.int32)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ring = [(ring_start + j) % E for j in range(E)]
    order = np.array([e for e in ring if counts[e] > 0], np.int32)
    return dict(counts=counts, offsets=offsets, src=src, slot=slot, order=order)


# ---- layer (dense fp64 chain per route) ----------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def layer(x, idx, w, pool, expert_off, expert_bytes, H, F, wtype):
    """out[t] = sum_k w[t,k] * down_e(q8_1(silu(gate_e q8_1(x_t)) * up_e q8_1(x_t)))."""
    x = np.asarray(x, np.float32)
    T = x.shape[0]
    K = idx.shape[1]
    xq = q8_1_rows_for(x, wtype)
    out = np.zeros((T, H), np.float64)
    cache = {}
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if e not in cache:
                o = int(expert_off[e])
                cache[e] = expert_mats(pool[o:o + expert_bytes], H, F, wtype)
            g_p, u_p, d_p = cache[e]
            g = qproduct(g_p, xq[t], H, wtype)
            u = qproduct(u_p, xq[t], H, wtype)
            h = (silu(g) * u).astype(np.float32)
            out[t] += float(w[t, k]) * qproduct(d_p, q8_1_rows_for(h[None, :], wtype)[0], F,
                                                wtype)
    return out


def layer_unquantized(x, idx, w, pool, expert_off, expert_bytes, H, F, wtype):
    """Same chain with fp64 activations (no q8_1 of x or h): a loose sanity reference."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    K = idx.shape[1]
    out = np.zeros((T, H), np.float64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            o = int(expert_off[e])
            bb = 20 if wtype == Q4_1 else 34
            gu = F * (H // 32) * bb
            ex = pool[o:o + expert_bytes]
            g_m = dequant_matrix(ex[0:gu], F, H, wtype)
            u_m = dequant_matrix(ex[gu:2 * gu], F, H, wtype)
            d_m = dequant_matrix(ex[2 * gu:], H, F, wtype)
            h = silu(g_m @ x[t]) * (u_m @ x[t])
            out[t] += float(w[t, k]) * (d_m @ h)
    return out
