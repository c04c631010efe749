"""Seeded synthetic inputs for the prefill MoE expert layer.

This module is the only code shared by the HIP path's tests/benchmark and the CPU oracle.  It
draws random numbers and lays them out in the weight pool's byte format; it computes none of
the layer's arithmetic (no routing, maps, quantisation of activations, products or combine).

Workloads (the pages measure real prompts on model packs that are not available here; these
stand in with the pages' chunk shapes: 10 of 512 experts, 2K..32K-token chunks, groups of 16):

  ========  ======  ====  ===  ===  ==  =====  ==========================================
  name      T       H     F    E    K   wtype  routing
  ========  ======  ====  ===  ===  ==  =====  ==========================================
  tiny      7       256   128  16   2   Q8_0   N(0,1) logits; token 3 all zero
  t2k       2048    2048  512  512  10  Q8_0   N(0,1) logits; one seeded all-zero token
  t8k       8192    2048  512  512  10  Q4_1   N(0,1) logits
  t32k      32768   2048  512  512  10  Q8_0   N(0,1) logits
  t30k_zipf 30118   2048  512  512  10  Q4_1   N(0,1) + (-1.2 ln rank) on a seeded permutation
  t30k_z092 30118   2048  512  512  10  Q4_1   the same draws with the exponent 0.92
  ========  ======  ====  ===  ===  ==  =====  ==========================================

The Zipf workload's text asks for about 60 experts without tokens and one expert above a quarter
of them; the literal bias -1.2 ln(rank) on N(0,1) logits leaves far more experts empty, and an
exponent near 0.92 gives about 60, so both are kept (the second shares every seed with the
first).

Value distributions: x ~ N(0,1) fp32; Q8_0 blocks q ~ U{-127..127}, d ~ U[1e-3, 1e-2] stored
fp16; Q4_1 blocks q ~ U{0..15}, d ~ U[1e-3, 1e-2], m ~ U[-0.05, 0] stored fp16.  Experts sit in
pool slots given by a seeded permutation, each slot ``expert_stride`` bytes (the expert's size
rounded up to 256), so a gather reads scattered slots.
"""
from __future__ import annotations

import dataclasses

import numpy as np

Q8_0, Q4_1, Q8_0_D4 = 0, 1, 2   # Q8_0_D4: Q8_0 weights, activations in the D4 q8_1 layout
BLOCK_BYTES = {Q8_0: 34, Q4_1: 20, Q8_0_D4: 34}
WTYPE_NAME = {Q8_0: "q8_0", Q4_1: "q4_1", Q8_0_D4: "q8_0_d4"}

CONFIGS = {
    "tiny": dict(no=1, T=7, H=256, F=128, E=16, K=2, wtype=Q8_0, zero_tokens=(3,)),
    "t2k": dict(no=2, T=2048, H=2048, F=512, E=512, K=10, wtype=Q8_0, zero_tokens="seeded"),
    "t8k": dict(no=3, T=8192, H=2048, F=512, E=512, K=10, wtype=Q4_1),
    "t32k": dict(no=4, T=32768, H=2048, F=512, E=512, K=10, wtype=Q8_0),
    "t30k_zipf": dict(no=5, T=30118, H=2048, F=512, E=512, K=10, wtype=Q4_1, zipf=1.2),
    "t30k_z092": dict(no=5, T=30118, H=2048, F=512, E=512, K=10, wtype=Q4_1, zipf=0.92),
}


def expert_bytes(H: int, F: int, wtype: int) -> int:
    return (2 * F * (H // 32) + H * (F // 32)) * BLOCK_BYTES[wtype]


def round_up(n: int, a: int) -> int:
    return (n + a - 1) // a * a


@dataclasses.dataclass
class Case:
    name: str
    T: int
    H: int
    F: int
    E: int
    K: int
    wtype: int
    x: np.ndarray            # [T, H] fp32
    logits: np.ndarray       # [T, E] fp32
    pool: np.ndarray         # [E * expert_stride] uint8
    expert_off: np.ndarray   # [E] int64 byte offsets into pool
    expert_bytes: int
    expert_stride: int
    ring_start: int
    group_size: int
    zero_tokens: tuple

    @property
    def R(self) -> int:
        return self.T * self.K

    def expert(self, e: int) -> np.ndarray:
        o = int(self.expert_off[e])
        return self.pool[o:o + self.expert_bytes]


def pack_q8_0(q: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """q int8 [nb, 32], d16 float16 [nb] -> [nb, 34] bytes (d little endian, then q)."""
    nb = q.shape[0]
    out = np.empty((nb, 34), np.uint8)
    out[:, 0:2] = d16.astype("<f2").view(np.uint8).reshape(nb, 2)
    out[:, 2:34] = q.astype(np.int8).view(np.uint8)
    return out


def pack_q4_1(q: np.ndarray, d16: np.ndarray, m16: np.ndarray) -> np.ndarray:
    """q uint8 0..15 [nb, 32], d16/m16 float16 [nb] -> [nb, 20] bytes.

    Byte j of the 16 packed bytes holds element j in its low nibble, element j+16 in its high.
    """
    nb = q.shape[0]
    q = q.astype(np.uint8)
    out = np.empty((nb, 20), np.uint8)
    out[:, 0:2] = d16.astype("<f2").view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = m16.astype("<f2").view(np.uint8).reshape(nb, 2)
    out[:, 4:20] = q[:, :16] | (q[:, 16:] << 4)
    return out


def random_blocks(rng: np.random.Generator, nb: int, wtype: int) -> np.ndarray:
    d16 = rng.uniform(1e-3, 1e-2, nb).astype(np.float16)
    if wtype != Q4_1:  # Q8_0 blocks (Q8_0_D4 differs only in the activations' layout)
        q = rng.integers(-127, 128, size=(nb, 32), dtype=np.int8)
        return pack_q8_0(q, d16)
    q = rng.integers(0, 16, size=(nb, 32), dtype=np.uint8)
    m16 = rng.uniform(-0.05, 0.0, nb).astype(np.float16)
    return pack_q4_1(q, d16, m16)


def make_pool(rng: np.random.Generator, E: int, H: int, F: int, wtype: int, perm_rng):
    eb = expert_bytes(H, F, wtype)
    stride = round_up(eb, 256)
    nb = eb // BLOCK_BYTES[wtype]
    pool = np.zeros(E * stride, np.uint8)
    perm = perm_rng.permutation(E)
    expert_off = perm.astype(np.int64) * stride
    for e in range(E):
        o = int(expert_off[e])
        pool[o:o + eb] = random_blocks(rng, nb, wtype).reshape(-1)
    return pool, expert_off, eb, stride


def make_case(name: str = "custom", *, T: int, H: int, F: int, E: int, K: int, wtype: int,
              seed: int, zero_tokens=(), zipf: float | None = None, ring_start=None,
              group_size: int = 16, with_pool: bool = True) -> Case:
    """``with_pool=False`` draws x and the logits only (the pool is left empty), for measurements
    of the steps that do not read the experts."""
    ss = np.random.SeedSequence(seed)
    s_x, s_logit, s_w, s_perm, s_ring, s_zipf, s_zero = ss.spawn(7)
    rx = np.random.default_rng(s_x)
    x = rx.standard_normal((T, H), dtype=np.float32)
    if zero_tokens == "seeded":
        zero_tokens = (int(np.random.default_rng(s_zero).integers(0, T)),)
    zero_tokens = tuple(int(t) for t in zero_tokens)
    for t in zero_tokens:
        x[t, :] = 0.0
    logits = np.random.default_rng(s_logit).standard_normal((T, E), dtype=np.float32)
    if zipf is not None:
        zperm = np.random.default_rng(s_zipf).permutation(E)
        bias = np.empty(E, np.float64)
        bias[zperm] = -zipf * np.log(np.arange(1, E + 1, dtype=np.float64))
        logits = (logits + bias.astype(np.float32)[None, :]).astype(np.float32)
    if with_pool:
        pool, expert_off, eb, stride = make_pool(np.random.default_rng(s_w), E, H, F, wtype,
                                                 np.random.default_rng(s_perm))
    else:
        eb = expert_bytes(H, F, wtype)
        stride = round_up(eb, 256)
        pool = np.zeros(0, np.uint8)
        expert_off = np.random.default_rng(s_perm).permutation(E).astype(np.int64) * stride
    if ring_start is None:
        ring_start = int(np.random.default_rng(s_ring).integers(1, E)) if E > 1 else 0
    return Case(name=name, T=T, H=H, F=F, E=E, K=K, wtype=wtype, x=x, logits=logits, pool=pool,
                expert_off=expert_off, expert_bytes=eb, expert_stride=stride,
                ring_start=int(ring_start), group_size=group_size, zero_tokens=zero_tokens)


def config_case(name: str, T: int | None = None, with_pool: bool = True) -> Case:
    """One of the named workloads (seed 1000 + its number).  ``T`` may shorten the chunk
    (its first T tokens keep the same rows of x and logits)."""
    c = dict(CONFIGS[name])
    no = c.pop("no")
    zero = c.pop("zero_tokens", ())
    zipf = c.pop("zipf", None)
    case = make_case(name, seed=1000 + no, zero_tokens=zero, zipf=zipf, with_pool=with_pool, **c)
    if T is not None and T < case.T:
        case.x = case.x[:T].copy()
        case.logits = case.logits[:T].copy()
        case.zero_tokens = tuple(t for t in case.zero_tokens if t < T)
        case.T = T
    return case
