"""Helpers for the GPU parity tests: move seeded inputs to the device and back."""
from __future__ import annotations

import sys

import numpy as np
import torch

from quantized_expert_grouped_amd import abi


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still leaves the name behind)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(shape, dtype) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device="cuda")


def gpu_maps(idx: np.ndarray, E: int, ring_start: int):
    T, K = idx.shape
    R = T * K
    d_idx = dev(idx.astype(np.int32))
    out = dict(counts=empty(E, torch.int32), offsets=empty(E + 1, torch.int32),
               src=empty(R, torch.int32), slot=empty(R, torch.int32),
               order=empty(E, torch.int32), n_active=empty(1, torch.int32))
    ws = empty(abi.build_maps_workspace_size(T, K, E), torch.uint8)
    abi.build_maps(d_idx, E, ring_start, out["counts"], out["offsets"], out["src"], out["slot"],
                   out["order"], out["n_active"], ws)
    res = {k: host(v) for k, v in out.items()}
    res["n_invalid"] = int(host(ws[:4]).view(np.int32)[0])   # the scratch's status word
    n = int(res["n_active"][0])
    res["n_active"] = n
    res["order"] = res["order"][:n]
    return res, out


def gpu_quantize(x: np.ndarray, K: int, slot: np.ndarray, src: np.ndarray, mode: int):
    T, H = x.shape
    q8 = torch.zeros((T * K, abi.q8_1_row_bytes(H)), dtype=torch.uint8, device="cuda")
    abi.quantize_scatter_q8_1(dev(x), K, dev(slot.astype(np.int32)), dev(src.astype(np.int32)),
                              mode, q8)
    return host(q8)


def rel_err(got, want) -> float:
    want = np.asarray(want, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - want)) /
                 max(float(np.max(np.abs(want))), 1e-300))


def gpu_group_buffer(orc, c, experts, stride=None):
    """A group buffer built by the library's MMQ-layout gather (one launch) from the case's pool
    on the device, checked before use: decoded, every position equals the oracle's verbatim copy
    of its expert (orc_gather).  Returns the device buffer."""
    import mmq_layout
    experts = np.asarray(experts, np.int32)
    stride = c.expert_stride if stride is None else stride
    d_pool = dev(c.pool)
    gbuf = torch.zeros(len(experts) * stride, dtype=torch.uint8, device="cuda")
    note(f"gather_group_mmq n={len(experts)} wtype={c.wtype} H={c.H} F={c.F}")
    abi.gather_group_mmq([d_pool.data_ptr() + int(c.expert_off[e]) for e in experts], c.wtype,
                         c.H, c.F, gbuf, 0, stride)
    raw = np.zeros(len(experts) * c.expert_bytes, np.uint8)
    orc.gather(c.pool, c.expert_off, experts, c.expert_bytes, raw, 0, c.expert_bytes)
    mmq_layout.check_positions(host(gbuf), c.wtype, c.H, c.F,
                               [raw[j * c.expert_bytes:(j + 1) * c.expert_bytes]
                                for j in range(len(experts))], 0, stride)
    del d_pool
    return gbuf
