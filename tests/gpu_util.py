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
