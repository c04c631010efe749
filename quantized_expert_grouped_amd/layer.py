"""A prefill MoE expert layer held on one GPU: the expert pool and the workspace stay resident in
HBM, and each call enqueues routing and the layer on the current torch stream.

Marshalling only -- the computation is libmoe_prefill.so's (see ``abi``).
"""
from __future__ import annotations

import numpy as np
import torch

from . import abi


class MoePrefillLayer:
    def __init__(self, pool, expert_off, H: int, F: int, E: int, wtype: int, max_tokens: int,
                 K: int, group_size: int = 16, ring_start: int = 0, device="cuda"):
        self.H, self.F, self.E, self.K, self.wtype = H, F, E, K, wtype
        self.group_size, self.ring_start = group_size, ring_start
        self.device = torch.device(device)
        self.pool = _to_device(pool, torch.uint8, self.device)
        self.expert_off = _to_device(expert_off, torch.int64, self.device)
        self.expert_bytes = abi.expert_bytes(H, F, wtype)
        self.max_tokens = max_tokens
        nbytes = abi.workspace_size(max_tokens, H, F, E, K, wtype, group_size)
        if nbytes == 0:
            raise ValueError("unsupported layer shape")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)

    def route(self, logits: torch.Tensor):
        T = logits.shape[0]
        idx = torch.empty((T, self.K), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.K), dtype=torch.float32, device=self.device)
        abi.route_topk(logits, self.K, idx, w)
        return idx, w

    def forward(self, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                out: torch.Tensor | None = None, group_size: int | None = None,
                ring_start: int | None = None) -> torch.Tensor:
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"T={T} exceeds the workspace's {self.max_tokens} tokens")
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        gs = self.group_size if group_size is None else group_size
        rs = self.ring_start if ring_start is None else ring_start
        abi.prefill_layer(x, idx, w, self.wtype, self.pool, self.expert_off, self.F, self.E, gs,
                          rs, self.ws, out)
        return out

    def pack_pool(self) -> torch.Tensor:
        """The pool with every expert put in the MMQ layout at its own offset (one gather launch
        per expert; done once, the experts never change), for forward_packed."""
        off = self.expert_off.cpu().numpy()
        if np.any(off % 16 != 0):
            raise ValueError("the packed layer reads experts at 16-byte aligned offsets only")
        packed = torch.zeros_like(self.pool)
        base, dst = self.pool.data_ptr(), packed.data_ptr()
        for e in range(self.E):
            o = int(off[e])
            abi.gather_group_mmq([base + o], self.wtype, self.H, self.F, dst + o, 0, 0)
        self.packed = packed
        return packed

    def forward_packed(self, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                       out: torch.Tensor | None = None, ring_start: int | None = None):
        """The layer reading the packed pool in place (no gather); pack_pool() first."""
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"T={T} exceeds the workspace's {self.max_tokens} tokens")
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        rs = self.ring_start if ring_start is None else ring_start
        abi.prefill_layer_packed(x, idx, w, self.wtype, self.packed, self.expert_off, self.F,
                                 self.E, rs, self.ws, out)
        return out

    def step(self, x: torch.Tensor, logits: torch.Tensor, out: torch.Tensor | None = None):
        """One pass of the whole hot path: routing, then the layer."""
        idx, w = self.route(logits)
        return self.forward(x, idx, w, out)

    def ws_view(self, which: int, T: int, nbytes: int) -> torch.Tensor:
        off = abi.workspace_offset(which, T, self.H, self.F, self.E, self.K, self.wtype,
                                   self.group_size)
        return self.ws[off:off + nbytes]


def _to_device(a, dtype, device):
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)
