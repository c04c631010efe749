#!/usr/bin/env python3
"""Benchmark of the prefill MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t8k]

A step is one pass of the whole hot path over one chunk of synthetic input already resident in
HBM: top-K routing from the router logits, then the layer (maps, q8_1 quantise-scatter, every
group's gather, MMQ gate/up with SwiGLU and requantisation, MMQ down, combine).  The metric is
routed rows per second (T*K rows per step).  Prints one JSON line.

Per-stage HIP events recorded on the layer's own stream give each kernel's duration; the
dominant kernel's roofline fraction uses its algorithmic work (ops or bytes) per launch.  The
CPU baseline times the plain C oracle on a bounded sample of the same workload.

Other lines (not the headline; each prints its own JSON line):
    --walk streamed [--ring-slots N] [--resident-frac f] [--gather-one] [--walk-group-size G]
                    [--mmq-per-group]
        routing + moe_prefill_layer_streamed: experts copied from a pinned host arena through a
        ring of device slots; reports the host->device rate against PCIe 5.0 x16.
    --walk packed       routing + moe_prefill_layer_packed (experts kept in the MMQ layout).
    --graph             routing + the layer captured in one HIP graph and replayed.
    --act-d4            a Q8_0 workload with D4 activations (fp32 scales).
    --cold-mib N        cold cache: N MiB of scratch written between steps (512 or more flushes
                        the 256 MB MALL and the L2s), each step timed by events around it.
    --copy-probe-mib N  one plain copy before the steps (the traffic counters' calibration).
    --quant-ab          the q8_1 quantiser alone: per-row gather against scatter at 2,048 /
                        8,192 / 32,768 tokens x 10 rows, warm and cold.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from quantized_expert_grouped_amd import abi, synth  # noqa: E402

# MI355X published peaks
PEAK_HBM_GBS = 8000.0          # HBM3E, GB/s
PEAK_I8_TOPS = 5000.0          # dense int8 MFMA, TOP/s (counted as 2 ops per multiply-add)

WORKLOAD_DOC = {
    "tiny": "T=7 H=256 F=128 E=16 K=2 Q8_0",
    "t2k": "T=2048 H=2048 F=512 E=512 K=10 Q8_0, uniform routing",
    "t8k": "T=8192 H=2048 F=512 E=512 K=10 Q4_1, uniform routing",
    "t32k": "T=32768 H=2048 F=512 E=512 K=10 Q8_0, uniform routing",
    "t30k_zipf": "T=30118 H=2048 F=512 E=512 K=10 Q4_1, Zipf-skewed routing",
    "t30k_z092": "T=30118 H=2048 F=512 E=512 K=10 Q4_1, Zipf-skewed routing, exponent 0.92",
}


def algorithmic_work(c, n_active: int):
    """Per-launch algorithmic work of each stage: (kind, amount) with kind 'ops' or 'bytes'.

    Bytes count each operand read once and each result written once; ops count two per
    multiply-add of the integer block dots."""
    T, H, F, E, K = c.T, c.H, c.F, c.E, c.K
    R = T * K
    xrb = abi.q8_1_row_bytes(H)
    hrb = abi.q8_1_row_bytes(F)
    eb = c.expert_bytes
    gu_bytes = 2 * F * (H // 32) * synth.BLOCK_BYTES[c.wtype]
    dn_bytes = eb - gu_bytes
    return {
        "route": ("bytes", 4 * T * E + 8 * R),
        "maps": ("bytes", 4 * R + 3 * 4 * R + 8 * E),
        "quantize": ("bytes", 4 * T * H + 4 * R + R * xrb),
        "gather": ("bytes", 2 * n_active * eb),
        "gate_up": ("ops", 4 * R * F * H),
        "down": ("ops", 2 * R * H * F),
        "combine": ("bytes", 4 * R * H + 8 * R + 4 * T * H),
        # memory side of the MMQ launches, for reference
        "gate_up_bytes": ("bytes", n_active * gu_bytes + R * xrb + R * hrb),
        "down_bytes": ("bytes", n_active * dn_bytes + R * hrb + 4 * R * H),
    }


CSRC = "quantized_expert_grouped_amd/csrc/"
# the sources each stage's kernel is built from (a traffic figure is valid while they are)
STAGE_SOURCES = {
    "route": ("route.hip", "common.hpp"),
    "maps": ("maps.hip", "common.hpp", "internal.hpp"),
    "quantize": ("quantize.hip", "common.hpp"),
    "gather": ("gather.hip", "common.hpp"),
    "gate_up": ("mmq.hip", "common.hpp", "internal.hpp"),
    "down": ("mmq.hip", "common.hpp", "internal.hpp"),
    "combine": ("combine.hip", "common.hpp"),
}


def _code_only(text: str) -> str:
    """A kernel source without its comments and with its whitespace collapsed, so that a change
    to comments alone keeps the hash (the compiled code is the same)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def stage_source_hash(stage: str) -> str:
    h = hashlib.sha256()
    for f in STAGE_SOURCES[stage]:
        with open(os.path.join(ROOT, CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")


def measured_traffic(stage: str, workload: str):
    """HBM-side bytes per launch of a stage's kernel from the committed counter summary
    (profiles/traffic_<workload>.txt, lines ``traffic <stage> <bytes> <source hash>``), or None
    when there is none or the stage's kernel sources have changed since the counters were
    taken."""
    path = traffic_path(workload)
    if stage not in STAGE_SOURCES or not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 4 and f[0] == "traffic" and f[1] == stage:
                if f[3] != stage_source_hash(stage):
                    return None
                try:
                    return int(f[2])
                except ValueError:
                    return None
    return None


def copy_probe(mib: int, dev) -> None:
    """One plain device-to-device copy of a known size, launched before the steps so that a
    counter run over this program also measures a kernel whose traffic is known (the
    calibration of FETCH_SIZE / WRITE_SIZE)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(c, idx, w, target_s: float = 12.0, threads: int = 0):
    """Time the oracle (as it stands) on the first tokens of the same workload, on all the
    host threads OpenMP gives it or on ``threads`` of them."""
    import oracle
    oracle.lib()
    if threads > 0:
        oracle.set_threads(threads)
    threads = oracle.get_threads()
    # size the sample from a short probe so that the measured run takes ~target_s
    probe_t = 16
    t0 = time.perf_counter()
    oracle.prefill_layer(c.x[:probe_t], idx[:probe_t], w[:probe_t], c.wtype, c.pool,
                         c.expert_off, c.F, c.E)
    dt = time.perf_counter() - t0
    n_tok = int(min(c.T, max(probe_t, probe_t * target_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    oracle.prefill_layer(c.x[:n_tok], idx[:n_tok], w[:n_tok], c.wtype, c.pool, c.expert_off, c.F,
                         c.E)
    dt = time.perf_counter() - t0
    rows = n_tok * c.K
    return {"value": rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_tok} tokens of {c.name} ({rows} routed rows): the whole oracle "
                      f"layer (maps, q8_1 scatter, every routed row through its expert, combine) "
                      f"in {dt:.2f} s on {threads} threads of {cpu_model()}"}


PEAK_PCIE_GBS = 64.0           # PCIe 5.0 x16, one direction, GB/s


def h2d_probe(mib: int, dev) -> float:
    """GB/s of one plain pinned-host -> device copy of `mib` MiB (the practical PCIe rate)."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(3):
        t0 = time.perf_counter()
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        best = max(best, (mib << 20) / (time.perf_counter() - t0) / 1e9)
    return best


def streamed_walk(args, c, layer, x, logits, out, dev):
    """Steps of routing + moe_prefill_layer_streamed; prints one JSON line."""
    import torch
    stride = abi.workspace_offset(abi.WS_GROUP_STRIDE, c.T, c.H, c.F, c.E, c.K, c.wtype, 16)
    # the host arena holds the experts by id, one slot stride apart (as a model loader lays
    # them out), so a batch's run of consecutive experts can go out as one transfer
    by_id = np.zeros(c.E * stride, np.uint8)
    for e in range(c.E):
        by_id[e * stride:e * stride + c.expert_bytes] = c.expert(e)
    arena = torch.from_numpy(by_id).pin_memory()
    host_off = np.arange(c.E, dtype=np.int64) * stride
    ring = torch.empty(args.ring_slots * stride, dtype=torch.uint8, device=dev)
    walk = abi.Walk(ring, args.ring_slots, stride)
    n_res = int(round(args.resident_frac * c.E))
    keep = set(np.random.default_rng(7).permutation(c.E)[:n_res].tolist())
    base = layer.pool.data_ptr()
    resident = [base + int(c.expert_off[e]) if e in keep else 0 for e in range(c.E)]
    flags = (abi.WALK_GATHER_ONE if args.gather_one else 0) | \
        (abi.WALK_MMQ_PER_GROUP if args.mmq_per_group else 0)
    G = args.walk_group_size
    share = None
    if args.cpu_share is not None:
        share = -1.0 if args.cpu_share == "auto" else float(args.cpu_share)
        walk.cpu_share(share, args.cpu_share_max_tokens, args.cpu_threads, c.T, c.H, c.T * c.K)

    def step():
        idx, w = layer.route(logits)
        abi.prefill_layer_streamed(walk, x, idx, w, c.wtype, arena, host_off, resident, c.F,
                                   c.E, G, c.ring_start, flags, layer.ws, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st0 = walk.stats()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st1 = walk.stats()
    last = ("share_ppm", "gpu_ns_per_expert", "host_ns_per_expert")   # the last call's values
    d = {k: (st1[k] if k in last else (st1[k] - st0[k]) / args.steps) for k in st1}
    pcie = h2d_probe(1024, dev)
    walk.close()
    ms_per_step = elapsed * 1e3 / args.steps
    h2d = d["bytes"] / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": "routed rows/sec (TxK) for the MoE prefill layer, streamed experts",
        "value": round(c.T * c.K * args.steps / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{c.name}: {WORKLOAD_DOC[c.name]}"
                               + (f", first {c.T} tokens" if args.tokens else ""),
                   "T": c.T, "walk": "streamed",
                   "ring_slots": args.ring_slots, "resident_experts": n_res,
                   "group_size": G, "gather_one": bool(args.gather_one),
                   "mmq_per_group": bool(args.mmq_per_group),
                   "cpu_share": args.cpu_share,
                   **({"cpu_share_max_tokens": args.cpu_share_max_tokens,
                       "cpu_share_isa": abi.cpu_share_isa(),
                       "cpu_share_threads": args.cpu_threads or os.cpu_count()}
                      if args.cpu_share is not None else {})},
        "roofline": {"kernel": "host->device expert copies (copy stream)", "bound": "pcie",
                     "achieved": round(h2d, 2), "peak": PEAK_PCIE_GBS, "unit": "GB/s",
                     "frac": round(h2d / PEAK_PCIE_GBS, 4), "traffic": None,
                     "h2d_probe_gbs": round(pcie, 2)},
        "per_step": {k: round(v, 1) for k, v in d.items()},
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


def packed_layer(args, c, layer, x, logits, out, dev):
    """Steps of routing + moe_prefill_layer_packed (no gather); prints one JSON line."""
    import torch
    layer.pack_pool()

    def step():
        idx, w = layer.route(logits)
        layer.forward_packed(x, idx, w, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    line = {
        "metric": "routed rows/sec (TxK) for the MoE prefill layer, packed resident experts "
                  "(no gather)",
        "value": round(c.T * c.K * args.steps / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{c.name}: {WORKLOAD_DOC[c.name]}", "walk": "packed"},
        "roofline": None,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


def graph_steps(args, c, layer, x, logits, out, dev):
    """Routing + the layer captured once in a HIP graph (torch.cuda.CUDAGraph over the layer's
    stream-ordered launches), then replayed; prints one JSON line."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(1, args.warmup)):
            layer.step(x, logits, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(x, logits, out)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    line = {
        "metric": "routed rows/sec (TxK) for the MoE prefill layer, one HIP graph per step",
        "value": round(c.T * c.K * args.steps / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{c.name}: {WORKLOAD_DOC[c.name]}", "graph": True},
        "roofline": None,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


QUANT_AB_TOKENS = (2048, 8192, 32768)


def quant_ab(args, dev):
    """The q8_1 quantiser alone, the per-row gather form against the scatter form ("#1368
    prefill: quantize each token's MoE input once and scatter it to its k rows", "Measured":
    2,048 / 8,192 / 32,768 tokens x 10 rows, median of 20), H = 2048, 10 of 512 experts routed
    by the GPU from N(0,1) logits (the t2k / t8k / t32k draws).  Warm: the launches back to back;
    cold: --cold-mib MiB of scratch written before each launch.  Each launch is timed by HIP
    events around it on the current stream.  Prints one JSON line."""
    import torch
    stream = torch.cuda.current_stream()
    flush = torch.empty(max(args.cold_mib, 1024) << 20, dtype=torch.uint8, device=dev)
    results = []
    for T, name in zip(QUANT_AB_TOKENS, ("t2k", "t8k", "t32k")):
        c = synth.config_case(name, with_pool=False)
        K, H, E = c.K, c.H, c.E
        x = torch.from_numpy(c.x).to(dev)
        logits = torch.from_numpy(c.logits).to(dev)
        idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
        abi.route_topk(logits, K, idx, w)
        R = T * K
        mk = lambda n, dt=torch.int32: torch.empty(n, dtype=dt, device=dev)
        m = dict(counts=mk(E), offsets=mk(E + 1), src=mk(R), slot=mk(R), order=mk(E),
                 n_active=mk(1))
        ws = mk(abi.build_maps_workspace_size(T, K, E), torch.uint8)
        abi.build_maps(idx, E, 0, m["counts"], m["offsets"], m["src"], m["slot"], m["order"],
                       m["n_active"], ws)
        q8 = torch.empty((R, abi.q8_1_row_bytes(H)), dtype=torch.uint8, device=dev)
        row = {"T": T, "rows": R}
        for cache in ("warm", "cold"):
            for mode_name, mode in (("gather", abi.QUANT_PER_ROW), ("scatter", 0)):
                for _ in range(args.warmup):
                    abi.quantize_scatter_q8_1(x, K, m["slot"], m["src"], mode, q8)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(args.steps)]
                for i in range(args.steps):
                    if cache == "cold":
                        flush.fill_(i & 0xFF)
                    ev[i][0].record(stream)
                    abi.quantize_scatter_q8_1(x, K, m["slot"], m["src"], mode, q8)
                    ev[i][1].record(stream)
                torch.cuda.synchronize()
                ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
                reads = 4 * T * H * (K if mode == abi.QUANT_PER_ROW else 1) + 4 * R
                row[f"{cache}_{mode_name}_ms"] = round(ms, 4)
                row[f"{cache}_{mode_name}_gbs"] = round((reads + R * abi.q8_1_row_bytes(H)) /
                                                        (ms * 1e-3) / 1e9, 1)
            row[f"{cache}_gather_over_scatter"] = round(row[f"{cache}_gather_ms"] /
                                                        row[f"{cache}_scatter_ms"], 3)
        results.append(row)
        del x, logits, q8, ws
        torch.cuda.empty_cache()
    line = {
        "metric": "q8_1 quantiser time, per-row gather over scatter (T x 10 rows, H = 2048), "
                  "cold cache, largest T",
        "value": results[-1]["cold_gather_over_scatter"],
        "unit": "x",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": results[-1]["cold_scatter_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32->int8",
        "data": "synthetic",
        "config": {"workload": "quantize-scatter vs per-row gather: T = 2048, 8192, 32768; "
                               "H = 2048, K = 10 of E = 512 (t2k / t8k / t32k draws)",
                   "cold_mib": max(args.cold_mib, 1024),
                   "clock": "HIP events around each launch, median of --steps launches"},
        "results": results,
        "roofline": None,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t8k", choices=sorted(synth.CONFIGS))
    ap.add_argument("--no-stage-events", action="store_true",
                    help="time the steps without the per-stage events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the CPU baseline (default: all OpenMP gives)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain copy of this many MiB before the steps (counter "
                         "calibration; outside the timed region)")
    ap.add_argument("--walk", choices=["resident", "streamed", "packed"], default="resident",
                    help="resident: every expert in HBM, the layer's one-launch schedule; "
                         "streamed: moe_prefill_layer_streamed, experts copied from a pinned "
                         "host arena through a ring of device slots; packed: "
                         "moe_prefill_layer_packed, experts kept in the MMQ layout and read in "
                         "place, no gather (the last two print other lines, not the headline)")
    ap.add_argument("--ring-slots", type=int, default=96)
    ap.add_argument("--resident-frac", type=float, default=0.0,
                    help="streamed walk: the fraction of experts held in HBM (not copied)")
    ap.add_argument("--walk-group-size", type=int, default=16)
    ap.add_argument("--mmq-per-group", action="store_true",
                    help="streamed walk: one MMQ launch pair per group (never merged)")
    ap.add_argument("--gather-one", action="store_true",
                    help="streamed walk: one gather launch, wait and event per expert")
    ap.add_argument("--cpu-share", default=None,
                    help="streamed walk: hand the least-routed streamed experts to host threads, "
                         "a fixed share in (0, 1] or 'auto' (g / (c + g) from measured rates)")
    ap.add_argument("--cpu-share-max-tokens", type=int, default=0,
                    help="streamed walk with --cpu-share: only experts routed by at most this "
                         "many tokens (0: any)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="the workload's first N tokens only (small chunks: the CPU share's "
                         "regime); not the headline")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (routing + the layer) in a HIP graph and time its "
                         "replays (another line, not the headline)")
    ap.add_argument("--cold-mib", type=int, default=0,
                    help="write this many MiB of scratch between steps (cache flush) and time "
                         "each step with events around it (another line, not the headline)")
    ap.add_argument("--quant-ab", action="store_true",
                    help="the q8_1 quantiser alone, per-row gather against scatter, at 2,048 / "
                         "8,192 / 32,768 tokens x 10 rows, warm and cold (another line)")
    ap.add_argument("--act-d4", action="store_true",
                    help="a Q8_0 workload with its activations in the D4 q8_1 layout (fp32 "
                         "scales) instead of DS4")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by token chunks with no exchange: each GPU would run its own "
              "chunk, so the one-GPU figure is the per-GPU rate)", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_expert_grouped_amd.layer import MoePrefillLayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.quant_ab:
        quant_ab(args, dev)
        return
    c = synth.config_case(args.workload, T=args.tokens or None)
    if args.act_d4:
        if c.wtype != synth.Q8_0:
            print("bench.py: --act-d4 applies to the Q8_0 workloads", file=sys.stderr)
            sys.exit(2)
        c.wtype = synth.Q8_0_D4          # the same experts, activations in D4
    layer = MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                            group_size=16, ring_start=c.ring_start, device=dev)
    x = torch.from_numpy(c.x).to(dev)
    logits = torch.from_numpy(c.logits).to(dev)
    out = torch.empty((c.T, c.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, dev)

    if args.walk == "streamed":
        streamed_walk(args, c, layer, x, logits, out, dev)
        return
    if args.walk == "packed":
        packed_layer(args, c, layer, x, logits, out, dev)
        return
    if args.graph:
        graph_steps(args, c, layer, x, logits, out, dev)
        return

    for _ in range(args.warmup):
        layer.step(x, logits, out)
    torch.cuda.synchronize()

    use_events = not args.no_stage_events
    if use_events:
        abi.profile_begin(args.steps)
        ev_route = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(args.steps)]
    flush = None
    if args.cold_mib > 0:
        flush = torch.empty(args.cold_mib << 20, dtype=torch.uint8, device=dev)
        ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)          # evicts the previous step's data from the caches
            ev_step[i][0].record(stream)
        if use_events:
            ev_route[i][0].record(stream)
            idx, w = layer.route(logits)
            ev_route[i][1].record(stream)
            layer.forward(x, idx, w, out)
        else:
            layer.step(x, logits, out)
        if flush is not None:
            ev_step[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    rows = c.T * c.K
    value = rows * args.steps / elapsed
    if flush is not None:                  # the steps alone, without the flushes
        ms_per_step = float(np.mean([a.elapsed_time(b) for a, b in ev_step]))
        value = rows / (ms_per_step * 1e-3)

    n_active = int(layer.ws_view(abi.WS_NACTIVE, c.T, 4).view(torch.int32).item())
    work = algorithmic_work(c, n_active)
    stages = {}
    roofline = None
    if use_events:
        ms = abi.profile_end(args.steps)               # [steps, 6]
        route_ms = np.array([a.elapsed_time(b) for a, b in ev_route])
        avg = dict(zip(abi.STAGES, ms.mean(axis=0).tolist()))
        avg = {"route": float(route_ms.mean()), **avg}
        for name, t_ms in avg.items():
            entry = {"ms": round(t_ms, 4)}
            if name in work:
                kind, amt = work[name]
                if kind == "ops":
                    entry["tops"] = round(amt / (t_ms * 1e-3) / 1e12, 2)
                    entry["frac_i8_peak"] = round(entry["tops"] / PEAK_I8_TOPS, 4)
                    kb, bb = work[name + "_bytes"]
                    roof = min(PEAK_I8_TOPS, amt / bb * PEAK_HBM_GBS / 1e3)
                    entry["frac_ai_roof"] = round(entry["tops"] / roof, 4)
                    entry["gbs"] = round(bb / (t_ms * 1e-3) / 1e9, 1)
                else:
                    entry["gbs"] = round(amt / (t_ms * 1e-3) / 1e9, 1)
                    entry["frac_hbm_peak"] = round(entry["gbs"] / PEAK_HBM_GBS, 4)
            stages[name] = entry
        for name, entry in stages.items():
            tb = measured_traffic(name, c.name)
            if tb is not None and name in work:
                alg = work[name + "_bytes"][1] if work[name][0] == "ops" else work[name][1]
                entry["traffic_bytes"] = tb
                entry["traffic_ratio"] = round(tb / alg, 3)
        dom = max(avg, key=avg.get)
        kind, amt = work.get(dom, ("bytes", 4 * c.R))
        t_s = avg[dom] * 1e-3
        clock = ("HIP events on the layer's stream around each launch (they add the event "
                 "records' gap; the kernel trace in profiles/ times the kernel alone)")
        if kind == "ops":
            achieved = amt / t_s / 1e12
            alg_bytes = work[dom + "_bytes"][1]
            roof = min(PEAK_I8_TOPS, amt / alg_bytes * PEAK_HBM_GBS / 1e3)
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                        "peak": PEAK_I8_TOPS, "unit": "TOP/s",
                        "frac": round(achieved / PEAK_I8_TOPS, 4),
                        "traffic": measured_traffic(dom, c.name),
                        "algorithmic_ops": amt, "algorithmic_bytes": alg_bytes,
                        "ai_roof": round(roof, 1), "frac_ai_roof": round(achieved / roof, 4),
                        "launch_ms": round(avg[dom], 4), "clock": clock}
        else:
            achieved = amt / t_s / 1e9
            roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(dom, c.name),
                        "algorithmic_bytes": amt, "launch_ms": round(avg[dom], 4),
                        "clock": clock}

    cpu = None
    if not args.no_cpu_baseline:
        idx_d, w_d = layer.route(logits)
        cpu = cpu_baseline(c, idx_d.cpu().numpy(), w_d.cpu().numpy(), threads=args.cpu_threads)

    line = {
        "metric": "routed rows/sec (TxK) for the MoE prefill layer"
                  + (", cold cache" if flush is not None else ""),
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{c.name}: {WORKLOAD_DOC[c.name]}"
                               + (", D4 activations" if c.wtype == synth.Q8_0_D4 else ""),
                   "T": c.T, "H": c.H,
                   "F": c.F, "E": c.E, "K": c.K, "wtype": synth.WTYPE_NAME[c.wtype],
                   "group_size": 16, "active_experts": n_active, "stage_events": use_events,
                   **({"cache": f"cold: {args.cold_mib} MiB written between steps, each step "
                                "timed by events around it"} if flush is not None else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": stages,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
