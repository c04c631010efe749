"""The C-ABI library loads and exports every entry point include/*.h declares (CPU only: no
compute call reaches a kernel here)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from quantized_expert_grouped_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z0-9_]+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_library_built_and_loads():
    assert os.path.exists(abi.LIB_PATH), "build with python -m quantized_expert_grouped_amd.build"
    abi.lib()


def test_every_declared_symbol_is_exported():
    declared = _declared_functions()
    assert len(declared) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(moe_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    # the binding covers exactly the declared functions
    assert sorted(abi.SIGNATURES) == declared


def test_version_and_sizes():
    assert abi.abi_version() == 7
    assert abi.block_bytes(abi.Q8_0) == 34 and abi.block_bytes(abi.Q4_1) == 20
    assert abi.block_bytes(7) == 0
    assert abi.block_bytes(abi.Q8_0_D4) == 34
    assert abi.expert_bytes(2048, 512, abi.Q8_0_D4) == abi.expert_bytes(2048, 512, abi.Q8_0)
    assert abi.expert_bytes(2048, 512, abi.Q8_0) == 3342336
    assert abi.expert_bytes(2048, 512, abi.Q4_1) == 1966080
    assert abi.q8_1_row_bytes(2048) == 2304
    assert abi.strerror(-3) == "workspace too small"
    assert abi.strerror(-5) == "host memory or threads could not be obtained"
    assert abi.STATUS[-5] == "MOE_ENOMEM"
    ws = abi.workspace_size(8192, 2048, 512, 512, 10, abi.Q4_1, 16)
    R = 8192 * 10
    # at least q8 rows of x and h, Dm, and one group position per expert
    assert ws >= R * 2304 + R * 576 + R * 2048 * 4 + 512 * 1966080
    assert abi.workspace_size(8192, 2048, 512, 512, 10, abi.Q4_1, 17) == 0
    assert abi.workspace_size(8192, 2000, 512, 512, 10, abi.Q4_1, 16) == 0     # H % 128
    assert abi.workspace_size(8192, 2048, 500, 512, 10, abi.Q4_1, 16) == 0     # F % 128
    assert abi.workspace_size(1 << 27, 2048, 512, 512, 10, abi.Q4_1, 16) == 0  # T*K > 2^30
    assert abi.build_maps_workspace_size(1 << 27, 10, 512) == 0
    assert abi.build_maps_workspace_size(8192, 10, 512) > 0
    offs = [abi.workspace_offset(i, 100, 256, 128, 16, 2, abi.Q8_0) for i in range(10)]
    assert all(o % 256 == 0 for o in offs)
    assert abi.workspace_offset(abi.WS_GROUP_STRIDE, 100, 256, 128, 16, 2, abi.Q8_0) % 256 == 0
    assert abi.workspace_offset(99, 100, 256, 128, 16, 2, abi.Q8_0) == ctypes.c_size_t(-1).value


def test_host_validation_rejects_before_any_launch():
    L = abi.lib()
    # null pointers / bad sizes are refused on the host (no GPU is touched)
    assert L.moe_route_topk(None, 4, 16, 2, None, None, None) == -1
    assert L.moe_route_topk(1, 4, 4096, 2, 1, 1, None) == -2          # E too large
    assert L.moe_quantize_scatter_q8_1(16, 4, 200, 2, 16, 16, 0, 16, None) == -2  # H % 128
    assert L.moe_quantize_scatter_q8_1(16, 4, 256, 2, None, 16, 0, 16, None) == -1  # no slot
    assert abi.raw_gather_group([16] * 17, 64, 16, 0, 64, stream=0) == -1        # more than 16 experts
    assert abi.raw_gather_group([16] * 4, 64, 16, 13, 64, stream=0) == -1        # 13 + 4 > 16
    assert abi.raw_gather_group([16, 0], 64, 16, 0, 64, stream=0) == -1          # a null expert pointer
    assert abi.raw_gather_group_mmq([16] * 2, abi.Q4_1, 256, 128, 16, 0, 64, stream=0) == -1  # stride
    assert abi.raw_gather_group_mmq([16], abi.Q4_1, 200, 128, 16, 0, 0, stream=0) == -2       # H % 128
    assert abi.raw_gather_group_mmq([16], 7, 256, 128, 16, 0, 0, stream=0) == -2              # type
    assert abi.raw_gather_group_mmq([0], abi.Q8_0, 256, 128, 16, 0, 0, stream=0) == -1        # null
    assert abi.raw_mmq_grouped(abi.Q8_0, 16, 256, 0, 128, 128, [0], 16, 4, 16, 3, 16, stream=0) == -1
    assert abi.raw_mmq_grouped(abi.Q8_0, 16, 256, 0, 100, 128, [0], 16, 4, 16, 0, 16, stream=0) == -2
    assert abi.raw_mmq_grouped(abi.Q8_0, 16, 256, 0, 128, 128, [4], 16, 4, 16, 0, 16, stream=0) == -1
    assert abi.raw_mmq_grouped(abi.Q8_0, 16, 256, 0, 128, 128, [0], 16, 4, 8, 0, 16, stream=0) == -1
    assert L.moe_combine(16, 16, 16, 3, 2, 6, 16, None) == -2           # H % 4
    eb = abi.expert_bytes(256, 128, abi.Q8_0)

    class T:
        def __init__(self, shape, p=256):
            self.shape = shape
            self._p = p

        def data_ptr(self):
            return self._p

        def numel(self):
            return 1 << 20

        def element_size(self):
            return 1

    x, idx, w, out = T((7, 256)), T((7, 2)), T((7, 2)), T((7, 256))
    ws = T((1,))
    args = dict(x=x, topk_idx=idx, topk_w=w, wtype=abi.Q8_0, pool=256, expert_off=256, F=128,
                E=16, group_size=16, ring_start=0, ws=ws, out=out, stream=0)
    assert abi.raw_prefill_layer(**{**args, "group_size": 0}) == -1
    assert abi.raw_prefill_layer(**{**args, "ring_start": 16}) == -1
    assert abi.raw_prefill_layer(**{**args, "wtype": 7}) == -2
    assert abi.raw_prefill_layer(**args, ws_bytes=100) == -3
    assert abi.raw_prefill_layer(**{**args, "x": T((7, 256), p=260)}) == -1   # misaligned x
    assert eb == 104448


def test_profiler_end_without_begin_is_empty():
    assert abi.profile_end(4).shape == (0, abi.N_STAGES)


def test_walk_host_validation():
    L = abi.lib()
    import ctypes as ct
    h = ct.c_void_p()
    assert L.moe_walk_create(None, 4, 256, ct.byref(h)) == -1           # no ring
    assert L.moe_walk_create(256, 0, 256, ct.byref(h)) == -1            # no slots
    assert L.moe_walk_create(256, 4, 300, ct.byref(h)) == -1            # stride % 256
    assert L.moe_walk_create(256, 4, 256, None) == -1                   # nowhere to put it
    assert L.moe_walk_destroy(None) == 0
    assert L.moe_walk_stats(None, None, 0) == -1
    assert L.moe_prefill_layer_streamed(None, 16, 4, 256, 128, 8, 2, 16, 16, 0, 16, 1 << 20, 16,
                                        16, 16, 0, 0, 16, 1 << 20, 16, None) == -1


def test_packed_layer_host_validation():
    L = abi.lib()
    # x, T, H, F, E, K, idx, w, wtype, packed_pool, expert_off, expert_bytes, ring_start, ws,
    # ws_bytes, out, stream
    eb = abi.expert_bytes(256, 128, abi.Q8_0)
    ok = [16, 4, 256, 128, 8, 2, 16, 16, abi.Q8_0, 256, 16, eb, 0, 256, 1 << 40, 16, None]

    def call(**kw):
        a = list(ok)
        names = ["x", "T", "H", "F", "E", "K", "idx", "w", "wtype", "pool", "off", "eb", "rs",
                 "ws", "ws_bytes", "out", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.moe_prefill_layer_packed(*a)

    assert call(pool=None) == -1                 # no pool
    assert call(off=None) == -1                  # no offsets
    assert call(wtype=7) == -2                   # unknown type
    assert call(H=200) == -2                     # H % 128
    assert call(eb=eb + 1) == -1                 # wrong expert size
    assert call(pool=264) == -1                  # pool not 16-byte aligned
    assert call(rs=8) == -1                      # ring_start >= E
    assert call(ws_bytes=16) == -3               # workspace too small


def test_host_checks_refuse_matrices_beyond_32_bit_offsets():
    """The MMQ addresses a weight matrix by 32-bit offsets: larger matrices are refused on the host
    (MOE_EUNSUPPORTED) before anything is enqueued, so no pointer here is ever dereferenced."""
    L = abi.lib()
    fake = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never touched
    experts = (ctypes.c_int32 * 1)(0)
    # gate and up of 32,768 x 2,048 Q8_0 blocks: 4.56 GB > 4 GiB
    rc = L.moe_mmq_grouped(0, fake, 1 << 33, 0, 32768, 65536, ctypes.cast(experts, ctypes.c_void_p),
                           1, fake, 1, fake, 1, fake, None, None)
    assert rc == -2
    # the same shape as a single matrix (fp32 epilogue): 2.28 GB, accepted by this check, then
    # refused further on only by what the fake pointers cannot satisfy
    rc = L.moe_mmq_grouped(0, fake, 1 << 33, 0, 32768, 65536, ctypes.cast(experts, ctypes.c_void_p),
                           1, fake, 1, fake, 0, ctypes.c_void_p(3), None, None)
    assert rc == -1                          # out not 4-byte aligned: MOE_EINVAL
    # the layer: H = 65,536, F = 32,768 (gate + up 4.56 GB)
    eb = abi.expert_bytes(65536, 32768, 0)
    rc = L.moe_prefill_layer(fake, 8, 65536, 32768, 16, 2, fake, fake, 0, fake, fake, eb, 16, 0,
                             fake, 1 << 62, fake, None)
    assert rc == -2
    # control: H = F = 32,768 (gate + up 2.28 GB, down 1.14 GB) passes that check and stops at the
    # workspace size (MOE_EWORKSPACE)
    eb = abi.expert_bytes(32768, 32768, 0)
    rc = L.moe_prefill_layer(fake, 8, 32768, 32768, 16, 2, fake, fake, 0, fake, fake, eb, 16, 0,
                             fake, 0, fake, None)
    assert rc == -3
