"""The CPU share's host computation (moe_cpu_expert_rows, the library's host code; no GPU) against
the oracle: an expert's unweighted rows for routed inputs ("#1282 prefill:
STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's least-routed experts to the idle CPU pool",
"What it does": the CPU's rows are not bit-identical to the GPU's but as accurate).

Every instruction-set path the host code has (AVX-512 VNNI, AVX2, scalar) is run, each in a
child process with MOE_CPU_ISA capping the choice; all must agree with the oracle's rows within
the layer's tolerance, and the two SIMD paths (the same lanes summed in the same order) bit for
bit."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from quantized_expert_grouped_amd import abi, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TOL = 1e-3

SHAPES = [(256, 128, synth.Q8_0, 5), (256, 128, synth.Q4_1, 9), (512, 256, synth.Q8_0_D4, 3),
          (2048, 512, synth.Q4_1, 17), (384, 384, synth.Q8_0, 1)]


def _inputs(H, F, wtype, n, seed):
    rng = np.random.default_rng(seed)
    nb = synth.expert_bytes(H, F, wtype) // synth.BLOCK_BYTES[wtype]
    expert = synth.random_blocks(rng, nb, wtype).reshape(-1)
    x = rng.standard_normal((n, H)).astype(np.float32)
    x[0] = 0.0                       # an all-zero input: an exact zero row
    if n > 2:
        x[1] *= np.float32(1e-30)    # subnormal-scale blocks
    return expert, x


def _run_paths():
    """Each path's rows for every shape, from child processes (the ISA is chosen once per
    process)."""
    out = {}
    for isa in ("vnni", "avx2", "scalar"):
        env = dict(os.environ, MOE_CPU_ISA=isa)
        code = ("import json, sys, numpy as np; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
                "from quantized_expert_grouped_amd import abi\n"
                "import test_cpu_share_kernel as t\n"
                "res = {}\n"
                "for i, (H, F, wt, n) in enumerate(t.SHAPES):\n"
                "    e, x = t._inputs(H, F, wt, n, 100 + i)\n"
                "    res[i] = abi.cpu_expert_rows(wt, H, F, e, x).tolist()\n"
                "print(json.dumps({'isa': abi.cpu_share_isa(), 'rows': res}))\n"
                % (ROOT, os.path.join(ROOT, "tests")))
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        d = json.loads(r.stdout.strip().splitlines()[-1])
        out[d["isa"]] = {int(k): np.array(v, np.float32) for k, v in d["rows"].items()}
    return out


@pytest.fixture(scope="module")
def paths():
    return _run_paths()


def test_every_path_ran(paths):
    assert "scalar" in paths and ("avx2" in paths or len(paths) == 1)


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_host_rows_against_oracle(orc, paths, i):
    H, F, wtype, n = SHAPES[i]
    expert, x = _inputs(H, F, wtype, n, 100 + i)
    xq = orc.q8_1_rows(x, orc.act_layout(wtype))
    want = np.stack([orc.expert_row(wtype, expert, H, F, xq[r])[2] for r in range(n)])
    scale = max(float(np.max(np.abs(want))), 1e-30)
    for isa, rows in paths.items():
        got = rows[i].astype(np.float64)
        assert np.max(np.abs(got - want)) <= TOL * scale, (isa, i)
        assert not got[0].any(), isa                    # zero input -> zero row
    if "avx512-vnni" in paths and "avx2" in paths:       # the same lanes in the same order
        assert np.array_equal(paths["avx512-vnni"][i], paths["avx2"][i])


def test_host_rows_argument_checks():
    e = np.zeros(synth.expert_bytes(256, 128, synth.Q8_0), np.uint8)
    x = np.zeros((2, 256), np.float32)
    with pytest.raises(abi.MoeError):
        abi.cpu_expert_rows(7, 256, 128, e, x)           # unknown type
    with pytest.raises(abi.MoeError):
        abi.cpu_expert_rows(synth.Q8_0, 200, 128, e, np.zeros((2, 200), np.float32))
