"""bench.py contract checks that need no GPU.

* More than one GPU is refused with a message and a non-zero exit, before any
  device work.
* The step's GEMM work is the 12 GEMMs of one decoder layer at M = 4096:
  sum of 2*M*N*K over fwd, dgrad and wgrad of the four linears = 1236.95 GFLOP.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_layer_gemm_work_at_m4096():
    sys.path.insert(0, ROOT)
    from blockwise_fp8_linear_quant_amd import workloads as W
    M = 4096
    flops = sum(3 * 2 * M * n_out * k for _, k, n_out in W.LINEARS)
    assert flops == 1236950581248
    shapes = {name: (k, n_out) for name, k, n_out in W.LINEARS}
    assert shapes == {"qkv": (2048, 4096), "o": (2048, 2048), "gate_up": (2048, 12288), "down": (6144, 2048)}
