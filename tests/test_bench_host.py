"""Host-side logic of the benchmark (no GPU): the command-line contract and
the expert-kernel names it looks up for its roofline and traffic entries."""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_mixture_experts_20_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("name", ["nanomoe", "mixtral", "skew", "finegrained", "nanomoe_gelu"])
def test_kernel_names_come_from_the_library(name):
    """bench.py names the roofline kernel with the library's own query
    (moe_expert_kernel_name, host-only); where the committed counter summary
    (profiles/traffic.json) was taken from the current expert-kernel source,
    those names are the ones rocprofv3 recorded for that workload."""
    cfg = W.CONFIGS[name]
    # the sizes only: no tensors are generated
    wl = types.SimpleNamespace(cfg=cfg, N=cfg.N, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff)
    names = [bench.gemm_kernel_name(wl, mode) for mode in (0, 1)]
    for mode, n in enumerate(names):
        assert n.startswith("expert_gemm_kernel<") and n.endswith(f", {mode}>"), n
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    sha = bench.source_sha(bench.GEMM_SRC)
    current = {k.rsplit("/", 1)[0] for k, v in t.items()
               if k.endswith("/" + name) and "gemm" in k and v.get("source_sha") == sha}
    if current:
        for n in names:
            assert n in current, (name, n)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_dropout_needs_a_training_pass():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--dropout", "0.1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--dropout" in r.stderr
