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
import oracle  # noqa: E402
from sparse_mixture_experts_20_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("name", ["nanomoe", "mixtral", "skew", "finegrained", "nanomoe_gelu"])
def test_kernel_names_match_the_profiled_kernels(name):
    """The names bench.py derives from the library's tile rule are the ones
    rocprofv3 recorded for that workload (profiles/traffic.json), so the
    roofline's kernel and traffic lookups refer to kernels that ran."""
    with open(bench.TRAFFIC_FILE) as f:
        recorded = {k.rsplit("/", 1)[0] for k in json.load(f) if k.endswith("/" + name)}
    cfg = W.CONFIGS[name]
    # the sizes only: no tensors are generated
    wl = types.SimpleNamespace(cfg=cfg, N=cfg.N, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff)
    C = oracle.capacity(cfg.N, cfg.E, cfg.k, cfg.cf)
    for mode in (0, 1):
        assert bench.gemm_kernel_name(wl, C, mode) in recorded, (name, mode)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_dropout_needs_a_training_pass():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--dropout", "0.1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--dropout" in r.stderr
