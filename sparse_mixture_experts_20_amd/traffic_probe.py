"""Workload for HBM-traffic counters: a plain device copy of known size (the
calibration) followed by a few layer forwards.

Run it under ``rocprofv3 --pmc FETCH_SIZE`` (and separately ``WRITE_SIZE``):
the copy's counter reading against its 1 GiB read and 1 GiB written gives the
counter-to-bytes factor applied to the layer's kernels.
"""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from sparse_mixture_experts_20_amd import binding as B
from sparse_mixture_experts_20_amd import device as D
from sparse_mixture_experts_20_amd import workloads as W

COPY_BYTES = 1 << 30


def main(workload: str = "nanomoe", steps: int = 3) -> None:
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    wl = W.make(workload)
    dev = D.upload(wl)
    fwd = B.Forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                    wl.cfg.cf)
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    print(f"traffic probe done: {workload}, {steps} forwards", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "nanomoe")
