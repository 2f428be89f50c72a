"""Workload for HBM-traffic counters: a plain device copy of known size (the
calibration) followed by a few layer forwards.

Run it under ``rocprofv3 --pmc FETCH_SIZE`` (and separately ``WRITE_SIZE``):
the copy's counter reading against its 1 GiB read and 1 GiB written gives the
counter-to-bytes factor applied to the layer's kernels.
"""
import json
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from sparse_mixture_experts_20_amd import binding as B
from sparse_mixture_experts_20_amd import device as D
from sparse_mixture_experts_20_amd import workloads as W

COPY_BYTES = 1 << 30


def main(workload: str = "nanomoe", steps: int = 3, info_path: str = "") -> None:
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    wl = W.make(workload)
    dev = D.upload(wl)
    fwd = B.Forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                    wl.cfg.cf, export=True, act=dev["act"],
                    b_up=dev["b_up"], b_down=dev["b_down"])
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    if info_path:
        # sizes and kept assignments, for the algorithmic byte counts
        info = {"workload": workload, "N": wl.N, "d": wl.d, "E": wl.E, "k": wl.k,
                "d_ff": wl.d_ff, "dtype": wl.cfg.dtype, "noise": dev["noise"] is not None,
                "kept": int(fwd.used.sum().item()), "steps": steps}
        with open(info_path, "w") as f:
            json.dump(info, f)
    print(f"traffic probe done: {workload}, {steps} forwards", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "nanomoe", 3,
         sys.argv[2] if len(sys.argv) > 2 else "")
