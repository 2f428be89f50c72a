"""Copy a seeded workload into device memory (torch is the allocator only).

Expert weights are generated on a host thread pool one expert at a time and
copied straight into the [E, d_ff, d] / [E, d, d_ff] device tensors, so the
host never holds more than a few experts unless the workload caches them.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(wl, device="cuda", threads: int = 16, keep_host: bool = False) -> dict:
    """Device tensors for ``wl``: x, W_g, noise (or None), W_up, W_down, the
    expert biases b_up, b_down (fp32, or None) and the activation name.

    With ``keep_host`` the generated expert matrices are also memoised in the
    workload so that later CPU-side consumers do not regenerate them."""
    dt = torch.bfloat16 if wl.cfg.dtype == "bf16" else torch.float32
    E, d, d_ff = wl.E, wl.d, wl.d_ff
    out = {
        "x": _t(wl.x, device),
        "W_g": _t(wl.wg, device),
        "noise": None if wl.noise is None else _t(wl.noise, device),
        "W_up": torch.empty((E, d_ff, d), dtype=dt, device=device),
        "W_down": torch.empty((E, d, d_ff), dtype=dt, device=device),
        "b_up": None if wl.b_up() is None else _t(wl.b_up(), device),
        "b_down": None if wl.b_down() is None else _t(wl.b_down(), device),
        "act": wl.cfg.act,
    }
    for which, key in (("up", "W_up"), ("down", "W_down")):
        for e, a in wl.experts(which, threads):
            out[key][e].copy_(_t(a, "cpu"))
            if keep_host:
                wl.memo(which, e, a)
    torch.cuda.synchronize()
    return out
