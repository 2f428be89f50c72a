"""Training-mode dropout on the expert outputs, HIP path against the oracle.

The keep/drop decision of every element is an integer comparison of a
Philox4x64-10 word on both sides, so the dropped positions must match
exactly; the kept values carry the usual bf16 / fp32 tolerances. The
backward through the same mask is compared like the other backward cases
(relative L2 <= 2e-2, max error <= 5e-2 of the largest entry)."""
import numpy as np
import pytest

import oracle
from sparse_mixture_experts_20_amd import workloads as W
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_mod():
    if not G.have_gpu():
        pytest.skip("no HIP device")
    import torch
    from sparse_mixture_experts_20_amd import binding as B
    B.lib()
    return torch


def _upload(wl):
    import torch
    from sparse_mixture_experts_20_amd import device as D
    dev = D.upload(wl, keep_host=True)
    dev["dout"] = torch.from_numpy(wl.dout().view(np.int16) if wl.cfg.dtype == "bf16"
                                   else wl.dout()).to("cuda")
    if wl.cfg.dtype == "bf16":
        dev["dout"] = dev["dout"].view(torch.bfloat16)
    return dev


def _drop(wl):
    return (wl.cfg.dropout, wl.cfg.dropout_seed, wl.cfg.dropout_offset)


# name -> (N, d, E, k, d_ff, dtype, cf, seed, act, bias_std, p, dseed, doffset)
CASES = {
    "drop_bf16": (333, 136, 5, 2, 200, "bf16", 1.0, 401, "relu", 0.0, 0.1, 17, 0),
    "drop_gelu_bias_bf16": (700, 200, 6, 2, 328, "bf16", 0.9, 402, "gelu", 0.05, 0.3, 2**40 + 3,
                            5),
    "drop_f32": (77, 13, 6, 3, 21, "f32", 0.7, 403, "relu", 0.3, 0.5, 9, 2**33),
    "drop_multi_tile_bf16": (1000, 264, 16, 4, 392, "bf16", 0.8, 404, "relu", 0.0, 0.05, 1, 1),
    # the 320-row tile's dropout epilogue (256 expected rows per expert)
    "drop_tile320_bf16": (2048, 264, 64, 8, 392, "bf16", 1.5, 406, "relu", 0.0, 0.1, 5, 7),
}


def _wl(name):
    N, d, E, k, d_ff, dt, cf, seed, act, bstd, p, ds, do = CASES[name]
    return W.custom(name, N=N, d=d, E=E, k=k, d_ff=d_ff, dtype=dt, cf=cf, sigma=0.3, seed=seed,
                    w_std=0.05, act=act, bias_std=bstd, dropout=p, dropout_seed=ds,
                    dropout_offset=do)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_with_dropout_matches_oracle(torch_mod, name):
    torch = torch_mod
    from sparse_mixture_experts_20_amd import binding as B
    wl = _wl(name)
    G.say(f"[dropout] {name}: N={wl.N} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff} "
          f"{wl.cfg.dtype} p={wl.cfg.dropout}")
    dev = _upload(wl)
    out, st = B.forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                        wl.cfg.cf, export=True, act=dev["act"], b_up=dev["b_up"],
                        b_down=dev["b_down"], dropout=_drop(wl))
    # the experts' rows through the stage entry points, for the exact mask
    ceff = min(st.capacity, wl.N)
    slot, used, slot_token, tiles = B.dispatch(st.idx, wl.E, st.capacity)
    H, Y = B.experts(dev["x"], dev["W_up"], dev["W_down"], wl.k, st.capacity, used, slot_token,
                     tiles, act=dev["act"], b_up=dev["b_up"], b_down=dev["b_down"],
                     dropout=_drop(wl))
    torch.cuda.synchronize()
    res = oracle.forward(wl, want_y=True)
    G.check_routing(res, st)
    G.check_out(wl.cfg.dtype, G.out_f64(wl, out), res.out)
    # dropped positions: exactly where the oracle's mask drops (kept rows only)
    y_ref = res.y.reshape(wl.N * wl.k, wl.d)
    arows = np.arange(wl.N * wl.k)
    keep_ref = oracle.dropout_rows(np.ones((wl.N * wl.k, wl.d)), arows, wl.cfg.dropout,
                                   wl.cfg.dropout_seed, wl.cfg.dropout_offset) != 0.0
    kept_assign = (res.slot.reshape(-1) >= 0)
    y_gpu = G.f64(Y)[kept_assign]
    yr = y_ref[kept_assign]
    kr = keep_ref[kept_assign]
    assert np.all(y_gpu[~kr] == 0.0)                       # dropped: exactly 0
    assert np.all(y_gpu[kr & (np.abs(yr) > 1e-20)] != 0.0)  # kept: there
    rel = np.linalg.norm(y_gpu - yr) / np.linalg.norm(yr)
    assert rel <= (1e-2 if wl.cfg.dtype == "bf16" else 1e-5), rel
    frac = 1.0 - kr.mean()
    G.say(f"    dropped fraction {frac:.4f} (p={wl.cfg.dropout})")
    del dev


@pytest.mark.parametrize("name", [n for n in CASES if CASES[n][5] == "bf16"])
def test_backward_with_dropout_matches_oracle(torch_mod, name):
    torch = torch_mod
    from sparse_mixture_experts_20_amd import binding as B
    wl = _wl(name)
    G.say(f"[dropout] backward {name}: p={wl.cfg.dropout}")
    dev = _upload(wl)
    grads, st = B.backward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                           wl.cfg.cf, dev["dout"], export=True, act=dev["act"],
                           b_up=dev["b_up"], b_down=dev["b_down"], dropout=_drop(wl))
    torch.cuda.synchronize()
    res = oracle.forward(wl, rows=[0])
    G.check_routing(res, st)
    wu = np.stack([wl.as_f64(wl.w_up(e)) for e in range(wl.E)])
    wd = np.stack([wl.as_f64(wl.w_down(e)) for e in range(wl.E)])
    ref = oracle.backward(wl.x64(), wl.wg64(), wl.noise64(), wu, wd, wl.k, wl.cfg.cf,
                          wl.as_f64(wl.dout()), act=wl.cfg.act, bup64=wl.b_up(),
                          bdown64=wl.b_down(), dropout=wl.cfg.dropout,
                          seed=wl.cfg.dropout_seed, offset=wl.cfg.dropout_offset)
    assert len(grads) == len(ref)
    for nm, got, r in zip(("dx", "dW_g", "dW_up", "dW_down", "db_up", "db_down"), grads, ref):
        r = np.asarray(r)
        g = G.to_np(got).astype(np.float64)
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        err = np.abs(g - r).max()
        G.say(f"    {nm}: rel_l2={rel:.2e} max_abs={err:.2e} max_ref={np.abs(r).max():.2e}")
        assert rel <= 2e-2 and err <= 5e-2 * np.abs(r).max(), nm
    del dev


def _sampled_case(which):
    import dataclasses
    if which == "nanomoe":
        base = W.make("nanomoe").cfg
        return W.make(dataclasses.replace(base, name="nanomoe_dropout", dropout=0.1,
                                          dropout_seed=2026, dropout_offset=3))
    # 512 rows per expert and d = 2048: the down product (and its dropout)
    # runs on the 256x256 tile, as at the Mixtral shape
    return W.custom("wide_dropout", N=2048, d=2048, E=8, k=2, d_ff=1024, dtype="bf16", cf=1.25,
                    sigma=0.3, seed=405, w_std=0.03, dropout=0.1, dropout_seed=2026,
                    dropout_offset=3)


@pytest.mark.parametrize("which", ["nanomoe", "wide"])
def test_dropout_sampled(torch_mod, which):
    """Dropout 0.1 on the nanoMoE layer (128x64 down tiles) and on a layer
    whose down product takes the 256x256 tile: layer output on sampled rows
    and dx on sampled rows, in the benchmark's launch configuration."""
    torch = torch_mod
    from sparse_mixture_experts_20_amd import binding as B
    wl = _sampled_case(which)
    dev = _upload(wl)
    out, st = B.forward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                        wl.cfg.cf, export=True, dropout=_drop(wl))
    grads = B.backward(dev["x"], dev["W_g"], dev["noise"], dev["W_up"], dev["W_down"], wl.k,
                       wl.cfg.cf, dev["dout"], dropout=_drop(wl))
    torch.cuda.synchronize()
    route = oracle.forward(wl, rows=[0])
    rows = G.sample_rows(route, 64, seed=4)
    res = oracle.forward(wl, rows=rows)
    G.check_routing(res, st)
    G.check_out("bf16", G.out_f64(wl, out, rows), res.out)
    wu = np.stack([wl.as_f64(wl.w_up(e)) for e in range(wl.E)])
    wd = np.stack([wl.as_f64(wl.w_down(e)) for e in range(wl.E)])
    ref = oracle.backward_rows(wl.x64(), wl.wg64(), wl.noise64(), wu, wd, wl.k, wl.cfg.cf,
                               wl.as_f64(wl.dout()), rows, dropout=0.1, seed=2026, offset=3)
    g = G.to_np(grads[0])[rows].astype(np.float64)
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    G.say(f"    dx[rows]: rel_l2={rel:.2e}")
    assert rel <= 2e-2 and np.abs(g - ref).max() <= 5e-2 * np.abs(ref).max()
    del dev
