"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases compare every output element; the five layer shapes of the
benchmark table compare routing, slots, drops and the router statistics for
all tokens and the layer output, in the launch configuration the benchmark
times, on every token row except at the fine-grained layer (256 experts,
15 GB of weights), where it is compared on the tokens that hold the first and
last kept row of every (expert, 128-row tile) of the expert products.
"""
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


def _upload(wl, keep_host=False):
    from sparse_mixture_experts_20_amd import device as D
    dev = D.upload(wl, keep_host=keep_host)
    dev["k"], dev["cf"] = wl.k, wl.cfg.cf
    return dev


def _free(torch, *objs):
    for o in objs:
        del o
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# name -> (N, d, E, k, d_ff, dtype, cf, sigma, bias0, seed)
SMALL = {
    "ragged_bf16": (333, 136, 5, 2, 200, "bf16", 1.0, 0.3, 0.0, 101),
    "multi_tile_bf16": (1000, 264, 16, 4, 392, "bf16", 0.8, 0.5, 0.0, 102),
    "many_experts_bf16": (300, 128, 256, 8, 96, "bf16", 2.0, 0.0, 0.0, 103),
    "mid_bf16": (1536, 512, 8, 2, 1024, "bf16", 1.25, 1.0, 0.0, 104),
    # about one 128x128 tile per CU in both products: the two-K-set tile,
    # with K tails (392, 520 = 128 q + 8), ragged columns and part-filled rows
    "kset_bf16": (1024, 392, 64, 4, 520, "bf16", 1.0, 0.5, 0.0, 114),
    # at least 384 tiles of 128x128 with few rows per expert: the plain
    # 128x128 tile (two workgroups per CU) in both products, ragged K and N
    # (weights scaled down, see W_STD)
    "plain128_bf16": (1024, 1544, 32, 2, 1544, "bf16", 1.0, 0.5, 0.0, 115),
    # 256 expected rows per expert: the 320-row tile in both products (the
    # kernel's own schedule prefix), K tails (264, 392), a partial column
    # tile (392) and one expert at capacity (384 rows: a second row tile)
    "tile320_bf16": (2048, 264, 64, 8, 392, "bf16", 1.5, 0.3, 0.5, 116),
    # the 320-row tile with few experts (fewer tiles than workgroups)
    "tile320_e8_bf16": (1024, 264, 8, 2, 392, "bf16", 1.25, 0.3, 0.0, 117),
    "k1_bf16": (200, 64, 3, 1, 64, "bf16", 1.0, 0.0, 0.0, 105),
    "k_equals_E_bf16": (100, 32, 4, 4, 48, "bf16", 1.0, 0.0, 0.0, 106),
    "max_top_k_bf16": (200, 64, 64, 16, 72, "bf16", 0.7, 0.2, 0.0, 112),
    "max_top_k_f32": (40, 24, 20, 16, 40, "f32", 1.0, 0.2, 0.0, 113),
    "ragged_f32": (77, 13, 6, 3, 21, "f32", 0.7, 0.5, 0.0, 107),
    "heavy_drop_bf16": (512, 64, 4, 2, 128, "bf16", 0.1, 0.0, 5.0, 108),
    "single_token_bf16": (1, 64, 8, 2, 64, "bf16", 1.0, 0.0, 0.0, 109),
    "one_expert_bf16": (50, 32, 1, 1, 40, "bf16", 1.0, 0.0, 0.0, 110),
    "wide_f32": (40, 96, 12, 3, 160, "f32", 1.5, 0.2, 0.0, 111),
}


# the nanoMoE slides' expert variant (slide 32): biases, GELU
# name -> (N, d, E, k, d_ff, dtype, cf, sigma, seed, act, bias_std)
VARIANT = {
    "gelu_bias_f32": (77, 13, 6, 3, 21, "f32", 0.7, 0.5, 201, "gelu", 0.3),
    "gelu_bias_bf16": (700, 200, 6, 2, 328, "bf16", 0.9, 0.4, 202, "gelu", 0.05),
    "relu_bias_bf16": (1000, 264, 16, 4, 392, "bf16", 0.8, 0.5, 203, "relu", 0.05),
    "gelu_nobias_bf16": (333, 136, 5, 2, 200, "bf16", 1.0, 0.3, 204, "gelu", 0.0),
    "gelu_bias_tile320_bf16": (2048, 264, 64, 8, 392, "bf16", 1.5, 0.3, 205, "gelu", 0.05),
}


# Weight scale of the small layers (0.05 unless listed): the wide layer's
# outputs would otherwise reach |out| ~ 10, where bf16 rounding alone (about
# 3 * 2^-9 of the value at worst) exceeds the absolute bound of the check.
W_STD = {"plain128_bf16": 0.02}


def _small(name):
    if name in VARIANT:
        N, d, E, k, d_ff, dt, cf, sg, seed, act, bstd = VARIANT[name]
        return W.custom(name, N=N, d=d, E=E, k=k, d_ff=d_ff, dtype=dt, cf=cf, sigma=sg,
                        seed=seed, w_std=0.05, act=act, bias_std=bstd)
    if name == "tiny":
        return W.make("tiny")
    if name == "router_example":
        return W.router_example()
    if name == "capacity_example":
        return W.capacity_example()
    N, d, E, k, d_ff, dt, cf, sg, b0, seed = SMALL[name]
    return W.custom(name, N=N, d=d, E=E, k=k, d_ff=d_ff, dtype=dt, cf=cf, sigma=sg, bias0=b0,
                    seed=seed, w_std=W_STD.get(name, 0.05))


@pytest.mark.parametrize("name", ["tiny", "router_example", "capacity_example"] + list(SMALL) +
                         list(VARIANT))
def test_small_layer_matches_oracle(torch_mod, name):
    torch = torch_mod
    wl = _small(name)
    G.say(f"[parity] {name}: N={wl.N} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff} "
          f"{wl.cfg.dtype} cf={wl.cfg.cf} act={wl.cfg.act} bias_std={wl.cfg.bias_std}")
    res = oracle.forward(wl)
    dev = _upload(wl)
    out, st = G.run_forward(dev)
    torch.cuda.synchronize()
    G.check_routing(res, st)
    G.check_router_stats(res, st)
    got = G.out_f64(wl, out)
    G.check_out(wl.cfg.dtype, got, res.out)
    alldrop = (res.slot < 0).all(axis=1)
    assert np.all(got[alldrop] == 0.0)
    if name == "capacity_example":
        assert res.drops == 5 and alldrop.sum() == 2
    if name == "heavy_drop_bf16":
        assert alldrop.sum() > 0
    _free(torch, dev, out)


# (workload, rows checked): every token, except at the fine-grained layer,
# where the rows are the strata of every (expert, 128-row tile)
FULL = [("nanomoe", "all"), ("mixtral", "all"), ("skew", "all"), ("finegrained", "strata"),
        ("nanomoe_gelu", "all")]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rows_mode", FULL)
def test_benchmark_layer_matches_oracle(torch_mod, name, rows_mode):
    torch = torch_mod
    wl = W.make(name)
    G.say(f"[parity] {name}: N={wl.N} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff}")
    dev = _upload(wl, keep_host=True)
    out, st = G.run_forward(dev)
    torch.cuda.synchronize()
    route = oracle.forward(wl, rows=[0])
    G.check_routing(route, st)
    G.check_router_stats(route, st)
    rows, pairs = G.strata_rows(route)
    if rows_mode == "all":
        rows = np.arange(wl.N)
    G.say(f"[parity] {name}: routing and router statistics exact; oracle on {len(rows)} rows "
          f"covering all {pairs} (expert, 128-row tile) pairs with kept rows")
    res = oracle.forward(wl, rows=rows)
    err = G.check_out(wl.cfg.dtype, G.out_f64(wl, out, rows), res.out)
    G.say(f"[parity] {name}: drops={res.drops} rows={len(rows)} max_abs_err={err:.3e}")
    if name == "skew":
        assert res.drops > 8000 and res.used[0] == res.C
    else:
        assert res.drops == 0
    _free(torch, dev, out)


def _tied_layer(name, E, k, dtype, N=512, d_ff=64, seed=701):
    """W_g = I (d = E) and token entries from {-1, -0.5, 0, 0.5, 1}: the
    scores are the entries themselves, so many tokens have exactly equal
    scores inside and at the edge of their top-k."""
    rng = np.random.default_rng(seed)
    x32 = rng.choice(np.array([-1.0, -0.5, 0.0, 0.5, 1.0], np.float32), size=(N, E))
    cfg = W.Config(name, N=N, d=E, E=E, k=k, d_ff=d_ff, dtype=dtype, cf=1.5, w_std=0.05,
                   seed=seed)
    x = W.f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    return W.Workload(cfg, x, np.eye(E, dtype=np.float32), None, seed)


@pytest.mark.parametrize("E,k,dtype", [(16, 4, "bf16"), (32, 3, "bf16"), (256, 8, "bf16"),
                                       (12, 4, "f32")])
def test_tied_scores_rank_lower_id_first(torch_mod, E, k, dtype):
    """Exactly tied scores (nanoMoE slide 12's top-k; equal scores take the
    lower expert id first) on each router path: the fused kernel for up to 16
    and up to 32 experts, the score product + ranking for 256, and fp32.
    Ids, slots and drops bit-exact against the oracle, outputs in tolerance."""
    torch = torch_mod
    wl = _tied_layer(f"ties_{E}_{dtype}", E, k, dtype)
    res = oracle.forward(wl)
    s = np.sort(res.scores, axis=1)[:, ::-1]
    ties = int(((s[:, :k] == s[:, 1:k + 1])).any(axis=1).sum())
    G.say(f"[parity] ties E={E} k={k} {dtype}: {ties} of {wl.N} tokens with a tie in the "
          f"top-{k + 1}")
    assert ties > wl.N // 2
    dev = _upload(wl)
    out, st = G.run_forward(dev)
    torch.cuda.synchronize()
    G.check_routing(res, st)
    G.check_router_stats(res, st)
    G.check_out(dtype, G.out_f64(wl, out), res.out)
    _free(torch, dev, out)


def test_light_tiles_last_with_split(torch_mod):
    """A layer whose up product (256x256 tiles: 288, of which 192 heavy) and
    down product (128x128 in two K sets: 320, of which 256 heavy) both
    overflow one round of 256 workgroups while their heavy tiles fit, and
    both cut their last round into K-ranges: the light last row tiles run
    last and are the ones the fix-up sums. Every token with a choice in an
    expert's last row tile (rank 512 or more) is compared, with random
    others."""
    torch = torch_mod
    wl = W.custom("light_last_split", N=2200, d=1024, E=8, k=2, d_ff=3072, dtype="bf16",
                  cf=1.25, sigma=0.3, seed=601, w_std=0.03)
    dev = _upload(wl, keep_host=True)
    out, st = G.run_forward(dev)
    torch.cuda.synchronize()
    route = oracle.forward(wl, rows=[0])
    assert sorted(route.used.tolist())[0] > 512   # three row tiles of 256 per expert
    late = np.nonzero((route.slot >= 512).any(axis=1))[0]
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([late, rng.choice(wl.N, size=64, replace=False)]))
    G.say(f"[parity] light_last_split: {len(late)} tokens in last row tiles, {len(rows)} rows")
    res = oracle.forward(wl, rows=rows)
    G.check_routing(res, st)
    G.check_out("bf16", G.out_f64(wl, out, rows), res.out)
    _free(torch, dev, out)


def test_compact_rows_keep_every_magnitude(torch_mod):
    """A bf16 layer keeps its experts' output rows as fp16 values with one
    power-of-two shift per 32 columns. Experts whose outputs lie far above
    fp16's range (W_down scaled by 2^24 and 2^60), far below it (2^-80,
    2^-90) and at ordinary magnitudes share one layer whose width (d = 200)
    leaves a partial last group of 8 columns; every token row matches the
    oracle relative to its own largest output (a token may mix experts of
    very different scales), and rows of ordinary magnitude within the
    layer's absolute bound."""
    torch = torch_mod
    wl = W.custom("compact_range", N=600, d=200, E=6, k=2, d_ff=136, dtype="bf16", cf=1.0,
                  sigma=0.3, seed=77, w_std=0.05)
    scale = [2.0**24, 2.0**-90, 1.0, 2.0**60, 2.0**-80, 1.0]
    for e in range(wl.E):
        w = W.bf16_bits_to_f32(wl.w_down(e)) * np.float32(scale[e])   # exact: powers of two
        wl.memo("down", e, W.f32_to_bf16_bits(w))
    G.say("[parity] compact_range: W_down scaled by 2^24, 2^-90, 1, 2^60, 2^-80, 1")
    res = oracle.forward(wl)
    dev = _upload(wl)
    out, st = G.run_forward(dev)
    torch.cuda.synchronize()
    G.check_routing(res, st)
    got = G.out_f64(wl, out)
    assert np.all(np.isfinite(got))
    peak = np.abs(res.out).max(axis=1)
    live = peak > 0
    err = np.abs(got - res.out).max(axis=1)
    assert np.all(err[live] <= 8e-3 * peak[live]), (err / np.maximum(peak, 1e-300)).max()
    assert np.all(got[~live] == 0.0)
    # both ends of the range are exercised, and rows of ordinary size
    assert peak.max() > 1e15 and peak[live].min() < 1e-20
    plain = (peak > 1e-3) & (peak < 1e3)
    assert plain.sum() > 0
    G.check_out("bf16", got[plain], res.out[plain])
    _free(torch, dev, out)


def test_forward_is_deterministic(torch_mod):
    torch = torch_mod
    wl = W.make("nanomoe")
    dev = _upload(wl)
    o1, s1 = G.run_forward(dev)
    o2, s2 = G.run_forward(dev)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1.slot, s2.slot) and torch.equal(s1.used, s2.used)
    assert torch.equal(s1.gate, s2.gate)
    _free(torch, dev)


def test_empty_call(torch_mod):
    torch = torch_mod
    from sparse_mixture_experts_20_amd import binding as B
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    wu = torch.zeros((4, 32, 64), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((4, 64, 32), dtype=torch.bfloat16, device="cuda")
    out, st = B.forward(x, wg, None, wu, wd, 2, 1.0, export=True)
    torch.cuda.synchronize()
    assert st.capacity == 0 and out.shape == (0, 64)
    assert int(st.used.abs().sum()) == 0
