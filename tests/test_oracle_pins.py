"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print for their worked examples (tests/golden), closed forms, special
cases that reduce to a textbook computation, invariants, and an independent
brute force on tiny inputs. These run on the CPU only.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_mixture_experts_20_amd import workloads as W
from tests import _bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _fixed_workload(name, x, wg, k, cf, wups, wdowns, noise=None, dtype="f32"):
    x = np.asarray(x, np.float32)
    N, d = x.shape
    E = wg.shape[0]
    cfg = W.Config(name, N=N, d=d, E=E, k=k, d_ff=wups[0].shape[0], dtype=dtype, cf=cf)
    return W.Workload(cfg, x, np.asarray(wg, np.float32), noise, 0,
                      fixed_experts=([np.asarray(a, np.float32) for a in wups],
                                     [np.asarray(a, np.float32) for a in wdowns]))


def _bf_inputs(wl):
    wups = [wl.as_f64(wl.w_up(e)) for e in range(wl.E)]
    wdowns = [wl.as_f64(wl.w_down(e)) for e in range(wl.E)]
    return wl.x64(), wl.wg64(), wl.noise64(), wups, wdowns


# ----------------------------------------------------------------------------
# worked examples printed on the pages
# ----------------------------------------------------------------------------
def test_router_example_matches_slides():
    """nanoMoE slides 11-13: kept experts and gates (3 decimals) of 8 tokens."""
    rows = _rows("router_example.txt")
    wl = W.router_example()
    r = oracle.forward(wl)
    assert len(rows) == wl.N == 8
    for t, row in enumerate(rows):
        assert int(row[0]) == t
        logits = [float(v) for v in row[1:4]]
        np.testing.assert_array_equal(wl.x[t], np.float32(logits))
        kept = [int(row[4]), int(row[5])]
        gates = [float(row[6]), float(row[7])]
        assert sorted(r.idx[t].tolist()) == kept
        by_expert = dict(zip(r.idx[t].tolist(), r.gate[t].tolist()))
        for e, g in zip(kept, gates):
            assert round(by_expert[e], 3) == pytest.approx(g, abs=1e-12), (t, e)
        # descending order: the first choice has the larger gate
        assert r.gate[t, 0] > r.gate[t, 1]


def test_capacity_example_matches_slides():
    """nanoMoE slides 15-29 and 34-40: slots, keep flags, used, drops, reach."""
    rows = _rows("capacity_example.txt")
    idx = [[int(v) for v in r[1:]] for r in rows if r[0] == "idx"]
    keep = [[int(v) for v in r[1:]] for r in rows if r[0] == "keep"]
    used = [int(v) for v in next(r for r in rows if r[0] == "used")[1:]]
    drops = int(next(r for r in rows if r[0] == "drops")[1])
    reach = {int(r[1]): sorted(int(v) for v in r[2:]) for r in rows if r[0] == "reach"}

    wl = W.capacity_example()
    r = oracle.forward(wl, want_y=True)
    assert r.C == 1
    np.testing.assert_array_equal(r.idx, np.array(idx))
    kept = (r.slot >= 0).astype(int).T  # [k, N] like the slides
    np.testing.assert_array_equal(kept, np.array(keep))
    assert r.used.tolist() == used
    assert r.drops == drops
    # every kept assignment holds slot 0 (capacity 1)
    assert set(r.slot[r.slot >= 0].tolist()) == {0}
    # output structure
    for t in range(wl.N):
        reached = sorted(int(e) for e, s in zip(r.idx[t], r.slot[t]) if s >= 0)
        assert reached == reach[t]
    assert np.all(r.out[2] == 0.0) and np.all(r.out[3] == 0.0)
    # token 1: only its second choice (expert 2) survives, scaled by its raw gate
    x64, wg64, n64, wups, wdowns = _bf_inputs(wl)
    y2 = BF.expert_all_tokens(x64[1:2], wups[2], wdowns[2])[0]
    np.testing.assert_allclose(r.out[1], r.gate[1, 1] * y2, rtol=1e-13, atol=1e-14)
    # token 0: both choices survive; with no renormalisation the gates sum to 1
    y0 = BF.expert_all_tokens(x64[0:1], wups[0], wdowns[0])[0]
    y1 = BF.expert_all_tokens(x64[0:1], wups[1], wdowns[1])[0]
    np.testing.assert_allclose(r.out[0], r.gate[0, 0] * y0 + r.gate[0, 1] * y1,
                               rtol=1e-13, atol=1e-14)


def test_router_stats_match_the_capacity_example():
    """Router statistics on the slides' capacity example (slides 15-29):
    demand [4, 2, 2] before the mask, drops [3, 1, 1]; each token's gates sum
    to one, so the gate sums add up to the token count."""
    rows = _rows("capacity_example.txt")
    demand = [int(v) for v in next(r for r in rows if r[0] == "demand")[1:]]
    drops = [int(v) for v in next(r for r in rows if r[0] == "expert_drops")[1:]]
    wl = W.capacity_example()
    r = oracle.forward(wl)
    assert r.demand.tolist() == demand
    assert r.expert_drops.tolist() == drops
    assert (r.demand - r.used).tolist() == drops
    assert r.gate_sum.sum() == pytest.approx(wl.N, abs=1e-12)
    # expert 0 is every token's first choice here
    np.testing.assert_allclose(r.gate_sum[0], r.gate[:, 0].sum(), rtol=0, atol=1e-15)


@pytest.mark.parametrize("N,E,k,cf,sigma,seed", [(300, 6, 2, 0.5, 0.5, 41),
                                                 (257, 16, 4, 1.0, 1.0, 42),
                                                 (64, 5, 5, 0.3, 0.0, 43)])
def test_router_stats_invariants(N, E, k, cf, sigma, seed):
    """demand is the column sum of the dense one-hot of the ids (brute force),
    drops are exactly the assignments whose slot is -1, and gate_sum is the
    column sum of the dense [N, E] gate matrix (non-top-k entries 0)."""
    wl = W.custom("stats", N=N, d=12, E=E, k=k, d_ff=8, dtype="f32", cf=cf, sigma=sigma,
                  seed=seed)
    r = oracle.forward(wl, rows=[0])
    onehot = np.zeros((N, E), np.int64)
    dense = np.zeros((N, E))
    for t in range(N):
        for j in range(k):
            onehot[t, r.idx[t, j]] += 1
            dense[t, r.idx[t, j]] = r.gate[t, j]
    assert onehot.max() == 1   # distinct experts per token
    np.testing.assert_array_equal(r.demand, onehot.sum(axis=0))
    dropped = np.zeros(E, np.int64)
    for t in range(N):
        for j in range(k):
            if r.slot[t, j] < 0:
                dropped[r.idx[t, j]] += 1
    np.testing.assert_array_equal(r.expert_drops, dropped)
    np.testing.assert_allclose(r.gate_sum, dense.sum(axis=0), rtol=1e-13, atol=1e-13)
    assert int(r.demand.sum()) == N * k
    assert int(r.expert_drops.sum()) == r.drops
    assert r.gate_sum.sum() == pytest.approx(N, rel=1e-12)


# ----------------------------------------------------------------------------
# independent brute force (all experts, dense masked gates) on tiny inputs
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("N,d,E,k,d_ff,sigma,seed", [
    (8, 3, 4, 2, 4, 0.0, 11),
    (13, 5, 6, 3, 7, 0.7, 12),
    (20, 8, 5, 1, 9, 0.0, 13),
    (9, 4, 3, 3, 6, 1.0, 14),
    (31, 16, 8, 2, 24, 0.3, 15),
])
def test_oracle_equals_bruteforce_without_drops(N, d, E, k, d_ff, sigma, seed):
    wl = W.custom("bf", N=N, d=d, E=E, k=k, d_ff=d_ff, dtype="f32", cf=float(E),
                  sigma=sigma, seed=seed, w_std=0.5, wg_std=0.7)
    r = oracle.forward(wl)
    assert r.drops == 0
    x64, wg64, n64, wups, wdowns = _bf_inputs(wl)
    ref, G, order = BF.layer(x64, wg64, n64, k, wups, wdowns)
    np.testing.assert_array_equal(r.idx, order)
    scale = np.abs(ref).max()
    assert np.abs(r.out - ref).max() <= 1e-12 * max(scale, 1.0)
    # gates: exactly k nonzero, summing to one; masked experts are exactly 0
    assert np.all((G > 0).sum(axis=1) == k)
    np.testing.assert_allclose(G.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    dense = np.zeros((N, E))
    np.put_along_axis(dense, r.idx, r.gate, axis=1)
    np.testing.assert_allclose(dense, G, rtol=0, atol=1e-15)


def test_bf16_workload_equals_bruteforce():
    """bf16 inputs widen exactly: the oracle sees the rounded values."""
    wl = W.custom("bf16", N=24, d=16, E=4, k=2, d_ff=32, dtype="bf16", cf=4.0,
                  sigma=0.5, seed=21, w_std=0.3, wg_std=0.5)
    assert wl.x.dtype == np.uint16
    r = oracle.forward(wl)
    x64, wg64, n64, wups, wdowns = _bf_inputs(wl)
    ref, _, order = BF.layer(x64, wg64, n64, wl.k, wups, wdowns)
    np.testing.assert_array_equal(r.idx, order)
    assert np.abs(r.out - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1.0)


def test_page1_preset_token():
    """Page 1 preset: x = [1.2, -0.4, -0.8], k = 2, sigma = 0, four experts, 3->4->3."""
    wl = W.make("tiny")
    np.testing.assert_array_equal(wl.x[0], np.float32([1.2, -0.4, -0.8]))
    assert (wl.E, wl.k, wl.d, wl.d_ff) == (4, 2, 3, 4) and wl.noise is None
    r = oracle.forward(wl)
    assert r.drops == 0
    g = np.zeros(4)
    g[r.idx[0]] = r.gate[0]
    assert (g > 0).sum() == 2 and g.sum() == pytest.approx(1.0, abs=1e-15)
    x64, wg64, n64, wups, wdowns = _bf_inputs(wl)
    ref, _, _ = BF.layer(x64, wg64, n64, 2, wups, wdowns)
    np.testing.assert_allclose(r.out, ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# closed forms and textbook special cases
# ----------------------------------------------------------------------------
def test_identity_router_scores_are_the_input():
    """W_g = I (d = E): the scores are x itself (page 1 STEP 2 with unit rows)."""
    x = np.random.default_rng(3).standard_normal((17, 6)).astype(np.float32)
    scores, _, _ = oracle.router(x.astype(np.float64), np.eye(6), None, 2)
    np.testing.assert_array_equal(scores, x)


def test_identity_experts_return_the_token():
    """d_ff = d, W_up = W_down = I, x > 0: each expert is the identity, so with
    no drops y = sum g_i x = x (the gates sum to one, page 1 STEP 6)."""
    rng = np.random.default_rng(5)
    N, d, E, k = 12, 6, 4, 3
    x = np.abs(rng.standard_normal((N, d))).astype(np.float32) + 0.1
    wg = rng.standard_normal((E, d)).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    wl = _fixed_workload("identity", x, wg, k, float(E), [eye] * E, [eye] * E)
    r = oracle.forward(wl)
    assert r.drops == 0
    np.testing.assert_allclose(r.out, x.astype(np.float64), rtol=1e-14, atol=0)


def test_single_expert_is_a_dense_mlp():
    """E = 1, k = 1: gate exactly 1 and the layer is the plain 2-layer ReLU MLP."""
    rng = np.random.default_rng(6)
    N, d, d_ff = 10, 5, 7
    x = rng.standard_normal((N, d)).astype(np.float32)
    wg = rng.standard_normal((1, d)).astype(np.float32)
    wu = rng.standard_normal((d_ff, d)).astype(np.float32)
    wd = rng.standard_normal((d, d_ff)).astype(np.float32)
    wl = _fixed_workload("dense", x, wg, 1, 1.0, [wu], [wd])
    r = oracle.forward(wl)
    assert np.all(r.gate == 1.0) and np.all(r.idx == 0) and r.drops == 0
    x64 = x.astype(np.float64)
    mlp = np.maximum(x64 @ wu.astype(np.float64).T, 0) @ wd.astype(np.float64).T
    np.testing.assert_allclose(r.out, mlp, rtol=1e-13, atol=1e-13)


def test_k_equals_E_is_a_full_softmax():
    """k = E keeps every expert: the gates are the textbook softmax."""
    from scipy.special import softmax
    rng = np.random.default_rng(7)
    x = rng.standard_normal((15, 5))
    wg = rng.standard_normal((5, 5))
    scores, idx, gate = oracle.router(x, wg, None, 5)
    full = softmax(scores.astype(np.float64), axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, idx, axis=1), gate, rtol=1e-14, atol=0)
    assert np.all(np.diff(np.take_along_axis(scores, idx, axis=1), axis=1) < 0)


def test_k_one_gate_is_one():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((20, 4))
    wg = rng.standard_normal((6, 4))
    scores, idx, gate = oracle.router(x, wg, None, 1)
    assert np.all(gate == 1.0)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(scores, axis=1))


def test_noise_is_added_to_the_scores():
    """Page 1 STEP 4: s = s_raw + eps. A zero noise tensor equals no noise; a
    per-token constant shifts every score alike, leaving ids and gates alone
    (softmax shift invariance, STEP 6)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, 8))
    wg = rng.standard_normal((6, 8)) * 0.5
    eps = rng.standard_normal((40, 6))
    s0, i0, g0 = oracle.router(x, wg, None, 2)
    s1, i1, g1 = oracle.router(x, wg, np.zeros((40, 6)), 2)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_array_equal(g0, g1)
    s2, i2, g2 = oracle.router(x, wg, eps, 2)
    np.testing.assert_allclose(s2, (x @ wg.T + eps).astype(np.float32), rtol=0, atol=0)
    shift = np.repeat(rng.uniform(-3, 3, (40, 1)), 6, axis=1)
    s3, i3, g3 = oracle.router(x, wg, eps + shift, 2)
    np.testing.assert_array_equal(i2, i3)
    np.testing.assert_allclose(g2, g3, atol=2e-6)


def test_ties_rank_lower_index_first():
    x = np.array([[1.0, 1.0, 0.5, 1.0]])
    _, idx, gate = oracle.router(x, np.eye(4), None, 3)
    assert idx[0].tolist() == [0, 1, 3]
    np.testing.assert_allclose(gate[0], [1 / 3] * 3, rtol=1e-15)


# ----------------------------------------------------------------------------
# capacity and slots
# ----------------------------------------------------------------------------
def _ranks_by_cumsum(idx, E, C):
    """The slides' formulation (slide 14): one-hot of every choice laid out
    top-1 block first, a running count down that axis, minus one; kept where
    the rank is below capacity. Written with numpy array ops."""
    N, k = idx.shape
    onehot = np.zeros((k, N, E), np.int64)
    onehot[np.arange(k)[:, None], np.arange(N)[None, :], idx.T] = 1
    run = np.cumsum(onehot.reshape(k * N, E), axis=0).reshape(k, N, E) - 1
    keep = onehot * (run < C)
    rank = (keep * run).sum(axis=2)
    slot = np.where(keep.sum(axis=2) > 0, rank, -1).T
    return slot, keep.sum(axis=(0, 1))


@pytest.mark.parametrize("N,E,k,C,seed", [
    (50, 5, 3, 7, 1), (64, 4, 2, 1, 2), (33, 8, 1, 3, 3), (100, 3, 2, 80, 4), (7, 7, 7, 1, 5),
])
def test_slots_match_the_cumsum_formulation(N, E, k, C, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(N)]).astype(np.int32)
    slot, used = oracle.assign(idx, E, C)
    ref_slot, ref_used = _ranks_by_cumsum(idx, E, C)
    np.testing.assert_array_equal(slot, ref_slot)
    np.testing.assert_array_equal(used, ref_used)
    # invariants: each expert's kept slots are exactly 0..used-1, each once
    for e in range(E):
        s = np.sort(slot[(idx == e) & (slot >= 0)])
        np.testing.assert_array_equal(s, np.arange(used[e]))
    assert (slot >= 0).sum() + (slot < 0).sum() == N * k
    assert np.all(used <= C)


def test_top1_has_priority_over_top2():
    """Slide 19: splitting the ranks back into top-1 and top-2 blocks makes
    every first choice count before any second choice."""
    idx = np.array([[1, 0], [0, 1], [0, 1]], np.int32)
    slot, used = oracle.assign(idx, 2, 2)
    # expert 0: token 1 (top-1), token 2 (top-1) take slots 0, 1; token 0's
    # second choice is dropped although token 0 comes first
    assert slot.tolist() == [[0, -1], [0, 1], [1, -1]]
    assert used.tolist() == [2, 2]


def test_large_capacity_drops_nothing():
    rng = np.random.default_rng(10)
    idx = np.stack([rng.permutation(6)[:2] for _ in range(40)]).astype(np.int32)
    slot, used = oracle.assign(idx, 6, 80)
    assert np.all(slot >= 0) and used.sum() == 80


@pytest.mark.parametrize("N,E,k,cf", [
    (2048, 8, 2, 1.25), (4096, 8, 2, 1.25), (16384, 16, 2, 1.0), (8192, 256, 8, 1.5),
    (8, 4, 2, 8.0), (4, 3, 2, 0.375), (1000, 7, 3, 0.1), (5, 3, 1, 1e-6), (333, 5, 2, 1.1),
])
def test_capacity_is_the_ceiling(N, E, k, cf):
    """C is the least integer >= cf*k*N/E, checked in exact rational arithmetic."""
    C = oracle.capacity(N, E, k, cf)
    q = Fraction(float(np.float32(cf))) * k * N / E
    assert C - 1 < q <= C


def test_capacity_of_the_benchmark_layers():
    assert oracle.capacity(2048, 8, 2, 1.25) == 640
    assert oracle.capacity(4096, 8, 2, 1.25) == 1280
    assert oracle.capacity(16384, 16, 2, 1.0) == 2048
    assert oracle.capacity(8192, 256, 8, 1.5) == 384
    assert oracle.capacity(0, 8, 2, 1.25) == 0


def test_drops_fill_capacity_in_order():
    """Drops on a random skewed routing: an expert that drops anything is full,
    and its kept assignments are the earliest in (choice, token) order."""
    rng = np.random.default_rng(11)
    N, E, k, C = 200, 4, 2, 60
    p = np.array([0.6, 0.2, 0.1, 0.1])
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(N)]).astype(np.int32)
    slot, used = oracle.assign(idx, E, C)
    for e in range(E):
        order = [(j, t) for j in range(k) for t in range(N) if idx[t, j] == e]
        kept = [(j, t) for (j, t) in order if slot[t, j] >= 0]
        assert kept == order[:C] if len(order) > C else kept == order
        assert used[e] == min(len(order), C)


# ----------------------------------------------------------------------------
# the nanoMoE slides' expert variant (slide 32): biases and GELU
# ----------------------------------------------------------------------------
#: the standard normal distribution function at tabulated points
PHI = {1.0: 0.8413447460685429, -1.0: 0.15865525393145707, 2.0: 0.9772498680518208,
       0.5: 0.6914624612740131, -3.0: 0.0013498980316301035}


def _one(z, act, bup=None, bdown=None):
    """A 1 -> 1 -> 1 expert with unit weights on the scalar input z."""
    b1 = None if bup is None else np.array([bup])
    b2 = None if bdown is None else np.array([bdown])
    return oracle.expert_rows(np.array([[z]]), [0], np.eye(1), np.eye(1), act, b1, b2)[0, 0]


def test_gelu_is_x_times_the_normal_cdf():
    """torch's default GELU (slide 32) is x * Phi(x): checked at the table values."""
    for z, phi in PHI.items():
        assert _one(z, "gelu") == pytest.approx(z * phi, rel=1e-14, abs=1e-300)
    assert _one(0.0, "gelu") == 0.0


def test_gelu_odd_part_is_the_identity():
    """Phi(x) + Phi(-x) = 1 gives GELU(x) - GELU(-x) = x."""
    for z in np.random.default_rng(31).standard_normal(50) * 3:
        assert _one(z, "gelu") - _one(-z, "gelu") == pytest.approx(z, rel=1e-14, abs=1e-15)


def test_biases_enter_before_and_after_the_activation():
    """Identity experts (d_ff = d, W = I) with ReLU and x + b_up > 0 give
    y = x + b_up + b_down; with GELU, y = GELU(x + b_up) + b_down."""
    rng = np.random.default_rng(32)
    d = 5
    x = np.abs(rng.standard_normal((7, d))) + 0.1
    bup = np.abs(rng.standard_normal(d))
    bdown = rng.standard_normal(d)
    y = oracle.expert_rows(x, np.arange(7), np.eye(d), np.eye(d), "relu", bup, bdown)
    np.testing.assert_allclose(y, x + bup + bdown, rtol=1e-15, atol=1e-15)
    # GELU: 0.5 + 0.5 = 1 and -4 + 1 = -3 land on tabulated points
    assert _one(0.5, "gelu", 0.5, 0.25) == pytest.approx(PHI[1.0] + 0.25, rel=1e-14)
    assert _one(-4.0, "gelu", 1.0, -1.0) == pytest.approx(-3.0 * PHI[-3.0] - 1.0, rel=1e-14)


@pytest.mark.parametrize("act,seed", [("gelu", 41), ("relu", 42), ("gelu", 43)])
def test_expert_variant_equals_bruteforce_without_drops(act, seed):
    """Full layer with biases (and GELU) against the all-experts brute force."""
    wl = W.custom("bfv", N=19, d=6, E=5, k=2, d_ff=11, dtype="f32", cf=5.0, sigma=0.4,
                  seed=seed, w_std=0.5, wg_std=0.7, act=act, bias_std=0.3)
    assert wl.b_up().shape == (5, 11) and wl.b_down().shape == (5, 6)
    r = oracle.forward(wl)
    assert r.drops == 0
    x64, wg64, n64, wups, wdowns = _bf_inputs(wl)
    ref, _, order = BF.layer(x64, wg64, n64, wl.k, wups, wdowns, act,
                             wl.b_up().astype(np.float64), wl.b_down().astype(np.float64))
    np.testing.assert_array_equal(r.idx, order)
    assert np.abs(r.out - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1.0)
