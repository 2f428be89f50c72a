"""Seeded synthetic inputs for the sparse MoE layer forward.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests. It draws random numbers and converts dtypes; it holds none of
the layer's arithmetic, with one exception that is input conditioning rather
than computation: :func:`separation_screen` evaluates the router scores of a
candidate input in numpy float64 so that tokens whose ranking is ambiguous
(two of the top-(k+1) scores within ``SEPARATION`` of each other) are redrawn.
Ranking decides integers (expert ids, slots, drops); the screen makes that
decision unique so both sides can be compared bit-exactly. It produces no
expected value and neither side imports it for arithmetic.

Workloads follow the pages:

* "MoE 12-step visual anatomy simulator" (page 1), preset panel: token
  x = [1.2, -0.4, -0.8], k = 2, sigma = 0, four experts, a 3 -> 4 -> 3 FFN.
* "nanoMoE deep dive" slides (page 2), slides 11-13 (router example, printed
  logits for B=2, T=4, E=3) and slides 15-29 (capacity example, B=1, T=4,
  E=3, k=2, capacity 1).
* The layer shapes of the benchmark table (nanoMoE-, Mixtral-, skewed- and
  fine-grained-shaped layers) with Gaussian weights.

Random streams: numpy ``Generator(PCG64(SeedSequence(seed, spawn_key=...)))``
with one stream per tensor and one per expert matrix, so any expert's weights
can be regenerated alone (the fine-grained layer holds 15 GB of bf16 weights).
Values are drawn in float32 and rounded to bfloat16 (round to nearest even)
where the workload is bf16; every consumer sees exactly the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

#: Minimum gap between adjacent scores among a token's top-(k+1) (or top-k
#: when k == E) after which its ranking is treated as unambiguous.
SEPARATION = 1e-4

# spawn_key namespaces of the random streams
_S_X, _S_WG, _S_NOISE, _S_RESAMPLE, _S_WUP, _S_WDOWN, _S_BUP, _S_BDOWN, _S_DOUT = range(9)


# --------------------------------------------------------------------------
# dtype plumbing (no arithmetic of the method)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even), returned as uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# workload definitions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    N: int                 # tokens per call (B*T, flattened row-major)
    d: int                 # model width
    E: int                 # experts
    k: int                 # experts per token
    d_ff: int              # expert hidden width
    dtype: str             # "f32" or "bf16": x, expert weights, H and out
    cf: float              # capacity factor
    sigma: float = 0.0     # noise std (noise tensor = sigma * eps)
    bias0: float = 0.0     # constant added to expert 0's score (folded into noise)
    wg_std: float = 0.0    # router weight std; 0 -> 1/sqrt(d)
    w_std: float = 0.02    # expert weight std
    x_std: float = 1.0
    seed: int = 20260
    B: int = 0
    T: int = 0
    description: str = ""
    act: str = "relu"      # expert activation: "relu" (page 1) or "gelu" (nanoMoE slide 32)
    bias_std: float = 0.0  # std of the fp32 expert biases (nanoMoE slide 32); 0 -> no biases
    dropout: float = 0.0   # training-mode dropout on the expert outputs (nanoMoE slide 32)
    dropout_seed: int = 0  # its generator key
    dropout_offset: int = 0

    @property
    def has_noise(self) -> bool:
        return self.sigma != 0.0 or self.bias0 != 0.0

    @property
    def router_std(self) -> float:
        return self.wg_std if self.wg_std > 0 else 1.0 / math.sqrt(self.d)


CONFIGS = {
    # page 1 preset panel: token 0 = [1.2, -0.4, -0.8], k=2, sigma=0, 4 experts, 3->4->3
    "tiny": Config("tiny", N=8, B=2, T=4, d=3, E=4, k=2, d_ff=4, dtype="f32", cf=8.0,
                   wg_std=0.5, w_std=0.5, seed=20261,
                   description="page-1 preset: B=2,T=4,d=3,E=4,k=2,d_ff=4,fp32,cf=8"),
    "nanomoe": Config("nanomoe", N=2048, B=8, T=256, d=768, E=8, k=2, d_ff=3072, dtype="bf16",
                      cf=1.25, sigma=1.0, seed=20262,
                      description="nanoMoE-shaped: 2048 tokens, d=768, E=8, k=2, d_ff=3072, bf16"),
    "mixtral": Config("mixtral", N=4096, d=4096, E=8, k=2, d_ff=14336, dtype="bf16", cf=1.25,
                      seed=20263,
                      description="Mixtral-shaped: 4096 tokens, d=4096, E=8, k=2, d_ff=14336, bf16"),
    "skew": Config("skew", N=16384, d=2048, E=16, k=2, d_ff=8192, dtype="bf16", cf=1.0,
                   sigma=0.5, bias0=3.0, wg_std=0.0310, seed=20264,
                   description="skewed load: 16384 tokens, d=2048, E=16, k=2, d_ff=8192, +3 on e0"),
    "finegrained": Config("finegrained", N=8192, d=7168, E=256, k=8, d_ff=2048, dtype="bf16",
                          cf=1.5, seed=20265,
                          description="fine-grained: 8192 tokens, d=7168, E=256, k=8, d_ff=2048"),
    # the nanoMoE slides' own expert (slide 32): GELU and biases, nanoMoE shape
    "nanomoe_gelu": Config("nanomoe_gelu", N=2048, B=8, T=256, d=768, E=8, k=2, d_ff=3072,
                           dtype="bf16", cf=1.25, sigma=1.0, seed=20268, act="gelu",
                           bias_std=0.02,
                           description="nanoMoE-shaped with the slides' GELU expert and "
                                       "biases: 2048 tokens, d=768, E=8, k=2, d_ff=3072, bf16"),
}

#: Benchmark-table order of the five layer shapes.
CONFIG_ORDER = ["tiny", "nanomoe", "mixtral", "skew", "finegrained"]


# --------------------------------------------------------------------------
# the pages' worked examples (fixed inputs; see tests/golden for the values)
# --------------------------------------------------------------------------
#: nanoMoE slides 11-13: printed logits of 8 tokens (B=2, T=4) over E=3.
ROUTER_EXAMPLE_LOGITS = np.array([
    [-0.8, 2.1, -1.4], [-2.5, 0.9, 1.8], [1.2, -0.3, 0.4], [0.5, 1.7, -2.1],
    [2.4, -1.1, -1.6], [0.7, 2.3, -3.0], [-1.3, 0.2, 1.5], [-0.4, -2.2, 2.8],
], dtype=np.float32)

#: nanoMoE slides 15-29: four tokens whose top-2 are [0,1],[0,2],[0,1],[0,2].
CAPACITY_EXAMPLE_X = np.array([
    [3.0, 2.0, 1.0], [3.0, 1.0, 2.0], [3.0, 2.0, 1.0], [3.0, 1.0, 2.0],
], dtype=np.float32)


# --------------------------------------------------------------------------
# the input screen
# --------------------------------------------------------------------------
def separation_screen(x64: np.ndarray, wg64: np.ndarray, noise64: Optional[np.ndarray],
                      k: int, sep: float = SEPARATION) -> np.ndarray:
    """Return a boolean mask of tokens whose top ranking is ambiguous.

    Scores are evaluated in float64 from the exact input values. A token is
    flagged when two adjacent scores among its sorted top-(k+1) (top-k when
    k == E) differ by less than ``sep``: the order inside the top-k sets
    capacity priority, so every adjacent pair there must be separated too.
    """
    s = x64 @ wg64.T
    if noise64 is not None:
        s = s + noise64
    E = s.shape[1]
    m = min(k + 1, E)
    top = -np.sort(-s, axis=1)[:, :m]
    if m < 2:
        return np.zeros(s.shape[0], dtype=bool)
    gaps = top[:, :-1] - top[:, 1:]
    return (gaps < sep).any(axis=1)


# --------------------------------------------------------------------------
# workload instances
# --------------------------------------------------------------------------
def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _cast(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


class Workload:
    """One seeded input set: x, W_g, noise and lazily generated expert weights.

    ``x`` is stored in the workload dtype (uint16 bf16 bits or float32),
    ``wg`` and ``noise`` in float32. ``w_up(e)`` is [d_ff, d] and
    ``w_down(e)`` is [d, d_ff] in the workload dtype: each row is one output
    neuron, contiguous along the reduction dimension (page 1, STEP 8 and
    STEP 10 write z = W_up x and E(x) = W_down h).
    """

    def __init__(self, cfg: Config, x: np.ndarray, wg: np.ndarray,
                 noise: Optional[np.ndarray], expert_seed: int,
                 fixed_experts: Optional[tuple] = None, resampled: int = 0):
        self.cfg = cfg
        self.x = x
        self.wg = wg
        self.noise = noise
        self.expert_seed = expert_seed
        self._fixed = fixed_experts
        self.resampled = resampled
        self._memo = {}

    def memo(self, which: str, e: int, a: np.ndarray) -> None:
        """Keep an already generated expert matrix for later calls."""
        self._memo[(which, e)] = a

    # shapes ---------------------------------------------------------------
    @property
    def N(self): return self.cfg.N
    @property
    def d(self): return self.cfg.d
    @property
    def E(self): return self.cfg.E
    @property
    def k(self): return self.cfg.k
    @property
    def d_ff(self): return self.cfg.d_ff

    # expert weights ---------------------------------------------------------
    def w_up(self, e: int) -> np.ndarray:
        if self._fixed is not None:
            return self._fixed[0][e]
        if ("up", e) in self._memo:
            return self._memo[("up", e)]
        a = _rng(self.expert_seed, _S_WUP, e).standard_normal((self.d_ff, self.d), dtype=np.float32)
        a *= np.float32(self.cfg.w_std)
        return _cast(a, self.cfg.dtype)

    def w_down(self, e: int) -> np.ndarray:
        if self._fixed is not None:
            return self._fixed[1][e]
        if ("down", e) in self._memo:
            return self._memo[("down", e)]
        a = _rng(self.expert_seed, _S_WDOWN, e).standard_normal((self.d, self.d_ff), dtype=np.float32)
        a *= np.float32(self.cfg.w_std)
        return _cast(a, self.cfg.dtype)

    def b_up(self) -> Optional[np.ndarray]:
        """Up-projection biases [E, d_ff] fp32, or None (nanoMoE slide 32)."""
        if self.cfg.bias_std == 0.0:
            return None
        a = _rng(self.expert_seed, _S_BUP).standard_normal((self.E, self.d_ff), dtype=np.float32)
        return a * np.float32(self.cfg.bias_std)

    def b_down(self) -> Optional[np.ndarray]:
        """Down-projection biases [E, d] fp32, or None."""
        if self.cfg.bias_std == 0.0:
            return None
        a = _rng(self.expert_seed, _S_BDOWN).standard_normal((self.E, self.d), dtype=np.float32)
        return a * np.float32(self.cfg.bias_std)

    def experts(self, which: str, threads: int = 8):
        """Yield (e, array) for every expert, generated on a thread pool in order."""
        fn = self.w_up if which == "up" else self.w_down
        with ThreadPoolExecutor(max(1, threads)) as ex:
            futs = [ex.submit(fn, e) for e in range(min(threads, self.E))]
            nxt = len(futs)
            for e in range(self.E):
                a = futs[e].result()
                futs[e] = None
                if nxt < self.E:
                    futs.append(ex.submit(fn, nxt))
                    nxt += 1
                yield e, a

    # float64 views for the CPU side -----------------------------------------
    def as_f64(self, a: np.ndarray) -> np.ndarray:
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def x64(self) -> np.ndarray:
        return self.as_f64(self.x)

    def wg64(self) -> np.ndarray:
        return self.wg.astype(np.float64)

    def noise64(self) -> Optional[np.ndarray]:
        return None if self.noise is None else self.noise.astype(np.float64)

    def dout(self, scale: float = 1.0) -> np.ndarray:
        """A seeded output gradient [N, d] in the workload dtype (standard
        normal times ``scale``), the input of the backward pass."""
        a = _rng(self.cfg.seed, _S_DOUT).standard_normal((self.N, self.d), dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        return _cast(a, self.cfg.dtype)


def _draw_x(cfg: Config, rng: np.random.Generator, n: int) -> np.ndarray:
    a = rng.standard_normal((n, cfg.d), dtype=np.float32)
    if cfg.x_std != 1.0:
        a *= np.float32(cfg.x_std)
    return a


def make(cfg_or_name, seed: Optional[int] = None) -> Workload:
    """Build the seeded workload for a config (name or :class:`Config`)."""
    cfg = CONFIGS[cfg_or_name] if isinstance(cfg_or_name, str) else cfg_or_name
    seed = cfg.seed if seed is None else seed
    N, d, E, k = cfg.N, cfg.d, cfg.E, cfg.k

    noise = None
    if cfg.has_noise:
        noise = _rng(seed, _S_NOISE).standard_normal((N, E), dtype=np.float32)
        noise *= np.float32(cfg.sigma)
        if cfg.bias0 != 0.0:
            noise[:, 0] += np.float32(cfg.bias0)

    x32 = _draw_x(cfg, _rng(seed, _S_X), N)
    if cfg.name == "tiny":
        x32[0] = np.array([1.2, -0.4, -0.8], dtype=np.float32)

    # The router weights; for the page-1 preset, token 0 is fixed, so an
    # ambiguous token 0 advances the router stream instead of redrawing x.
    wg_attempt = 0
    while True:
        wg = _rng(seed, _S_WG, wg_attempt).standard_normal((E, d), dtype=np.float32)
        wg *= np.float32(cfg.router_std)
        x = _cast(x32, cfg.dtype)
        wk = Workload(cfg, x, wg, noise, seed)
        if cfg.name != "tiny":
            break
        bad = separation_screen(wk.x64()[:1], wk.wg64(), wk.noise64()[:1] if noise is not None else None, k)
        if not bad[0]:
            break
        wg_attempt += 1

    # Redraw ambiguous tokens from a dedicated stream until all are separated.
    rs = _rng(seed, _S_RESAMPLE)
    resampled = 0
    wg64 = wg.astype(np.float64)
    n64 = None if noise is None else noise.astype(np.float64)
    bad = separation_screen(wk.x64(), wg64, n64, k)
    if cfg.name == "tiny":
        bad[0] = False
    while bad.any():
        rows = np.nonzero(bad)[0]
        resampled += len(rows)
        new = _draw_x(cfg, rs, len(rows))
        x[rows] = _cast(new, cfg.dtype)
        sub = separation_screen(wk.as_f64(x[rows]), wg64, None if n64 is None else n64[rows], k)
        bad[:] = False
        bad[rows[sub]] = True
    wk.resampled = resampled
    return wk


def _fixed_example(name: str, x: np.ndarray, k: int, cf: float, d_ff: int,
                   seed: int) -> Workload:
    """The pages' worked examples: W_g = I so the printed numbers are the scores."""
    N, d = x.shape
    E = d
    cfg = Config(name, N=N, d=d, E=E, k=k, d_ff=d_ff, dtype="f32", cf=cf,
                 w_std=0.5, seed=seed)
    wg = np.eye(E, d, dtype=np.float32)
    return Workload(cfg, np.ascontiguousarray(x, np.float32), wg, None, seed)


def router_example() -> Workload:
    """nanoMoE slides 11-13: 8 tokens, E=3, k=2, scores = printed logits (cf=8: no drops)."""
    return _fixed_example("router_example", ROUTER_EXAMPLE_LOGITS, k=2, cf=8.0, d_ff=4, seed=20266)


def capacity_example() -> Workload:
    """nanoMoE slides 15-29: 4 tokens, E=3, k=2, capacity ceil(0.375*2*4/3) = 1."""
    return _fixed_example("capacity_example", CAPACITY_EXAMPLE_X, k=2, cf=0.375, d_ff=4, seed=20267)


def custom(name: str, N: int, d: int, E: int, k: int, d_ff: int, dtype: str, cf: float,
           sigma: float = 0.0, bias0: float = 0.0, seed: int = 1, w_std: float = 0.05,
           wg_std: float = 0.0, act: str = "relu", bias_std: float = 0.0,
           dropout: float = 0.0, dropout_seed: int = 0, dropout_offset: int = 0) -> Workload:
    """A seeded workload of any shape (test cases: ragged tails, edge cases)."""
    if act not in ("relu", "gelu"):
        raise ValueError("act must be 'relu' or 'gelu'")
    cfg = Config(name, N=N, d=d, E=E, k=k, d_ff=d_ff, dtype=dtype, cf=cf, sigma=sigma,
                 bias0=bias0, seed=seed, w_std=w_std, wg_std=wg_std, act=act,
                 bias_std=bias_std, dropout=dropout, dropout_seed=dropout_seed,
                 dropout_offset=dropout_offset)
    return make(cfg)

