"""Seeded synthetic inputs for the FlashMap drafting step.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
no arithmetic of the drafting method: only the workload shapes, seeded normal
draws, rounding of those draws to the storage type (bfloat16 bit patterns or
float32), the gate-slot variants used by the tests, and the planting of target
logits for a chosen accept length.

Recipe (every draw is numpy ``default_rng`` / PCG64, standard normal in float32,
scaled, then rounded to nearest-even bfloat16 for bf16 workloads):

* weights: tensor ``i`` of the canonical order (``weight_names``) is drawn in
  chunks of ``CHUNK`` elements, chunk ``c`` from seed ``[0, i, c]``, std 0.02;
* context features ``[C][5][H]``: seed ``[1, c]`` per chunk, std 1 (request r > 0
  of a batch of requests: seed ``[4, r, c]``);
* noise block of branch ``b`` ``[K][V]``: seed ``[2, b, c]``, std 1; a parity
  test that meets a near-tie re-runs on the next draw k = 1, 2, ..., seed
  ``[6, k, b, c]``;
* target logits of branch ``b`` ``[K+1][V]``: seed ``[3, b, c]``, std 1.

Shapes follow the drafter the pages describe (a 6-block DiT of width 2048 with
16 heads reading five target layers, K=16 drafts, a 151,936-entry vocabulary).
Trained weights are not available, so random weights of that shape stand in.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
WEIGHT_STD = 0.02
N_CTX_LAYERS = 5
CTX_LAYER_IDS = (1, 9, 17, 25, 33)
T_FREQ = 256


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: drafter shape, context, batch of branches and schedule."""

    name: str
    K: int          # block length (drafted tokens per step)
    V: int          # vocabulary size
    d: int          # drafter width
    L: int          # number of DiT blocks
    nh: int         # attention heads
    H: int          # target hidden width (per context layer)
    dtype: str      # 'bf16' or 'f32' storage / compute type
    c_prefill: int  # context rows already in the cache before the step
    n_new: int      # context rows appended inside the step
    B: int = 1      # independent noise branches (draft tree)
    times: tuple = (0.0, 1.0)   # flow-map schedule s_0=0 < ... < s_n=1
    mlp_mult: int = 4
    c_max: int = 0  # context capacity (0: c_prefill + n_new)
    temperature: float = 0.0    # 0: greedy drafting and verification; > 0: sampled
    requests: int = 1           # independent requests drafted together, each with its own
                                # context of c_prefill + n_new rows

    @property
    def hd(self) -> int:
        return self.d // self.nh

    @property
    def F(self) -> int:
        return self.mlp_mult * self.d

    @property
    def C(self) -> int:
        return self.c_prefill + self.n_new

    @property
    def capacity(self) -> int:
        return self.c_max if self.c_max else self.C

    @property
    def num_steps(self) -> int:
        return len(self.times) - 1

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _qwen8b(**kw):
    base = dict(K=16, V=151936, d=2048, L=6, nh=16, H=4096, dtype="bf16",
                c_prefill=504, n_new=8)
    base.update(kw)
    return Config(**base)


CONFIGS = {
    # small parity case, float32 throughout
    "tiny": Config(name="tiny", K=16, V=1024, d=256, L=2, nh=4, H=512,
                   dtype="f32", c_prefill=24, n_new=8),
    # Qwen3-8B-shaped 1-step drafter, context 512 (504 cached + 8 appended per step)
    "qwen3_8b": _qwen8b(name="qwen3_8b"),
    # Qwen3-4B-shaped: same drafter, target width 2560, context 2048
    "qwen3_4b": _qwen8b(name="qwen3_4b", H=2560, c_prefill=2040),
    # two jumps 0 -> 0.5 -> 1, context 1024
    "qwen3_8b_2step": _qwen8b(name="qwen3_8b_2step", c_prefill=1016,
                              times=(0.0, 0.5, 1.0)),
    # tree of 4 noise branches sharing one context of 4096
    "qwen3_8b_tree4": _qwen8b(name="qwen3_8b_tree4", c_prefill=4088, B=4),
    # as qwen3_8b, sampled at temperature 1 (probabilistic drafting + verify)
    "qwen3_8b_t1": _qwen8b(name="qwen3_8b_t1", temperature=1.0),
    # four concurrent requests, each with its own context of 512 rows (508 cached
    # + 4 appended per step), drafted together
    "qwen3_8b_batch4": _qwen8b(name="qwen3_8b_batch4", c_prefill=508, n_new=4, requests=4),
}

# seeds of the random streams of sampled steps (one per replayed step)
SAMPLE_SEEDS = tuple(range(1, 11))


# --------------------------------------------------------------------------
# storage helpers (draw rounding only)
# --------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def values(a: np.ndarray) -> np.ndarray:
    """Storage array (uint16 bf16 bits or float32) -> float32 values."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


def _draw(seed_prefix, shape, std, dtype, pool=None):
    """Normal draws of ``shape`` in chunks; chunk c from seed seed_prefix+[c]."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.default_rng(list(seed_prefix) + [c])
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = _store(x, dtype)

    chunks = range((n + CHUNK - 1) // CHUNK)
    if pool is not None and n > CHUNK:
        list(pool.map(one, chunks))
    else:
        for c in chunks:
            one(c)
    return out.reshape(shape)


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def weight_shapes(cfg: Config):
    """Canonical (name, shape) list; the index in this list is the seed index."""
    d, F, V = cfg.d, cfg.F, cfg.V
    out = [("E", (V, d)), ("W_f", (d, N_CTX_LAYERS * cfg.H)), ("b_f", (d,))]
    for te in ("te_s", "te_t"):
        out += [(f"{te}.W1", (d, T_FREQ)), (f"{te}.b1", (d,)),
                (f"{te}.W2", (d, d)), (f"{te}.b2", (d,))]
    for l in range(cfg.L):
        p = f"blk{l}."
        out += [(p + "W_ada", (6 * d, d)), (p + "b_ada", (6 * d,)),
                (p + "W_qkv", (3 * d, d)), (p + "b_qkv", (3 * d,)),
                (p + "W_o", (d, d)), (p + "b_o", (d,)),
                (p + "W_1", (F, d)), (p + "b_1", (F,)),
                (p + "W_2", (d, F)), (p + "b_2", (d,))]
    out += [("W_fa", (2 * d, d)), ("b_fa", (2 * d,)), ("W_lm", (V, d))]
    return out


def weight_names(cfg: Config):
    return [n for n, _ in weight_shapes(cfg)]


# adaLN output slots of a block, in the order the modulation vector holds them:
# shift/scale/gate before attention, then shift/scale/gate before the MLP.
ADA_SLOTS = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")


def make_weights(cfg: Config, variant: str = "random") -> dict:
    """All drafter weights as storage arrays.

    variant:
      'random'     every tensor ~ N(0, 0.02^2)
      'gate_zero'  every block's adaLN weights and biases are zero (gates = 0)
      'unit_gate'  every block's adaLN weights are zero and its bias sets both
                   gates to 1 and every shift/scale to 0
    """
    shapes = weight_shapes(cfg)
    w = {}
    with ThreadPoolExecutor(_workers()) as pool:
        for i, (name, shape) in enumerate(shapes):
            if variant != "random" and (".W_ada" in name or ".b_ada" in name):
                x = np.zeros(shape, dtype=np.float32)
                if variant == "unit_gate" and ".b_ada" in name:
                    for slot in ("gate1", "gate2"):
                        j = ADA_SLOTS.index(slot)
                        x[j * cfg.d:(j + 1) * cfg.d] = 1.0
                w[name] = _store(x, cfg.dtype)
            else:
                w[name] = _draw([0, i], shape, WEIGHT_STD, cfg.dtype, pool)
    return w


# --------------------------------------------------------------------------
# activations: context features, noise, target logits
# --------------------------------------------------------------------------

def make_features(cfg: Config, rows: int | None = None, request: int = 0) -> np.ndarray:
    """Target hidden states [rows][5][H] of layers 1, 9, 17, 25, 33, N(0,1);
    request 0 from seed [1], request r > 0 (its own context) from seed [4, r]."""
    rows = cfg.C if rows is None else rows
    with ThreadPoolExecutor(_workers()) as pool:
        return _draw([1] if request == 0 else [4, request], (rows, N_CTX_LAYERS, cfg.H), 1.0, cfg.dtype, pool)


def make_noise(cfg: Config, B: int | None = None, draw: int = 0) -> np.ndarray:
    """Gaussian noise blocks [B][K][V], N(0,1); branch b from seed [2, b], or
    from seed [6, draw, b] for a later draw (draw >= 1)."""
    B = cfg.B if B is None else B
    with ThreadPoolExecutor(_workers()) as pool:
        return np.stack([_draw([2, b] if draw == 0 else [6, draw, b], (cfg.K, cfg.V), 1.0, cfg.dtype, pool)
                         for b in range(B)])


def make_target_logits(cfg: Config, B: int | None = None) -> np.ndarray:
    """Random target logits [B][K+1][V], N(0,1); branch b from seed [3, b]."""
    B = cfg.B if B is None else B
    with ThreadPoolExecutor(_workers()) as pool:
        return np.stack([_draw([3, b], (cfg.K + 1, cfg.V), 1.0, cfg.dtype, pool)
                         for b in range(B)])


def plant(T: np.ndarray, draft: np.ndarray, n: int) -> np.ndarray:
    """Return a copy of target logits T [K+1][V] edited so that a greedy verifier
    accepts exactly ``n`` tokens of ``draft`` [K]: rows j < n get draft[j] raised
    one above the row maximum; row n (if n < K) gets draft[n]+1 (mod V) raised the
    same way so that it disagrees with the draft.  Other rows stay random."""
    T = np.array(T, copy=True)
    K, V = T.shape[0] - 1, T.shape[1]
    assert 0 <= n <= K and draft.shape == (K,)
    vals = values(T)
    for j in range(n + (1 if n < K else 0)):
        tok = int(draft[j]) if j < n else (int(draft[j]) + 1) % V
        top = np.float32(vals[j].max() + 1.0)
        if T.dtype == np.uint16:
            b = to_bf16_bits(np.array([top], dtype=np.float32))[0]
            while bf16_bits_to_f32(np.array([b]))[0] <= vals[j].max():
                b += 1
            T[j, tok] = b
        else:
            T[j, tok] = top
    return T


# accept lengths of the ten planted target sets the headline workload cycles
# through: mean 6.7 accepted + 1 target token = 7.7 tokens per cycle, in line
# with the 7.69 acceptance length reported for GSM8K at temperature 0.
PLANTED_ACCEPT = (7, 7, 7, 7, 7, 7, 7, 6, 6, 6)
# per-branch accept lengths of the planted tree workload (best branch: 2)
PLANTED_ACCEPT_TREE = (7, 3, 9, 5)
