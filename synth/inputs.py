"""Seeded synthetic workloads shaped like the decode stacks the pages describe.

Nothing here quantises, packs, permutes or multiplies: it only fixes shapes and
draws random numbers, so the oracle and the library see identical inputs.

Recipe (all draws from numpy's ``default_rng``):

* single INT8 linear (out = in = 4096): ``default_rng(0)``; W is drawn first as
  ``standard_normal((4096, 4096), float32) * 0.02``, then x as
  ``standard_normal((1, 4096), float32)`` rounded to fp16.
* stacks: every draw has its own ``SeedSequence([cfg_id, layer, slot])``.
  slot 0..6 = weights of q, k, v, o, gate, up, down; 10..13 = the four decode
  inputs of a layer (hidden for q/k/v, attention output for o, hidden for
  gate/up, intermediate for down); 20 + space = activation profile of an input
  space; 30 + space = the planted channel set of an input space.
* weights: ``standard_normal((N, K), float32) * float32(std)``.
* activations: ``standard_normal`` in float32 rounded to fp16; drawn at the
  largest batch of the workload, smaller batches take a prefix of the rows.
* outlier-format stacks plant ``ceil(K/100)`` channels per input space (the
  same set in every layer): weight columns x10, profile and decode activation
  columns x20, applied in float32 before any rounding to fp16.
* the activation profile has 128 rows.
* the tied embedding / lm_head table: slot 40 of layer 0, [vocab, hidden],
  std as the stack, planted hidden channels x10; decode token ids: slot 41,
  uniform integers in [0, vocab).
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SPACES = ("h", "a", "m")          # hidden, attention output (heads x head_dim), intermediate
LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
# decode input index -> (input space, linears fed by it)
INPUTS = ((0, "h", ("q", "k", "v")), (1, "a", ("o",)), (2, "h", ("gate", "up")), (3, "m", ("down",)))
PROFILE_ROWS = 128


@dataclass(frozen=True)
class LinearSpec:
    name: str
    slot: int
    N: int        # output features
    K: int        # input features
    space: str    # input space the linear reads
    inp: int      # decode input index 0..3


@dataclass(frozen=True)
class StackSpec:
    cfg_id: int
    fmt: str                 # "int8" or "int4o"
    hidden: int
    inter: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    std: float
    batches: tuple = (1,)
    planted: bool = False
    w_planted_gain: float = 10.0
    x_planted_gain: float = 20.0
    name: str = field(default="")

    def space_width(self, space: str) -> int:
        return {"h": self.hidden, "a": self.q_heads * self.head_dim, "m": self.inter}[space]

    def linears(self) -> list[LinearSpec]:
        h, a, m = self.hidden, self.q_heads * self.head_dim, self.inter
        kv = self.kv_heads * self.head_dim
        return [
            LinearSpec("q", 0, a, h, "h", 0),
            LinearSpec("k", 1, kv, h, "h", 0),
            LinearSpec("v", 2, kv, h, "h", 0),
            LinearSpec("o", 3, h, a, "a", 1),
            LinearSpec("gate", 4, m, h, "h", 2),
            LinearSpec("up", 5, m, h, "h", 2),
            LinearSpec("down", 6, h, m, "m", 3),
        ]

    def linear(self, name: str) -> LinearSpec:
        return next(l for l in self.linears() if l.name == name)

    @property
    def bmax(self) -> int:
        return max(self.batches)


CONFIGS = {
    2: StackSpec(2, "int4o", hidden=3072, inter=8192, layers=28, q_heads=24, kv_heads=8,
                 head_dim=128, std=0.02, batches=(1,), planted=True,
                 name="3B-shaped outlier-INT4 stack, 28 layers"),
    3: StackSpec(3, "int8", hidden=3584, inter=14336, layers=42, q_heads=16, kv_heads=8,
                 head_dim=256, std=0.02, batches=(1, 4), planted=False,
                 name="9B-shaped INT8 stack, 42 layers"),
    4: StackSpec(4, "int4o", hidden=8192, inter=28672, layers=80, q_heads=64, kv_heads=8,
                 head_dim=128, std=0.015, batches=(1, 8, 32), planted=True,
                 name="70B-shaped outlier-INT4 stack, 80 layers"),
}
# the streamed workload reuses the INT8 9B-shaped stack unchanged
CONFIGS[5] = CONFIGS[3]


# vocabulary of the tied embedding / lm_head table: the 3B- and 70B-shaped
# models use a 128256-token vocabulary, the 9B-shaped one 256000; reduced
# stacks use 1000
VOCAB = {2: 128256, 3: 256000, 4: 128256}


def vocab_size(spec: StackSpec) -> int:
    return VOCAB.get(spec.cfg_id, 1000)


def embedding(spec: StackSpec, out: np.ndarray | None = None) -> np.ndarray:
    """float32 [vocab, hidden] tied embedding table (also the lm_head weight):
    slot 40 of layer 0, std as the stack's weights, planted hidden channels x10."""
    V, H = vocab_size(spec), spec.hidden
    if out is None:
        out = np.empty((V, H), np.float32)
    _rng(spec.cfg_id, 0, 40).standard_normal(dtype=np.float32, out=out)
    out *= np.float32(spec.std)
    if spec.planted:
        out[:, planted_set(spec, "h")] *= np.float32(spec.w_planted_gain)
    return out


def token_ids(spec: StackSpec, b: int | None = None) -> np.ndarray:
    """int32 [b] decode token ids (slot 41), uniform over the vocabulary."""
    ids = _rng(spec.cfg_id, 0, 41).integers(0, vocab_size(spec), size=spec.bmax, dtype=np.int32)
    return ids if b is None else ids[:b].copy()


def stack_spec(cfg: int) -> StackSpec:
    return CONFIGS[cfg]


def small_stack_spec(cfg: int, layers: int = 2, hidden: int = 384, inter: int = 1000,
                     q_heads: int = 3, kv_heads: int = 1, head_dim: int = 128,
                     batches=None) -> StackSpec:
    """Same recipe as ``cfg`` at reduced, deliberately ragged widths (own seed id)."""
    base = CONFIGS[cfg]
    return StackSpec(100 + cfg, base.fmt, hidden=hidden, inter=inter, layers=layers,
                     q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim, std=base.std,
                     batches=batches or base.batches, planted=base.planted,
                     name=f"reduced {base.name}")


def planted_count(K: int) -> int:
    """1% of the channels of an input space, rounded up."""
    return (K + 99) // 100


def _rng(cfg_id: int, layer: int, slot: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, layer, slot]))


@functools.lru_cache(maxsize=64)
def _planted(spec: "StackSpec", space: str) -> np.ndarray:
    K = spec.space_width(space)
    if not spec.planted:
        return np.zeros(0, np.int64)
    rng = _rng(spec.cfg_id, 0, 30 + SPACES.index(space))
    S = np.sort(rng.choice(K, size=planted_count(K), replace=False)).astype(np.int64)
    S.setflags(write=False)
    return S


def planted_set(spec: StackSpec, space: str) -> np.ndarray:
    """Sorted channel indices planted as outliers in an input space (empty if none)."""
    return _planted(spec, space)


def weight(spec: StackSpec, layer: int, lin: LinearSpec | str, out: np.ndarray | None = None) -> np.ndarray:
    """float32 [N, K] weight of one linear of one layer."""
    if isinstance(lin, str):
        lin = spec.linear(lin)
    if out is None:
        out = np.empty((lin.N, lin.K), np.float32)
    _rng(spec.cfg_id, layer, lin.slot).standard_normal(dtype=np.float32, out=out)
    out *= np.float32(spec.std)
    if spec.planted:
        S = planted_set(spec, lin.space)
        out[:, S] *= np.float32(spec.w_planted_gain)
    return out


def decode_input(spec: StackSpec, layer: int, idx: int, b: int | None = None) -> np.ndarray:
    """fp16 [b, K] decode activation number ``idx`` (0..3) of a layer."""
    _, space, _ = INPUTS[idx]
    K = spec.space_width(space)
    # rows are drawn in order, so a smaller batch is a prefix of a larger one
    rows = spec.bmax if b is None else max(b, spec.bmax)
    z = _rng(spec.cfg_id, layer, 10 + idx).standard_normal((rows, K), dtype=np.float32)
    if spec.planted:
        z[:, planted_set(spec, space)] *= np.float32(spec.x_planted_gain)
    x = z.astype(np.float16)
    return x if b is None else np.ascontiguousarray(x[:b])


def profile(spec: StackSpec, space: str, rows: int = PROFILE_ROWS) -> np.ndarray:
    """fp16 [rows, K] activation profile of an input space."""
    K = spec.space_width(space)
    z = _rng(spec.cfg_id, 0, 20 + SPACES.index(space)).standard_normal((rows, K), dtype=np.float32)
    if spec.planted:
        z[:, planted_set(spec, space)] *= np.float32(spec.x_planted_gain)
    return z.astype(np.float16)


def config1_inputs(N: int = 4096, K: int = 4096, std: float = 0.02, seed: int = 0):
    """Single INT8 linear: W float32 [N, K] drawn first, then x fp16 [1, K]."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    x = rng.standard_normal((1, K), dtype=np.float32).astype(np.float16)
    return W, x


def generate_parallel(spec: StackSpec, jobs, fn, threads: int | None = None):
    """Run ``fn(layer, lin, W)`` for every (layer, LinearSpec) in ``jobs``.

    Weights are drawn into reusable per-thread buffers (pre-faulted, so the
    draws scale across threads) and handed to ``fn`` while still in the buffer;
    ``fn`` must copy what it keeps.  Returns the list of ``fn`` results in job
    order.
    """
    threads = threads or min(16, os.cpu_count() or 1)
    jobs = list(jobs)
    if not jobs:
        return []
    maxel = max(l.N * l.K for _, l in jobs)
    import threading
    local = threading.local()

    def run(job):
        layer, lin = job
        buf = getattr(local, "buf", None)
        if buf is None:
            buf = local.buf = np.ones(maxel, np.float32)
        W = buf[: lin.N * lin.K].reshape(lin.N, lin.K)
        weight(spec, layer, lin, out=W)
        return fn(layer, lin, W)

    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(run, jobs))
