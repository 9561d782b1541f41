"""The workloads that bench.py times, as data.

Every launch bench.py times is listed here once -- block type, shape, number
of vectors, activation type -- together with the builders of its seeded
inputs (through :mod:`.synth` only; nothing here computes any part of the
method).  bench.py builds its timed launches from these lists and the GPU
parity tests walk the same lists, so every launch configuration that is timed
is also compared with the oracle.

Shapes:

* dense decoder layer, hidden 2560 (Q4_K): q 4096x2560, k/v 1024x2560,
  o 2560x4096, gate/up 9728x2560, down 2560x9728 -- issued as four launches
  over row-concatenated weights (q|k|v, o, gate|up, down);
* mixed layer, hidden 5120, FFN 17408: q/k/o/gate/up Q4_K, v/down Q6_K
  (q 5120x5120, k/v 1024x5120, o 5120x5120, gate/up 17408x5120,
  down 5120x17408) -- five launches (q|k, v, o, gate|up, down), bf16
  activations;
* a Q4_0 2048x2048 matrix; a Q5_K 17408x5120 matrix;
* routed experts: 128 Q4_0 experts, hidden 2816, expert FFN 704, 8 tokens
  routed top-8;
* prefill: 3015 bf16 activation rows against Q4_K 17408x5120, Q6_K
  5120x17408 and Q4_0 17408x5120.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import synth

S_DENSE, S_MIXED, S_Q4_0, S_MOE, S_PREFILL, S_Q5_K = (synth.SEED_BASE + i for i in (2, 3, 1, 4, 5, 7))

# (projection, N, K) of the dense layer, in seed-stream order
DENSE_PROJ = [("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
              ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728)]
DENSE_LAUNCHES = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gu", ("gate", "up")), ("down", ("down",))]

# (projection, type, N, K) of the mixed layer, in seed-stream order
MIXED_PROJ = [("q", "q4_k", 5120, 5120), ("k", "q4_k", 1024, 5120), ("v", "q6_k", 1024, 5120),
              ("o", "q4_k", 5120, 5120), ("gate", "q4_k", 17408, 5120), ("up", "q4_k", 17408, 5120),
              ("down", "q6_k", 5120, 17408)]
MIXED_LAUNCHES = [("qk", ("q", "k")), ("v", ("v",)), ("o", ("o",)), ("gu", ("gate", "up")), ("down", ("down",))]

_cache: dict = {}


def _proj_weights(kind: str) -> dict:
    """name -> packed weight of every projection of the dense or mixed layer
    (generated once per process)."""
    if kind not in _cache:
        if kind == "dense":
            _cache[kind] = {n: synth.weight("q4_k", synth.rng(S_DENSE, i), N, K)
                            for i, (n, N, K) in enumerate(DENSE_PROJ)}
        else:
            _cache[kind] = {n: synth.weight(t, synth.rng(S_MIXED, i), N, K)
                            for i, (n, t, N, K) in enumerate(MIXED_PROJ)}
    return _cache[kind]


def layer_bytes(kind: str) -> int:
    return sum(w.nbytes for w in _proj_weights(kind).values())


@dataclass(frozen=True)
class Launch:
    """One timed gq_matvec launch: rows `parts` of a layer (concatenated) or a
    stand-alone matrix, against `batch` activation vectors of type xdt."""
    workload: str
    name: str
    t: str
    N: int
    K: int
    batch: int
    xdt: str  # "f32" or "bf16"
    parts: tuple = field(default=())
    seed: int = 0

    @property
    def id(self) -> str:
        return "%s-%s-%s-%dx%d-b%d-%s" % (self.workload, self.name, self.t, self.N, self.K, self.batch, self.xdt)

    def weight(self) -> np.ndarray:
        if self.workload.startswith("dense"):
            w = _proj_weights("dense")
            return np.concatenate([w[p] for p in self.parts])
        if self.workload.startswith("mixed"):
            w = _proj_weights("mixed")
            return np.concatenate([w[p] for p in self.parts])
        return synth.weight(self.t, synth.rng(self.seed, 0), self.N, self.K)

    def x(self) -> np.ndarray:
        """fp32 activations [batch][K] (bf16-representable when xdt is bf16)."""
        x = synth.normal_f32(synth.rng(self.seed, 100 + 16 * self.batch + hash_name(self.name)), (self.batch, self.K))
        if self.xdt == "bf16":
            x = synth.bf16_to_f32(synth.bf16_bits(x))
        return x


def hash_name(name: str) -> int:
    return sum((i + 1) * ord(c) for i, c in enumerate(name)) % 997


def dense_launches(batch: int) -> list[Launch]:
    rows = {n: N for n, N, K in DENSE_PROJ}
    kk = {n: K for n, N, K in DENSE_PROJ}
    return [Launch("dense_b%d" % batch, name, "q4_k", sum(rows[p] for p in parts), kk[parts[0]], batch, "f32",
                   parts, S_DENSE) for name, parts in DENSE_LAUNCHES]


def mixed_launches(batch: int) -> list[Launch]:
    info = {n: (t, N, K) for n, t, N, K in MIXED_PROJ}
    return [Launch("mixed_b%d" % batch, name, info[parts[0]][0], sum(info[p][1] for p in parts), info[parts[0]][2],
                   batch, "bf16", parts, S_MIXED) for name, parts in MIXED_LAUNCHES]


# the headline: the dense layer at one vector
HEADLINE = dense_launches(1)
# the launch whose roofline the bench reports (the largest of the headline step)
DOMINANT = HEADLINE[2]

MIXED_BATCHES = (1, 2, 8, 16)

TIMED_MATVEC: list[Launch] = (
    HEADLINE + dense_launches(4) + [l for B in MIXED_BATCHES for l in mixed_launches(B)] +
    [Launch("q4_0_2048", "w", "q4_0", 2048, 2048, 1, "f32", (), S_Q4_0)] +
    [Launch("q5_k_17408x5120", "w", "q5_k", 17408, 5120, B, "bf16", (), S_Q5_K) for B in (1, 8)])


@dataclass(frozen=True)
class GluLaunch:
    """One timed gq_matvec_glu launch (the dense layer's gate and up)."""
    t: str = "q4_k"
    N: int = 9728
    K: int = 2560
    batch: int = 1
    xdt: str = "f32"
    act: str = "silu"
    hdt: str = "f32"

    @property
    def id(self) -> str:
        return "glu-%s-%dx%d-b%d-%s-%s-h%s" % (self.t, self.N, self.K, self.batch, self.xdt, self.act, self.hdt)

    def weights(self) -> tuple[np.ndarray, np.ndarray]:
        w = _proj_weights("dense")
        return w["gate"], w["up"]

    def x(self) -> np.ndarray:
        return synth.normal_f32(synth.rng(S_DENSE, 400 + self.batch), (self.batch, self.K))


TIMED_GLU = [GluLaunch()]


@dataclass(frozen=True)
class MoeLayer:
    """The routed-expert workload: E experts of gate/up F x H and down H x F
    (Q4_0), T tokens routed top-k from seeded N(0,1) router logits."""
    E: int = 128
    H: int = 2816
    F: int = 704
    T: int = 8
    k: int = 8
    t: str = "q4_0"

    def logits(self) -> np.ndarray:
        return synth.router_logits(synth.rng(S_MOE, 0), self.T, self.E)

    def experts(self) -> dict:
        if "moe" not in _cache:
            _cache["moe"] = {"gate": synth.weight(self.t, synth.rng(S_MOE, 1), self.E * self.F, self.H),
                             "up": synth.weight(self.t, synth.rng(S_MOE, 2), self.E * self.F, self.H),
                             "down": synth.weight(self.t, synth.rng(S_MOE, 3), self.E * self.H, self.F)}
        return _cache["moe"]

    def x(self) -> np.ndarray:
        return synth.normal_f32(synth.rng(S_MOE, 10), (self.T, self.H))

    def h(self) -> np.ndarray:
        """Per-slot down-projection inputs for the launch that takes a seeded h."""
        return synth.normal_f32(synth.rng(S_MOE, 11), (self.T, self.k, self.F))


MOE = MoeLayer()


@dataclass(frozen=True)
class MatmulLaunch:
    """One timed gq_matmul launch: M bf16 activation rows against an N x K matrix."""
    t: str
    N: int
    K: int
    M: int = 3015
    stream: int = 0

    @property
    def id(self) -> str:
        return "prefill-%s-%dx%dx%d" % (self.t, self.M, self.N, self.K)

    def weight(self) -> np.ndarray:
        return synth.weight(self.t, synth.rng(S_PREFILL, self.stream), self.N, self.K)

    def x_bf16_bits(self) -> np.ndarray:
        return synth.bf16_bits(synth.normal_f32(synth.rng(S_PREFILL, 100 + self.stream), (self.M, self.K)))


TIMED_MATMUL = [MatmulLaunch("q4_k", 17408, 5120, stream=0), MatmulLaunch("q6_k", 5120, 17408, stream=2),
                MatmulLaunch("q4_0", 17408, 5120, stream=4)]
