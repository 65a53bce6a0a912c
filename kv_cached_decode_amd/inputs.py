"""Seeded synthetic inputs shaped like the decode workloads.

This module only draws random numbers and casts them once, round-to-nearest-
even, to the storage dtype. It holds no step of the decode method. The HIP
path and the CPU oracle both consume the arrays it returns.

Storage arrays are numpy: ``np.float32`` for f32, ``np.float16`` for f16 and
``np.uint16`` bit patterns for bf16.

Every tensor comes from its own generator, keyed by (seed, stream id, layer,
...), so a test can regenerate one layer or one step without drawing the rest.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# stream ids: each kind of tensor draws from its own numpy SeedSequence branch
_S_SELF_K, _S_SELF_V, _S_CROSS_K, _S_CROSS_V = 1, 2, 3, 4
_S_Q_SELF, _S_Q_CROSS, _S_PARENT, _S_LOGITS, _S_DRAFT = 5, 6, 7, 8, 9
_S_BEAM_LOGITS, _S_BEAM_SCORES = 10, 11


def rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), *[int(k) for k in key]])


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 draws to the storage dtype once (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(g: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return to_storage(x, dtype)


@dataclass(frozen=True)
class Workload:
    """Shape of one decode workload (all sizes per GPU)."""

    name: str
    layers: int
    B: int          # batch rows (beams count as rows)
    Hq: int
    Hkv: int
    D: int
    S_max: int      # self-cache capacity
    frames: int     # cross-cache length (0: decoder-only, no cross attention)
    dtype: str
    scale: float    # standard deviation of q, k, v draws
    seed: int
    rope_base: float = 0.0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def attn_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


# The five workloads. Shapes: Whisper large-v2 decoder (32 layers, 20 heads of
# 64, 448 text positions, 1500 encoder frames) and a GQA decoder-only LM
# (30 layers, 9 query / 3 KV heads of 64, RoPE base 10000).
TINY = Workload("tiny decode step: 1 layer, B1, 6 heads x 64, fp32, self 32+1, cross 1500",
                1, 1, 6, 6, 64, 33, 1500, "f32", 1.0, seed=1)
WHISPER_GREEDY = Workload(
    "whisper-large-v2 greedy decode: 32 layers, B1, 20 heads x 64, fp16, self 1..448, cross 1500",
    32, 1, 20, 20, 64, 448, 1500, "f16", 1.0 / 8.0, seed=2)
WHISPER_VERIFY = Workload(
    "whisper-large-v2 speculative verify: N=5 drafts, self 64..448, cross 1500, vocab 51865",
    32, 1, 20, 20, 64, 448, 1500, "f16", 1.0 / 8.0, seed=3,
    extra={"N": 5, "V": 51865, "logit_sigma": 2.0, "p_match": 0.75,
           "L_before": (64, 128, 192, 256, 320, 384, 443)})
WHISPER_BEAM = Workload(
    "whisper-large-v2 beam search: 5 beams, 224 steps, fp16, cross 1500 shared",
    32, 5, 20, 20, 64, 448, 1500, "f16", 1.0 / 8.0, seed=4, extra={"steps": 224})
GQA_PREFILL_DECODE = Workload(
    "GQA LM prefill 512 + decode to 1024: 30 layers, B8, 9q/3kv heads x 64, bf16, RoPE",
    30, 8, 9, 3, 64, 1024, 0, "bf16", 1.0, seed=5, rope_base=10000.0,
    extra={"prefill": 512, "decode": 512})

WORKLOADS = {
    "tiny": TINY,
    "whisper_greedy": WHISPER_GREEDY,
    "whisper_verify": WHISPER_VERIFY,
    "whisper_beam": WHISPER_BEAM,
    "gqa_prefill_decode": GQA_PREFILL_DECODE,
}


def self_kv(w: Workload, layer: int, B: int | None = None, S: int | None = None):
    """K and V of every token position of one layer: [B, Hkv, S, D] each.

    Token t's rows are what gets appended at position t.
    """
    B = w.B if B is None else B
    S = w.S_max if S is None else S
    shape = (B, w.Hkv, S, w.D)
    return (normal(rng(w.seed, _S_SELF_K, layer), shape, w.dtype, w.scale),
            normal(rng(w.seed, _S_SELF_V, layer), shape, w.dtype, w.scale))


def cross_kv(w: Workload, layer: int, Bkv: int = 1):
    """Encoder-derived cross K and V of one layer: [Bkv, Hkv, frames, D]."""
    shape = (Bkv, w.Hkv, w.frames, w.D)
    return (normal(rng(w.seed, _S_CROSS_K, layer), shape, w.dtype, w.scale),
            normal(rng(w.seed, _S_CROSS_V, layer), shape, w.dtype, w.scale))


def queries(w: Workload, layer: int, step: int, N: int = 1, cross: bool = False,
            B: int | None = None):
    """Query rows of one layer at one step: [B, Hq, N, D]."""
    B = w.B if B is None else B
    sid = _S_Q_CROSS if cross else _S_Q_SELF
    return normal(rng(w.seed, sid, layer, step), (B, w.Hq, N, w.D), w.dtype, w.scale)


def parents(w: Workload, step: int) -> np.ndarray:
    """Beam parent indices of one step, uniform in [0, B): int32[B]."""
    return rng(w.seed, _S_PARENT, step).integers(0, w.B, size=w.B, dtype=np.int64).astype(np.int32)


def verify_logits(w: Workload, trial: int, B: int = 1, R: int | None = None,
                  V: int | None = None, plant: bool = True):
    """Logits rows ~ N(0, sigma^2) and the drafts that go with them.

    With ``plant`` each row gets one token raised to 7 sigma above the mean, so
    that row's argmax is (almost surely) that token; a draft copies the planted
    token with probability p_match and is uniform in [0, V) otherwise. The
    planted token is not an oracle result: the oracle and the kernel each
    compute the real argmax of every row.
    Returns (logits f32 [B, R, V], draft int32 [B, N]).
    """
    N = w.extra["N"]
    R = N if R is None else R
    V = w.extra["V"] if V is None else V
    sigma = w.extra["logit_sigma"]
    g = rng(w.seed, _S_LOGITS, trial)
    logits = (g.standard_normal(size=(B, R, V), dtype=np.float32) * np.float32(sigma))
    gd = rng(w.seed, _S_DRAFT, trial)
    planted = gd.integers(0, V, size=(B, R))
    if plant:
        for b in range(B):
            for r in range(R):
                logits[b, r, planted[b, r]] = np.float32(7.0 * sigma)
    match = gd.random(size=(B, N)) < w.extra["p_match"]
    rand_tok = gd.integers(0, V, size=(B, N))
    draft = np.where(match, planted[:, :N], rand_tok).astype(np.int32)
    return np.ascontiguousarray(logits), np.ascontiguousarray(draft)


def beam_logits(w: Workload, step: int, B: int = 1, K: int | None = None, V: int = 51865,
                sigma: float = 2.0):
    """Beam-search scoring inputs of one step: logits [B, K, V] ~ N(0,
    sigma^2) (f32) and running scores [B, K], uniform in [-step - 1, -step]
    (running log-probabilities fall as a sequence grows)."""
    K = w.B if K is None else K
    g = rng(w.seed, _S_BEAM_LOGITS, step)
    logits = g.standard_normal(size=(B, K, V), dtype=np.float32) * np.float32(sigma)
    sums = (rng(w.seed, _S_BEAM_SCORES, step).random(size=(B, K)) - 1.0 - step).astype(np.float32)
    return np.ascontiguousarray(logits), np.ascontiguousarray(sums)

