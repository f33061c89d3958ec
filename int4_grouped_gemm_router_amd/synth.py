"""Seeded synthetic inputs for the int4 MoE layer.

Shared by the tests, the bench and the smoke check, on both sides of the
parity comparison. This module holds random draws and the rounding of drawn
values to bf16 only: none of the layer's arithmetic lives here.

Recipe (one numpy ``default_rng(seed)`` per workload; draws in this order):
  1. router weights Wr ~ N(0, 0.02^2) fp32, shape [E, H];
  2. for each expert e = 0..E-1, then the shared expert: for gate, up, down in
     turn, q ~ U{0..15} (uint8) then scale ~ U(0.005, 0.02) rounded to bf16;
     bias = -8 * scale (exact in bf16);
  3. skewed routing only: a random permutation of the E experts; expert e's
     router logit bias is -s * ln(rank_e), rank_e = 1 + its position in the
     permutation, s = 1.1 (a Zipf prior over experts, added to the logit);
  4. activations x ~ N(0, 1) rounded to bf16, shape [T, H] (decode workloads
     draw one such x per step).
The pages measure whole-model prompts and decode on a trained checkpoint;
these synthetic tensors stand in for them with the layer's shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

MATS = ("gate", "up", "down")


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round-to-nearest-even of finite float32 values to bf16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class LayerWeights:
    """Logical (unpacked) weights of one layer: E routed experts + 1 shared.

    q[m]     uint8  [E+1, rows, cols]   (gate/up: rows=I, cols=H; down: rows=H, cols=I)
    scale[m] uint16 [E+1, rows, cols/64] bf16 bits
    bias[m]  uint16 [E+1, rows, cols/64] bf16 bits
    Index E is the shared expert.
    """
    H: int
    I: int
    E: int
    router_w: np.ndarray
    router_bias: Optional[np.ndarray]
    q: Dict[str, np.ndarray] = field(default_factory=dict)
    scale: Dict[str, np.ndarray] = field(default_factory=dict)
    bias: Dict[str, np.ndarray] = field(default_factory=dict)

    def expert(self, e, m):
        return self.q[m][e], self.scale[m][e], self.bias[m][e]


def _shape(m, H, I):
    return (I, H) if m in ("gate", "up") else (H, I)


def make_weights(rng, H, I, E=256, skew=False, zipf_s=1.1) -> LayerWeights:
    router_w = rng.normal(0.0, 0.02, size=(E, H)).astype(np.float32)
    w = LayerWeights(H=H, I=I, E=E, router_w=router_w, router_bias=None)
    for m in MATS:
        rows, cols = _shape(m, H, I)
        w.q[m] = np.empty((E + 1, rows, cols), np.uint8)
        w.scale[m] = np.empty((E + 1, rows, cols // 64), np.uint16)
        w.bias[m] = np.empty((E + 1, rows, cols // 64), np.uint16)
    for e in range(E + 1):
        for m in MATS:
            rows, cols = _shape(m, H, I)
            w.q[m][e] = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
            s = rng.uniform(0.005, 0.02, size=(rows, cols // 64)).astype(np.float32)
            sb = f32_to_bf16_bits(s)
            w.scale[m][e] = sb
            w.bias[m][e] = f32_to_bf16_bits(-8.0 * bf16_bits_to_f32(sb))
    if skew:
        perm = rng.permutation(E)
        rank = np.empty(E, np.float64)
        rank[perm] = np.arange(1, E + 1)
        w.router_bias = (-zipf_s * np.log(rank)).astype(np.float32)
    return w


def make_x(rng, T, H) -> np.ndarray:
    return f32_to_bf16_bits(rng.normal(0.0, 1.0, size=(T, H)).astype(np.float32))


@dataclass
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int = 256
    k: int = 8
    skew: bool = False
    chunk: int = 0          # 0: one pass over all T tokens
    steps: int = 0          # decode: number of steps with fresh x
    describe: str = ""


WORKLOADS = {
    "tiny_t32": Workload("tiny_t32", T=32, H=512, I=128,
                         describe="T=32, H=512, I=128, E=256 top-8 + shared"),
    "prefill_t512": Workload("prefill_t512", T=512, H=2048, I=512,
                             describe="T=512, H=2048, I=512, E=256 top-8 + shared, uniform routing"),
    "skew_t2048": Workload("skew_t2048", T=2048, H=2048, I=512, skew=True,
                           describe="T=2048, Zipf(1.1)-skewed router bias"),
    "long_t16384": Workload("long_t16384", T=16384, H=2048, I=512, chunk=4096,
                            describe="T=16384 in 4096-token chunks"),
    "decode_t1": Workload("decode_t1", T=1, H=2048, I=512, steps=1000,
                          describe="batch-1 decode, 1000 steps"),
    "decode_t4": Workload("decode_t4", T=4, H=2048, I=512, steps=1000,
                          describe="T=4 decode, 1000 steps"),
}


def generate(name_or_wl, seed=0, T=None, steps=None, with_x=True):
    """Weights and activations for a named workload.

    Returns (workload, LayerWeights, x) where x is [T, H] bf16 bits, or
    [steps, T, H] for decode workloads. ``T``/``steps`` override the sizes
    (tests use them to shrink a workload without changing its recipe).
    """
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    T = wl.T if T is None else T
    steps = wl.steps if steps is None else steps
    rng = np.random.default_rng(seed)
    w = make_weights(rng, wl.H, wl.I, wl.E, skew=wl.skew)
    x = None
    if with_x:
        if steps:
            x = np.stack([make_x(rng, T, wl.H) for _ in range(steps)])
        else:
            x = make_x(rng, T, wl.H)
    return wl, w, x


def random_logits(rng, T, E, ties=0):
    """Synthetic fp32 router logits for routing-only tests.

    ``ties`` > 0 rounds the logits to multiples of 2**-ties, so that many exact
    ties occur (also across the 8th/9th rank).
    """
    l = rng.normal(0.0, 1.0, size=(T, E)).astype(np.float32)
    if ties:
        q = np.float32(2.0 ** -ties)
        l = (np.round(l / q) * q).astype(np.float32)
    return l
