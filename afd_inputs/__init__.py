"""Seeded synthetic inputs for the MoE FFN-service layer.

This module is shared by the fp64 oracle side and the HIP side.  It only
draws random numbers and rounds them to the storage type of the workload
(bf16 or fp32); it holds none of the layer's arithmetic (no routing, no
quantisation, no GEMM).  Both sides receive the same arrays.

Workload shapes follow the FFN-side step of Attention-FFN Disaggregation
(the vLLM AFD plugin page, "FFN Service": the FFN side receives hidden
states and returns the layer output; the A/F-separation page, "深入推导":
h = 4096, k = 8 in its FP8 example).  The expert counts, intermediate sizes
and value distributions are fixed by the five workload descriptions this
package is benchmarked on (see ``CONFIGS``).

Seeding: every tensor has its own ``numpy.random.SeedSequence`` child,
addressed by a fixed spawn key, so any tensor (for instance one expert's
weights) can be drawn alone, in any order, in parallel, and always gets the
same values:

    (0,)        hidden states X            N(0, 1)
    (1,)        router weight W_r          N(0, 0.02)   (N(0, 1/sqrt(h)) for "zipf")
    (2,)        router bias permutation    (only for the "zipf" router)
    (3, e, m)   routed expert e, matrix m  N(0, 0.02)   m = 0 gate, 1 up, 2 down
    (4, s, m)   shared expert s, matrix m  N(0, 0.02)

Values are drawn as float32 (PCG64, ``standard_normal``), multiplied by the
std in float32, then kept as float32 (mode "f32") or rounded to bf16 with
round-to-nearest-even (all other modes).  bf16 arrays are returned as their
raw uint16 bit patterns.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

__all__ = ["LayerShape", "CONFIGS", "SyntheticLayer", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "tie_case"]


@dataclass(frozen=True)
class LayerShape:
    """Sizes of one MoE FFN layer and of the token batch fed to it."""
    name: str
    T: int              # tokens in the batch
    h: int              # hidden size
    E: int              # routed experts
    k: int              # experts selected per token
    I: int              # routed-expert intermediate size
    S: int = 0          # always-on shared experts
    Is: int = 0         # shared-expert intermediate size
    mode: str = "bf16"  # "f32" | "bf16" | "w8a8"
    router: str = "plain"   # "plain" | "zipf" (log-Zipf router bias)
    zipf_s: float = 1.2
    micro_batches: int = 1

    def with_tokens(self, T: int) -> "LayerShape":
        return replace(self, T=T)

    @property
    def act_dtype(self) -> str:
        return "f32" if self.mode == "f32" else "bf16"


CONFIGS = {
    # Tiny fp32 layer: T=16, h=256, E=8, top-2, I=512, no shared expert.
    "tiny_fp32": LayerShape("tiny_fp32", T=16, h=256, E=8, k=2, I=512,
                            mode="f32"),
    # Decode micro-batch: T=256, h=4096, E=64, top-8, I=1536, 1 shared (1536).
    "decode_h4096_e64": LayerShape("decode_h4096_e64", T=256, h=4096, E=64,
                                   k=8, I=1536, S=1, Is=1536, mode="bf16"),
    # DeepSeek-V3-shaped decode: T=512, h=7168, E=256, top-8, I=2048, 1 shared.
    "dsv3_decode_t512": LayerShape("dsv3_decode_t512", T=512, h=7168, E=256,
                                   k=8, I=2048, S=1, Is=2048, mode="bf16"),
    # Same shape as W8A8: T=2048, fp8 e4m3 weights with 128x128 block scales.
    "dsv3_w8a8_t2048": LayerShape("dsv3_w8a8_t2048", T=2048, h=7168, E=256,
                                  k=8, I=2048, S=1, Is=2048, mode="w8a8"),
    # Prefill chunk with Zipf(1.2)-skewed routing, 2 micro-batches of 8192.
    "prefill_skew_t16384": LayerShape("prefill_skew_t16384", T=16384, h=7168,
                                      E=256, k=8, I=2048, S=1, Is=2048,
                                      mode="bf16", router="zipf",
                                      micro_batches=2),
    # One GPU's share of the two DeepSeek-V3 decode layers under 8-way expert
    # parallelism: 32 local experts, the T*k/8 dispatched rows that arrive
    # (one local expert each), no shared expert (it stays with the tokens).
    "dsv3_ep8_shard_t512": LayerShape("dsv3_ep8_shard_t512", T=512, h=7168,
                                      E=32, k=1, I=2048, mode="bf16"),
    "dsv3_w8a8_ep8_shard_t2048": LayerShape("dsv3_w8a8_ep8_shard_t2048", T=2048,
                                            h=7168, E=32, k=1, I=2048,
                                            mode="w8a8"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits.

    Inputs here are finite normals, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _normal(seed: int, key: tuple, n: int, std: float) -> np.ndarray:
    ss = np.random.SeedSequence(seed, spawn_key=key)
    g = np.random.Generator(np.random.PCG64(ss))
    v = g.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


class SyntheticLayer:
    """Lazily drawn, seeded tensors of one synthetic MoE layer.

    Storage types: mode "f32" -> float32 arrays; otherwise bf16 bit patterns
    (uint16).  The W8A8 mode draws the same bf16 tensors as the bf16 mode;
    each side then quantises them itself."""

    WEIGHT_STD = 0.02

    def __init__(self, shape: LayerShape, seed: int = 0):
        self.shape = shape
        self.seed = int(seed)
        self._hidden = None

    # -- storage conversion -------------------------------------------------
    def _store(self, v32: np.ndarray) -> np.ndarray:
        if self.shape.mode == "f32":
            return v32
        return f32_to_bf16_bits(v32)

    # -- tensors ------------------------------------------------------------
    def hidden(self) -> np.ndarray:
        """X [T, h]: N(0, 1)."""
        if self._hidden is None:
            s = self.shape
            v = _normal(self.seed, (0,), s.T * s.h, 1.0).reshape(s.T, s.h)
            self._hidden = self._store(v)
        return self._hidden

    def router_weight(self) -> np.ndarray:
        """W_r [E, h]: N(0, 0.02); N(0, 1/sqrt(h)) for the Zipf router so that
        the unbiased logits are close to N(0, 1)."""
        s = self.shape
        std = (1.0 / math.sqrt(s.h)) if s.router == "zipf" else self.WEIGHT_STD
        return self._store(_normal(self.seed, (1,), s.E * s.h, std)
                           .reshape(s.E, s.h))

    def router_bias(self) -> Optional[np.ndarray]:
        """b [E] float32 = log p_e, p_e proportional to rank^-zipf_s, ranks
        assigned to experts by a seeded permutation.  None if unbiased."""
        s = self.shape
        if s.router != "zipf":
            return None
        ss = np.random.SeedSequence(self.seed, spawn_key=(2,))
        perm = np.random.Generator(np.random.PCG64(ss)).permutation(s.E)
        rank = perm.astype(np.float64) + 1.0
        logp = -s.zipf_s * np.log(rank)
        logp -= np.log(np.sum(np.exp(-s.zipf_s * np.log(np.arange(1, s.E + 1,
                                                                  dtype=np.float64)))))
        return logp.astype(np.float32)

    def expert(self, e: int):
        """(gate [I, h], up [I, h], down [h, I]) of routed expert e."""
        s = self.shape
        return tuple(
            self._store(_normal(self.seed, (3, e, m), s.I * s.h, self.WEIGHT_STD)
                        .reshape(shp))
            for m, shp in enumerate(((s.I, s.h), (s.I, s.h), (s.h, s.I))))

    def shared(self, j: int):
        """(gate [Is, h], up [Is, h], down [h, Is]) of shared expert j."""
        s = self.shape
        return tuple(
            self._store(_normal(self.seed, (4, j, m), s.Is * s.h, self.WEIGHT_STD)
                        .reshape(shp))
            for m, shp in enumerate(((s.Is, s.h), (s.Is, s.h), (s.h, s.Is))))

    def stacked_experts(self, threads: int = 16):
        """All routed experts stacked: gate [E,I,h], up [E,I,h], down [E,h,I]."""
        s = self.shape
        dt = np.float32 if s.mode == "f32" else np.uint16
        gate = np.empty((s.E, s.I, s.h), dt)
        up = np.empty((s.E, s.I, s.h), dt)
        down = np.empty((s.E, s.h, s.I), dt)

        def fill(e):
            g, u, d = self.expert(e)
            gate[e], up[e], down[e] = g, u, d

        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(fill, range(s.E)))
        return gate, up, down

    def stacked_shared(self):
        """All shared experts stacked: gate [S,Is,h], up [S,Is,h], down [S,h,Is]."""
        s = self.shape
        parts = [self.shared(j) for j in range(s.S)]
        if not parts:
            return None
        return tuple(np.stack([p[m] for p in parts]) for m in range(3))


def tie_case(T: int, h: int, E: int, seed: int = 0, span: int = 2):
    """Integer-valued hidden states and router weights (bf16 bit patterns).

    With |x| and |w| small integers every product and every partial sum is an
    integer far below 2^24, so fp32 and fp64 dot products agree exactly in any
    order, and equal logits are common: this exposes the tie-break rule."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = g.integers(-span, span + 1, size=(T, h)).astype(np.float32)
    w = g.integers(-1, 2, size=(E, h)).astype(np.float32)
    # Duplicate some router rows so that exact ties between experts occur.
    for e in range(1, E, 3):
        w[e] = w[e - 1]
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)
