"""Seeded synthetic inputs for the sparse MoE layer.

This module only draws numbers and stores them in the layer's storage
formats (bf16 bit patterns, fp16 bit patterns, packed uint32 code words).
It performs none of the layer's arithmetic, so the HIP path and the CPU
oracle can both be fed from it without sharing any of the method.

Layer shape and storage (this library's layer definition; the pages give
only the structure -- 8 of 256 routed experts plus one shared expert per
token, 4-bit weights -- see "Perplexity Open-Sources Lily ...",
section "A runtime shaped around one model"):

  x              bf16 [T, H]                       ~ N(0, 1)
  w_router       bf16 [E, H]                       ~ N(0, 0.02^2)
  w_shared_gate  bf16 [H]                          ~ N(0, 0.02^2)
  router_bias    fp32 [E] or None                  b_e = 2*ln(1/rank_e^1.2)
  per expert (E routed, 1 shared):
    gate_q, up_q uint32 [n, I, H/8]   eight 4-bit codes per word along K
    down_q       uint32 [n, H, I/8]
    *_s, *_b     fp16   [n, rows, K/G] one scale and one bias per 64-wide
                                       group along K; bias = -7.5 * scale
                                       (rounded to fp16)

Every tensor has its own PCG64 stream keyed by (seed, layer, tensor id), so
a layer is reproducible on its own and chains can be generated layer by
layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# Production shape of the layer.
HIDDEN = 2048
INTER = 512
EXPERTS = 256
TOPK = 8
GROUP = 64

# Tensor ids inside a layer's seed tree.
_TID_X = 0
_TID_WR = 1
_TID_WSG = 2
_TID_ROUTED = 3      # 3..8: gate_q, gate_s, up_q, up_s, down_q, down_s
_TID_SHARED = 9      # 9..14: same for the shared expert
_TID_RANKS = 15
_TID_HEAD = 16       # greedy step: output head [V, H]
_TID_EMB = 17        # greedy step: embedding table [V, H]
_STEP_BASE = 100000  # chain-step inputs use layer key STEP_BASE + step


@dataclass(frozen=True)
class Dims:
    """Layer dimensions. The oracle is shape generic; the HIP path is built
    for the production shape only."""
    E: int = EXPERTS
    topk: int = TOPK
    H: int = HIDDEN
    I: int = INTER
    G: int = GROUP

    def check(self) -> None:
        assert self.H % 8 == 0 and self.I % 8 == 0
        assert self.H % self.G == 0 and self.I % self.G == 0 and self.G % 8 == 0
        assert 1 <= self.topk <= self.E


PROD = Dims()


@dataclass
class QFFN:
    """Quantised SwiGLU expert stack (n experts), numpy host storage."""
    gate_q: np.ndarray   # uint32 [n, I, H/8]
    gate_s: np.ndarray   # uint16 (fp16 bits) [n, I, H/G]
    gate_b: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    up_b: np.ndarray
    down_q: np.ndarray   # uint32 [n, H, I/8]
    down_s: np.ndarray   # uint16 (fp16 bits) [n, H, I/G]
    down_b: np.ndarray

    FIELDS = ("gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b",
              "down_q", "down_s", "down_b")

    def arrays(self):
        return [getattr(self, f) for f in self.FIELDS]

    @property
    def nbytes(self) -> int:
        return sum(a.nbytes for a in self.arrays())


@dataclass
class Layer:
    dims: Dims
    w_router: np.ndarray           # uint16 (bf16 bits) [E, H]
    w_shared_gate: np.ndarray      # uint16 (bf16 bits) [H]
    routed: QFFN
    shared: QFFN
    router_bias: Optional[np.ndarray] = None   # float32 [E]
    meta: dict = field(default_factory=dict)


def _rng(seed: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=(layer, tensor_id))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store float32 values as bf16 bit patterns (round to nearest even,
    done by torch's dtype conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_fp16_bits(a: np.ndarray) -> np.ndarray:
    """Store float32 values as IEEE binary16 bit patterns (numpy's RNE cast)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    # Uniform 32-bit words = eight independent uniform 4-bit codes each.
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint32)


def _scales_biases(rng: np.random.Generator, shape):
    scale = (rng.random(shape) * 1.0 + 0.5) * 0.003          # U(0.5,1.5)*0.003
    s16 = scale.astype(np.float32).astype(np.float16)
    b16 = (np.float32(-7.5) * s16.astype(np.float32)).astype(np.float16)
    return s16.view(np.uint16), b16.view(np.uint16)


def make_qffn(dims: Dims, n: int, seed: int, layer: int, tid0: int) -> QFFN:
    H, I, G = dims.H, dims.I, dims.G
    gq = _codes(_rng(seed, layer, tid0 + 0), (n, I, H // 8))
    gs, gb = _scales_biases(_rng(seed, layer, tid0 + 1), (n, I, H // G))
    uq = _codes(_rng(seed, layer, tid0 + 2), (n, I, H // 8))
    us, ub = _scales_biases(_rng(seed, layer, tid0 + 3), (n, I, H // G))
    dq = _codes(_rng(seed, layer, tid0 + 4), (n, H, I // 8))
    ds, db = _scales_biases(_rng(seed, layer, tid0 + 5), (n, H, I // G))
    return QFFN(gq, gs, gb, uq, us, ub, dq, ds, db)


def make_layer(dims: Dims = PROD, seed: int = 0, layer: int = 0,
               skewed_bias: bool = False) -> Layer:
    """One seeded MoE layer. ``skewed_bias`` adds the Zipf-like router bias
    b_e = 2*ln(1/rank_e^1.2) with ranks a seeded permutation of 1..E."""
    dims.check()
    E, H = dims.E, dims.H
    wr = 0.02 * _rng(seed, layer, _TID_WR).standard_normal((E, H), dtype=np.float32)
    wsg = 0.02 * _rng(seed, layer, _TID_WSG).standard_normal((H,), dtype=np.float32)
    routed = make_qffn(dims, E, seed, layer, _TID_ROUTED)
    shared = make_qffn(dims, 1, seed, layer, _TID_SHARED)
    bias = None
    if skewed_bias:
        ranks = _rng(seed, layer, _TID_RANKS).permutation(E) + 1
        bias = (2.0 * np.log(1.0 / ranks.astype(np.float64) ** 1.2)).astype(np.float32)
    return Layer(dims, f32_to_bf16_bits(wr), f32_to_bf16_bits(wsg), routed, shared,
                 bias, {"seed": seed, "layer": layer, "skewed_bias": skewed_bias})


def make_x(T: int, dims: Dims = PROD, seed: int = 0, layer: int = 0,
           step: Optional[int] = None) -> np.ndarray:
    """Token activations, bf16 bits [T, H], ~N(0,1). Chain steps draw from
    their own stream (layer key STEP_BASE + step)."""
    key = layer if step is None else _STEP_BASE + step
    a = _rng(seed, key, _TID_X).standard_normal((T, dims.H), dtype=np.float32)
    return f32_to_bf16_bits(a)


def make_head(V: int, dims: Dims = PROD, seed: int = 0) -> tuple:
    """The greedy decode step's synthetic tables (the pages give none): an
    output head and an embedding table, bf16 bits [V, H], ~N(0, 0.02^2)."""
    head = 0.02 * _rng(seed, 0, _TID_HEAD).standard_normal((V, dims.H), dtype=np.float32)
    emb = 0.02 * _rng(seed, 0, _TID_EMB).standard_normal((V, dims.H), dtype=np.float32)
    return f32_to_bf16_bits(head), f32_to_bf16_bits(emb)


# ---- hand-built layers for closed-form pins -------------------------------

def constant_layer(dims: Dims, code: int, scale_bits: int, bias_bits: int,
                   w_router: Optional[np.ndarray] = None,
                   w_shared_gate: Optional[np.ndarray] = None) -> Layer:
    """Every expert identical: all codes equal ``code``, every group has the
    given fp16 scale/bias bit patterns."""
    E, H, I, G = dims.E, dims.H, dims.I, dims.G
    word = np.uint32(sum(code << (4 * i) for i in range(8)))

    def q(n):
        return QFFN(np.full((n, I, H // 8), word, np.uint32),
                    np.full((n, I, H // G), scale_bits, np.uint16),
                    np.full((n, I, H // G), bias_bits, np.uint16),
                    np.full((n, I, H // 8), word, np.uint32),
                    np.full((n, I, H // G), scale_bits, np.uint16),
                    np.full((n, I, H // G), bias_bits, np.uint16),
                    np.full((n, H, I // 8), word, np.uint32),
                    np.full((n, H, I // G), scale_bits, np.uint16),
                    np.full((n, H, I // G), bias_bits, np.uint16))
    wr = w_router if w_router is not None else np.zeros((E, H), np.uint16)
    wsg = w_shared_gate if w_shared_gate is not None else np.zeros((H,), np.uint16)
    return Layer(dims, wr, wsg, q(E), q(1), None, {"constant": code})


# ------------------------------------------------- gated delta rule inputs
#
# One recurrent (Gated DeltaNet) layer's scan inputs, shapes of the
# published layer form this library takes (the pages give none): hk key
# heads and hv value heads of dimension 128 (hv a multiple of hk), for T
# tokens of one sequence.
#   k      bf16 [T, hk, d]   unit-length random directions
#   q      bf16 [T, hk, d]   unit-length random directions / sqrt(d)
#   v      bf16 [T, hv, d]   ~ N(0, 1)
#   beta   fp32 [T, hv]      1 / (1 + exp(-z)), z ~ N(0, 1)
#   g      fp32 [T, hv]      -log(1 + exp(z)), z ~ N(-4.5, 1) (decay e^g
#                            around 0.99 per token, about 0.5 per 64 tokens)
#   s0     fp32 [hv, d, d]   ~ N(0, 0.05^2) (a state carried in), optional
GDN_DIM = 128
GDN_HK = 16
GDN_HV = 32
_TID_GDN = 20        # 20..25: q, k, v, beta, g, s0


@dataclass
class GdnInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    s0: Optional[np.ndarray]


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def make_gdn(T: int, hk: int = GDN_HK, hv: int = GDN_HV, d: int = GDN_DIM, seed: int = 0,
             with_state: bool = True) -> GdnInputs:
    q = f32_to_bf16_bits(_unit_rows(_rng(seed, 0, _TID_GDN), (T, hk, d)) / np.float32(np.sqrt(d)))
    k = f32_to_bf16_bits(_unit_rows(_rng(seed, 0, _TID_GDN + 1), (T, hk, d)))
    v = f32_to_bf16_bits(_rng(seed, 0, _TID_GDN + 2).standard_normal((T, hv, d), dtype=np.float32))
    zb = _rng(seed, 0, _TID_GDN + 3).standard_normal((T, hv))
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    zg = _rng(seed, 0, _TID_GDN + 4).normal(-4.5, 1.0, (T, hv))
    g = (-np.log1p(np.exp(zg))).astype(np.float32)
    s0 = None
    if with_state:
        s0 = (0.05 * _rng(seed, 0, _TID_GDN + 5).standard_normal((hv, d, d))).astype(np.float32)
    return GdnInputs(q, k, v, g, beta, s0)
