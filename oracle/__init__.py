"""Python access to the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users.  The HIP library never
imports, links or calls anything in this package.

``load()`` compiles ``moe_oracle.c`` and ``gdn_oracle.c`` with gcc (OpenMP, -O2, no fast-math)
when the shared object is missing or older than the source, then wraps it.
``build(mutant=n)`` produces a build with planted mistake ``n`` for the
mutation tests.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
SRCS = [SRC, os.path.join(HERE, "gdn_oracle.c")]
LIB = os.path.join(HERE, "libmoe_oracle.so")

# Planted mistakes available through ORACLE_MUTANT (see moe_oracle.c).
MUTANTS = {
    1: "nibble order reversed inside a code word",
    2: "group bias dropped from the dequantised weight",
    3: "scale/bias taken from the wrong group",
    4: "top-k tie goes to the higher expert index",
    5: "top-k picks the smallest logits",
    6: "routing weights not renormalised over the selected experts",
    7: "shared-expert gate uses sigmoid(-z)",
    8: "permutation not stable inside an expert segment",
    9: "silu evaluated as g*sigmoid(-g)",
    10: "SwiGLU intermediate not rounded to bf16",
    11: "down-projection output rows reversed",
    12: "combine drops the shared expert",
    13: "bf16 rounding breaks ties away from zero",
    14: "combine reads the routed rows through a transposed slot index",
    15: "greedy selection breaks ties toward the higher token",
    16: "embedding lookup reads the neighbouring row",
    17: "gated delta rule decays the new write as well",
    18: "gated delta rule erases with beta = 1",
    19: "gated delta rule maps value head h to key head h % hk",
    20: "gated delta rule output read before the token's update",
}


def build(out: Optional[str] = None, mutant: int = 0, force: bool = False) -> str:
    out = out or LIB
    if (not force and mutant == 0 and os.path.exists(out)
            and all(os.path.getmtime(out) >= os.path.getmtime(f) for f in SRCS)):
        return out
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", *SRCS, "-o", out + ".tmp", "-lm"]
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Dims(C.Structure):
    _fields_ = [("E", C.c_int), ("topk", C.c_int), ("H", C.c_int), ("I", C.c_int),
                ("G", C.c_int)]


class _QFFN(C.Structure):
    _fields_ = [("gate_q", C.c_void_p), ("up_q", C.c_void_p), ("down_q", C.c_void_p),
                ("gate_s", C.c_void_p), ("gate_b", C.c_void_p), ("up_s", C.c_void_p),
                ("up_b", C.c_void_p), ("down_s", C.c_void_p), ("down_b", C.c_void_p)]


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _dims(d) -> _Dims:
    return _Dims(d.E, d.topk, d.H, d.I, d.G)


def _qffn(q) -> _QFFN:
    return _QFFN(_p(q.gate_q), _p(q.up_q), _p(q.down_q), _p(q.gate_s), _p(q.gate_b),
                 _p(q.up_s), _p(q.up_b), _p(q.down_s), _p(q.down_b))


@dataclass
class RouteOut:
    ids: np.ndarray      # int32 [T, topk]
    w: np.ndarray        # float64 [T, topk]
    sg: np.ndarray       # float64 [T]
    logits: np.ndarray   # float64 [T, E]
    gap: np.ndarray      # float64 [T]


@dataclass
class PermOut:
    counts: np.ndarray
    offsets: np.ndarray
    perm: np.ndarray
    inv: np.ndarray


@dataclass
class LayerOut:
    y: np.ndarray        # uint16 bf16 bits [T, H]
    y32: np.ndarray      # float64 [T, H] before the final rounding
    ids: np.ndarray
    w: np.ndarray
    sg: np.ndarray
    gap: np.ndarray


@dataclass
class GdnOut:
    o: np.ndarray        # float64 [T, hv, dv]
    o_bf16: np.ndarray   # uint16 bf16 bits [T, hv, dv]
    state: np.ndarray    # float64 [hv, dv, dk]: the state after the last token


@dataclass
class GreedyOut:
    token: np.ndarray    # int32 [T]
    logits: np.ndarray   # float64 [T, V] (before the fp32 rounding)
    gap: np.ndarray      # float64 [T]: selected fp32 logit - best other fp32 logit


class Oracle:
    def __init__(self, path: Optional[str] = None):
        self.path = path or build()
        L = C.CDLL(self.path)
        self.lib = L
        vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64
        L.oracle_mutant.restype = i32
        L.oracle_threads.restype = i32
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = None
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_fp16_to_double.argtypes = [C.c_uint16]
        L.oracle_fp16_to_double.restype = C.c_double
        L.oracle_double_to_bf16.argtypes = [C.c_double]
        L.oracle_double_to_bf16.restype = C.c_uint16
        for fn in ("oracle_round_bf16_array", "oracle_fp16_decode_array",
                   "oracle_bf16_decode_array"):
            getattr(L, fn).argtypes = [vp, vp, i64]
            getattr(L, fn).restype = None
        L.oracle_dequant.argtypes = [vp, vp, vp, i64, i32, i32, i32]
        L.oracle_dequant.restype = C.c_double
        L.oracle_route.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_route.restype = i32
        L.oracle_permute.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        L.oracle_permute.restype = i32
        L.oracle_expert_ffn.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp]
        L.oracle_expert_ffn.restype = i32
        L.oracle_combine.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_combine.restype = i32
        L.oracle_layer_forward.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp]
        L.oracle_layer_forward.restype = i32
        L.oracle_lm_head_argmax.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_lm_head_argmax.restype = i32
        L.oracle_embed.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_gdn_scan.argtypes = [i32] * 5 + [vp] * 9
        L.oracle_gdn_scan.restype = i32
        L.oracle_embed.restype = i32
        self.mutant = L.oracle_mutant()

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        """Thread count of the OpenMP loops from here on (timing only)."""
        self.lib.oracle_set_threads(int(n))

    # ---- formats
    def round_bf16(self, a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, np.uint16)
        self.lib.oracle_round_bf16_array(_p(a), _p(out), a.size)
        return out

    def fp16_decode(self, bits) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float64)
        self.lib.oracle_fp16_decode_array(_p(bits), _p(out), bits.size)
        return out

    def bf16_decode(self, bits) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float64)
        self.lib.oracle_bf16_decode_array(_p(bits), _p(out), bits.size)
        return out

    def dequant(self, q, s, b, row: int, K: int, G: int, k: int) -> float:
        return self.lib.oracle_dequant(_p(q), _p(s), _p(b), row, K, G, k)

    # ---- stages
    def route(self, layer, x: np.ndarray, forced_ids=None) -> RouteOut:
        d = layer.dims
        T = x.shape[0]
        ids = np.empty((T, d.topk), np.int32)
        w = np.empty((T, d.topk), np.float64)
        sg = np.empty((T,), np.float64)
        logits = np.empty((T, d.E), np.float64)
        gap = np.empty((T,), np.float64)
        fi = None if forced_ids is None else np.ascontiguousarray(forced_ids, np.int32)
        rc = self.lib.oracle_route(C.byref(_dims(d)), T, _p(x), _p(layer.w_router),
                                   _p(layer.router_bias), _p(layer.w_shared_gate), _p(fi),
                                   _p(ids), _p(w), _p(sg), _p(logits), _p(gap))
        if rc:
            raise ValueError(f"oracle_route failed ({rc})")
        return RouteOut(ids, w, sg, logits, gap)

    def permute(self, dims, ids: np.ndarray) -> PermOut:
        ids = np.ascontiguousarray(ids, np.int32)
        T = ids.shape[0]
        n = T * dims.topk
        counts = np.empty(dims.E, np.int32)
        offsets = np.empty(dims.E + 1, np.int32)
        perm = np.empty(n, np.int32)
        inv = np.empty(n, np.int32)
        rc = self.lib.oracle_permute(C.byref(_dims(dims)), T, _p(ids), _p(counts),
                                     _p(offsets), _p(perm), _p(inv))
        if rc:
            raise ValueError(f"oracle_permute failed ({rc})")
        return PermOut(counts, offsets, perm, inv)

    def expert_ffn(self, layer, x: np.ndarray, offsets, perm, rows=None,
                   want_h: bool = False):
        d = layer.dims
        T = x.shape[0]
        offsets = np.ascontiguousarray(offsets, np.int32)
        perm = np.ascontiguousarray(perm, np.int32)
        if rows is None:
            n = (d.topk + 1) * T
            rr = None
        else:
            rr = np.ascontiguousarray(rows, np.int32)
            n = rr.size
        out = np.empty((n, d.H), np.float64)
        hb = np.empty((n, d.I), np.uint16) if want_h else None
        rc = self.lib.oracle_expert_ffn(C.byref(_dims(d)), T, _p(x),
                                        C.byref(_qffn(layer.routed)),
                                        C.byref(_qffn(layer.shared)), _p(offsets), _p(perm),
                                        _p(rr), n if rr is not None else 0, _p(out), _p(hb))
        if rc:
            raise ValueError(f"oracle_expert_ffn failed ({rc})")
        return (out, hb) if want_h else out

    def combine(self, dims, out: np.ndarray, inv, w, sg):
        T = np.asarray(sg).shape[0]
        out = np.ascontiguousarray(out, np.float64)
        inv = np.ascontiguousarray(inv, np.int32)
        w = np.ascontiguousarray(w, np.float64)
        sg = np.ascontiguousarray(sg, np.float64)
        y = np.empty((T, dims.H), np.uint16)
        y32 = np.empty((T, dims.H), np.float64)
        self.lib.oracle_combine(C.byref(_dims(dims)), T, _p(out), _p(inv), _p(w), _p(sg),
                                _p(y), _p(y32))
        return y, y32

    def layer_forward(self, layer, x: np.ndarray, forced_ids=None) -> LayerOut:
        d = layer.dims
        x = np.ascontiguousarray(x, np.uint16)
        T = x.shape[0]
        y = np.empty((T, d.H), np.uint16)
        y32 = np.empty((T, d.H), np.float64)
        ids = np.empty((T, d.topk), np.int32)
        w = np.empty((T, d.topk), np.float64)
        sg = np.empty((T,), np.float64)
        gap = np.empty((T,), np.float64)
        fi = None if forced_ids is None else np.ascontiguousarray(forced_ids, np.int32)
        rc = self.lib.oracle_layer_forward(C.byref(_dims(d)), T, _p(x), _p(layer.w_router),
                                           _p(layer.router_bias), _p(layer.w_shared_gate),
                                           C.byref(_qffn(layer.routed)),
                                           C.byref(_qffn(layer.shared)), _p(fi), _p(y),
                                           _p(ids), _p(w), _p(sg), _p(gap), _p(y32))
        if rc:
            raise ValueError(f"oracle_layer_forward failed ({rc})")
        return LayerOut(y, y32, ids, w, sg, gap)


    # ---- greedy decode step
    def lm_head_argmax(self, x: np.ndarray, w_head: np.ndarray) -> GreedyOut:
        x = np.ascontiguousarray(x, np.uint16)
        w_head = np.ascontiguousarray(w_head, np.uint16)
        T, H = x.shape
        V = w_head.shape[0]
        assert w_head.shape == (V, H)
        token = np.empty((T,), np.int32)
        logits = np.empty((T, V), np.float64)
        gap = np.empty((T,), np.float64)
        rc = self.lib.oracle_lm_head_argmax(T, H, V, _p(x), _p(w_head), _p(token), _p(logits),
                                            _p(gap))
        if rc:
            raise ValueError(f"oracle_lm_head_argmax failed ({rc})")
        return GreedyOut(token, logits, gap)

    def embed(self, token: np.ndarray, emb: np.ndarray) -> np.ndarray:
        token = np.ascontiguousarray(token, np.int32)
        emb = np.ascontiguousarray(emb, np.uint16)
        V, H = emb.shape
        x = np.empty((token.shape[0], H), np.uint16)
        if self.lib.oracle_embed(token.shape[0], H, V, _p(token), _p(emb), _p(x)):
            raise ValueError("oracle_embed: token outside the table")
        return x


    # ---- gated delta rule scan
    def gdn_scan(self, q, k, v, g, beta, s0=None) -> GdnOut:
        """q, k: bf16 bits [T, hk, dk]; v: bf16 bits [T, hv, dv]; g, beta:
        float32 [T, hv]; s0: float32 [hv, dv, dk] or None (zero state)."""
        q = np.ascontiguousarray(q, np.uint16)
        k = np.ascontiguousarray(k, np.uint16)
        v = np.ascontiguousarray(v, np.uint16)
        g = np.ascontiguousarray(g, np.float32)
        beta = np.ascontiguousarray(beta, np.float32)
        T, hk, dk = k.shape
        hv, dv = v.shape[1], v.shape[2]
        assert q.shape == k.shape and v.shape[0] == T and g.shape == (T, hv) == beta.shape
        if s0 is not None:
            s0 = np.ascontiguousarray(s0, np.float32)
            assert s0.shape == (hv, dv, dk)
        o = np.empty((T, hv, dv), np.float64)
        ob = np.empty((T, hv, dv), np.uint16)
        st = np.empty((hv, dv, dk), np.float64)
        rc = self.lib.oracle_gdn_scan(T, hk, hv, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                                      _p(s0), _p(o), _p(ob), _p(st))
        if rc:
            raise ValueError(f"oracle_gdn_scan failed ({rc})")
        return GdnOut(o, ob, st)


_DEFAULT: Optional[Oracle] = None


def load() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
