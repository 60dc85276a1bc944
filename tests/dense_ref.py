"""Dense, all-experts NumPy evaluation of the MoE layer.

An independent second implementation used only to pin the C oracle: it
dequantises whole weight matrices with vectorised numpy, evaluates EVERY
routed expert on every token and masks the result with the renormalised
routing weights, instead of gathering the selected experts.  It shares no
code with the oracle (fp16 decoding goes through numpy's float16, bf16
rounding through torch's dtype conversion, softmax/sigmoid through scipy).

torch converts float64 to bfloat16 through float32, i.e. with a double
rounding; the two roundings differ only when a value lies within 2^-29
relative of a bf16 midpoint, so comparisons against the oracle allow a
handful of one-ulp flips.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def unpack_codes(q: np.ndarray, K: int) -> np.ndarray:
    """uint32 [..., K/8] -> codes [..., K], code k in bits 4*(k%8).. of word k/8."""
    shifts = (np.arange(8, dtype=np.uint32) * 4)
    c = (q[..., :, None] >> shifts) & np.uint32(0xF)
    return c.reshape(*q.shape[:-1], K)


def dequant(q: np.ndarray, s: np.ndarray, b: np.ndarray, K: int, G: int) -> np.ndarray:
    codes = unpack_codes(q, K).astype(np.float64)
    sc = np.repeat(fp16_to_f64(s), G, axis=-1)
    bi = np.repeat(fp16_to_f64(b), G, axis=-1)
    return codes * sc + bi


def expert_dense(qffn, e: int, x: np.ndarray, dims):
    """SwiGLU expert e of a QFFN stack on real rows x [T, H] -> (d [T,H], h bits)."""
    H, I, G = dims.H, dims.I, dims.G
    Wg = dequant(qffn.gate_q[e], qffn.gate_s[e], qffn.gate_b[e], H, G)   # [I, H]
    Wu = dequant(qffn.up_q[e], qffn.up_s[e], qffn.up_b[e], H, G)
    Wd = dequant(qffn.down_q[e], qffn.down_s[e], qffn.down_b[e], I, G)   # [H, I]
    g = x @ Wg.T
    u = x @ Wu.T
    hbits = f64_to_bf16_bits(g * scipy.special.expit(g) * u)
    h = bf16_to_f64(hbits)
    return h @ Wd.T, hbits


def route_dense(layer, x: np.ndarray):
    d = layer.dims
    Wr = bf16_to_f64(layer.w_router)
    logits = x @ Wr.T
    if layer.router_bias is not None:
        logits = logits + layer.router_bias.astype(np.float64)[None, :]
    sel = np.argsort(-logits.astype(np.float32), axis=1, kind="stable")[:, :d.topk]
    p = scipy.special.softmax(logits, axis=1)
    psel = np.take_along_axis(p, sel, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    sg = scipy.special.expit(x @ bf16_to_f64(layer.w_shared_gate))
    return logits, sel, w, sg


def layer_dense(layer, x_bits: np.ndarray):
    """Returns (y bits [T,H], y32 [T,H], ids [T,k], w [T,k], sg [T])."""
    d = layer.dims
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    logits, sel, w, sg = route_dense(layer, x)
    mask = np.zeros((T, d.E))
    np.put_along_axis(mask, sel, w, axis=1)
    y32 = np.zeros((T, d.H))
    for e in range(d.E):
        if not mask[:, e].any():
            # masked evaluation still runs every expert on tiny shapes; on
            # production shapes experts nobody selected are skipped for time
            if d.E * d.H * d.I > (1 << 22):
                continue
        de, _ = expert_dense(layer.routed, e, x, d)
        y32 += mask[:, e:e + 1] * de
    ds, _ = expert_dense(layer.shared, 0, x, d)
    y32 += sg[:, None] * ds
    return f64_to_bf16_bits(y32), y32, sel.astype(np.int32), w, sg
