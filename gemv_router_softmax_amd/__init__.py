"""Python binding of libmoe.so, the MI355X sparse mixture-of-experts layer.

Argument marshalling only: every function checks the torch tensors it is
given (device, dtype, shape, contiguity -- the C side cannot see shapes),
passes raw device pointers and the current HIP stream to the C ABI of the
same name (include/moe.h), and raises MoeError on a non-zero status.  All
computation happens in the HIP kernels; if libmoe.so is missing the calls
fail loudly, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_HIDDEN = 2048
MOE_INTER = 512
MOE_EXPERTS = 256
MOE_TOPK = 8
MOE_GROUP = 64
MOE_T_MAX = 65536
MOE_DECODE_T = 8
MOE_DECODE_T_MAX = 32
MOE_NOALLOC_T_MAX = 64
MOE_NOALLOC_WS_BYTES = 8388608

MOE_GDN_DIM = 128
MOE_GDN_CHUNK = 64
MOE_GDN_STEP_T_MAX = 48
MOE_GDN_HEADS_MAX = 64
MOE_PATH_AUTO = 0
MOE_PATH_DECODE = 1
MOE_PATH_PREFILL = 2

# Every symbol include/moe.h declares.
EXPORTS = ("moe_workspace_bytes", "moe_status_string", "moe_route", "moe_permute",
           "moe_expert_ffn", "moe_combine", "moe_layer_forward", "moe_layer_forward_ex",
           "moe_layer_forward_chunked", "moe_chain_forward", "moe_chain_forward_noalloc",
           "moe_lm_head_argmax", "moe_embed", "moe_router_transpose", "moe_probe_read",
           "moe_probe_copy", "moe_gdn_workspace_bytes", "moe_gdn_scan")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} ({status})")
        self.status = status


class moe_qffn(C.Structure):
    _fields_ = [("gate_q", C.c_void_p), ("up_q", C.c_void_p), ("down_q", C.c_void_p),
                ("gate_s", C.c_void_p), ("gate_b", C.c_void_p), ("up_s", C.c_void_p),
                ("up_b", C.c_void_p), ("down_s", C.c_void_p), ("down_b", C.c_void_p),
                ("expert_stride", C.c_int64)]


class moe_layer(C.Structure):
    _fields_ = [("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("w_shared_gate", C.c_void_p), ("routed", moe_qffn), ("shared", moe_qffn),
                ("w_router_t", C.c_void_p)]


class moe_options(C.Structure):
    _fields_ = [("path", C.c_int), ("residual_out", C.c_void_p), ("route_ids", C.c_void_p),
                ("route_w", C.c_void_p), ("route_sg", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(or python gemv_router_softmax_amd/build.py)")
    L = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int, C.c_size_t
    L.moe_workspace_bytes.argtypes = [i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = C.c_char_p
    L.moe_route.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_permute.argtypes = [vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn.argtypes = [vp, i32, C.POINTER(moe_qffn), C.POINTER(moe_qffn), vp, vp, vp,
                                 vp, sz, vp, C.POINTER(moe_options)]
    L.moe_combine.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    L.moe_layer_forward.argtypes = [vp, i32, C.POINTER(moe_layer), vp, vp, sz, vp]
    L.moe_layer_forward_ex.argtypes = [vp, i32, C.POINTER(moe_layer), vp, vp, sz, vp,
                                       C.POINTER(moe_options)]
    L.moe_layer_forward_chunked.argtypes = [vp, i32, C.POINTER(moe_layer), vp, i32, vp, vp, sz,
                                            vp]
    L.moe_chain_forward.argtypes = [vp, i32, C.POINTER(moe_layer), i32, vp, vp, vp, sz, vp,
                                    C.POINTER(moe_options)]
    L.moe_chain_forward_noalloc.argtypes = [vp, i32, C.POINTER(moe_layer), i32, vp, vp, vp,
                                            C.POINTER(moe_options)]
    L.moe_router_transpose.argtypes = [vp, vp, vp]
    L.moe_lm_head_argmax.argtypes = [vp, i32, vp, i32, vp, vp, sz, vp]
    L.moe_embed.argtypes = [vp, i32, vp, i32, vp, vp]
    L.moe_probe_read.argtypes = [vp, sz, vp, vp]
    L.moe_probe_copy.argtypes = [vp, vp, sz, vp]
    L.moe_gdn_workspace_bytes.argtypes = [i32, i32]
    L.moe_gdn_workspace_bytes.restype = sz
    L.moe_gdn_scan.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    for fn in EXPORTS:
        if fn not in ("moe_workspace_bytes", "moe_status_string", "moe_gdn_workspace_bytes"):
            getattr(L, fn).restype = i32
    _lib = L
    return L


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_workspace_bytes(T: int) -> int:
    return int(lib().moe_workspace_bytes(T))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status, moe_status_string(status))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_U16 = (torch.int16, torch.bfloat16, torch.float16, torch.uint16)
_U32 = (torch.int32, torch.uint32)


# Expert-major layout: one 2 MiB-aligned 2 MiB block per expert holding its
# nine arrays at these byte offsets (1,769,472 bytes used).
EXPERT_BLOCK = 2 << 20
_BLOCK_OFFSETS = {"gate_q": 0, "up_q": 1 << 19, "down_q": 2 << 19,
                  "gate_s": 3 << 19, "gate_b": (3 << 19) + (1 << 15), "up_s": (3 << 19) + (2 << 15),
                  "up_b": (3 << 19) + (3 << 15), "down_s": (3 << 19) + (4 << 15),
                  "down_b": (3 << 19) + (5 << 15)}


class DeviceQFFN:
    """A quantised expert stack resident in device memory.

    layout "dense" (default): the nine arrays each contiguous over experts
    (moe_qffn.expert_stride = 0); "expert": every expert's codes, scales and
    biases in one 2 MiB-aligned 2 MiB block (expert_stride = 2 MiB)."""

    def __init__(self, q, n: int, device="cuda", layout: str = "dense"):
        H, I, G = MOE_HIDDEN, MOE_INTER, MOE_GROUP
        shapes = {"gate_q": ((n, I, H // 8), np.int32), "up_q": ((n, I, H // 8), np.int32),
                  "down_q": ((n, H, I // 8), np.int32),
                  "gate_s": ((n, I, H // G), np.int16), "gate_b": ((n, I, H // G), np.int16),
                  "up_s": ((n, I, H // G), np.int16), "up_b": ((n, I, H // G), np.int16),
                  "down_s": ((n, H, I // G), np.int16), "down_b": ((n, H, I // G), np.int16)}
        arrays = {}
        for k, (shape, dt) in shapes.items():
            a = np.ascontiguousarray(getattr(q, k))
            assert a.shape == shape, (k, a.shape, shape)
            arrays[k] = a.view(dt)
        self.layout = layout
        self._nbytes = sum(a.nbytes for a in arrays.values())
        if layout == "dense":
            self.tensors = {k: torch.from_numpy(a).to(device) for k, a in arrays.items()}
            self.c = moe_qffn(**{k: v.data_ptr() for k, v in self.tensors.items()},
                              expert_stride=0)
        elif layout == "expert":
            host = np.zeros((n, EXPERT_BLOCK), dtype=np.uint8)
            for k, a in arrays.items():
                per = a.reshape(n, -1).view(np.uint8)
                o = _BLOCK_OFFSETS[k]
                host[:, o:o + per.shape[1]] = per
            self.buf = torch.empty(n * EXPERT_BLOCK + EXPERT_BLOCK, dtype=torch.uint8, device=device)
            skip = (-self.buf.data_ptr()) % EXPERT_BLOCK
            self.blocks = self.buf[skip:skip + n * EXPERT_BLOCK]
            self.blocks.copy_(torch.from_numpy(host.reshape(-1)))
            base = self.blocks.data_ptr()
            self.tensors = {}
            self.c = moe_qffn(**{k: base + o for k, o in _BLOCK_OFFSETS.items()},
                              expert_stride=EXPERT_BLOCK)
        else:
            raise ValueError(f"unknown layout {layout!r}")

    @property
    def nbytes(self) -> int:
        """Bytes of weights (codes, scales, biases), without block padding."""
        return self._nbytes


class DeviceLayer:
    """One MoE layer resident in device memory, with its C descriptor."""

    def __init__(self, layer, device="cuda", layout: str = "dense"):
        assert (layer.dims.E, layer.dims.topk, layer.dims.H, layer.dims.I, layer.dims.G) == (
            MOE_EXPERTS, MOE_TOPK, MOE_HIDDEN, MOE_INTER, MOE_GROUP), "production shape only"
        self.w_router = torch.from_numpy(np.ascontiguousarray(layer.w_router).view(np.int16)).to(device)
        self.w_shared_gate = torch.from_numpy(
            np.ascontiguousarray(layer.w_shared_gate).view(np.int16)).to(device)
        self.router_bias = (None if layer.router_bias is None else
                            torch.from_numpy(np.ascontiguousarray(layer.router_bias, np.float32)).to(device))
        self.routed = DeviceQFFN(layer.routed, MOE_EXPERTS, device, layout)
        self.shared = DeviceQFFN(layer.shared, 1, device, layout)
        assert tuple(self.w_router.shape) == (MOE_EXPERTS, MOE_HIDDEN)
        assert tuple(self.w_shared_gate.shape) == (MOE_HIDDEN,)
        # the transposed router matrix a chain's previous layer reads
        self.w_router_t = torch.empty((MOE_HIDDEN, MOE_EXPERTS), dtype=torch.int16, device=device)
        moe_router_transpose(self.w_router, self.w_router_t)
        self.c = moe_layer(self.w_router.data_ptr(),
                           None if self.router_bias is None else self.router_bias.data_ptr(),
                           self.w_shared_gate.data_ptr(), self.routed.c, self.shared.c,
                           self.w_router_t.data_ptr())

    @property
    def nbytes(self) -> int:
        return (self.routed.nbytes + self.shared.nbytes + self.w_router.numel() * 2 +
                self.w_shared_gate.numel() * 2)


def workspace(T: int, device="cuda") -> torch.Tensor:
    """Device workspace of moe_workspace_bytes(T) bytes (allocated by torch;
    it needs no preparation)."""
    return torch.empty(max(moe_workspace_bytes(T), 256), dtype=torch.uint8, device=device)


def _ws(ws: torch.Tensor):
    return _ptr(ws, "ws", torch.uint8), ws.numel()


def _route_out(route_out, T: int, nlayers: Optional[int] = None):
    """(ids, w, sg) device tensors -> their pointers, shapes checked."""
    if route_out is None:
        return None, None, None
    ids, w, sg = route_out
    lead = () if nlayers is None else (nlayers,)
    return (_ptr(ids, "route ids", torch.int32, lead + (T, MOE_TOPK)),
            _ptr(w, "route w", torch.float32, lead + (T, MOE_TOPK)),
            _ptr(sg, "route sg", torch.float32, lead + (T,)))


def moe_route(x, w_router, router_bias, w_shared_gate, topk_ids, topk_w, shared_gate, ws,
              stream=None) -> None:
    T = x.shape[0]
    wsp, wsn = _ws(ws)
    _check("moe_route", lib().moe_route(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T,
        _ptr(w_router, "w_router", _U16, (MOE_EXPERTS, MOE_HIDDEN)),
        _ptr(router_bias, "router_bias", torch.float32, (MOE_EXPERTS,)),
        _ptr(w_shared_gate, "w_shared_gate", _U16, (MOE_HIDDEN,)),
        _ptr(topk_ids, "topk_ids", torch.int32, (T, MOE_TOPK)),
        _ptr(topk_w, "topk_w", torch.float32, (T, MOE_TOPK)),
        _ptr(shared_gate, "shared_gate", torch.float32, (T,)), wsp, wsn, _stream(stream)))


def moe_permute(topk_ids, expert_counts, expert_offsets, perm, inv_perm, ws, stream=None) -> None:
    T = topk_ids.shape[0]
    wsp, wsn = _ws(ws)
    _check("moe_permute", lib().moe_permute(
        _ptr(topk_ids, "topk_ids", torch.int32, (T, MOE_TOPK)), T,
        _ptr(expert_counts, "expert_counts", torch.int32, (MOE_EXPERTS,)),
        _ptr(expert_offsets, "expert_offsets", torch.int32, (MOE_EXPERTS + 1,)),
        _ptr(perm, "perm", torch.int32, (T * MOE_TOPK,)),
        _ptr(inv_perm, "inv_perm", torch.int32, (T * MOE_TOPK,)), wsp, wsn, _stream(stream)))


def moe_expert_ffn(x, layer: DeviceLayer, expert_offsets, perm, expert_out, ws,
                   path: int = MOE_PATH_AUTO, stream=None) -> None:
    T = x.shape[0]
    wsp, wsn = _ws(ws)
    opt = moe_options(path)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, C.byref(layer.routed.c), C.byref(layer.shared.c),
        _ptr(expert_offsets, "expert_offsets", torch.int32, (MOE_EXPERTS + 1,)),
        _ptr(perm, "perm", torch.int32, (T * MOE_TOPK,)),
        _ptr(expert_out, "expert_out", torch.float32, ((MOE_TOPK + 1) * T, MOE_HIDDEN)),
        wsp, wsn, _stream(stream), C.byref(opt)))


def moe_combine(expert_out, inv_perm, topk_w, shared_gate, y, stream=None) -> None:
    T = y.shape[0]
    _check("moe_combine", lib().moe_combine(
        _ptr(expert_out, "expert_out", torch.float32, ((MOE_TOPK + 1) * T, MOE_HIDDEN)),
        _ptr(inv_perm, "inv_perm", torch.int32, (T * MOE_TOPK,)),
        _ptr(topk_w, "topk_w", torch.float32, (T, MOE_TOPK)),
        _ptr(shared_gate, "shared_gate", torch.float32, (T,)), T,
        _ptr(y, "y", _U16, (T, MOE_HIDDEN)), _stream(stream)))


def moe_layer_forward_ex(x, layer: DeviceLayer, y, ws, path: int = MOE_PATH_AUTO,
                         residual_out=None, route_out=None, stream=None) -> None:
    """route_out: optional (ids int32 [T,8], w fp32 [T,8], sg fp32 [T]) device
    tensors that receive the routing the call used."""
    T = x.shape[0]
    wsp, wsn = _ws(ws)
    ri, rw, rs = _route_out(route_out, T)
    opt = moe_options(path, _ptr(residual_out, "residual_out", _U16, (T, MOE_HIDDEN)), ri, rw, rs)
    _check("moe_layer_forward_ex", lib().moe_layer_forward_ex(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, C.byref(layer.c),
        _ptr(y, "y", _U16, (T, MOE_HIDDEN)), wsp, wsn, _stream(stream), C.byref(opt)))


def moe_layer_forward_chunked(x, layer: DeviceLayer, y, chunk: int, ws0, ws1,
                              stream=None) -> None:
    """One layer over T tokens in chunks of `chunk`, the next chunk's routing
    overlapping the current chunk's expert GEMMs; ws0 / ws1: two workspaces
    of at least moe_workspace_bytes(chunk) bytes each."""
    T = x.shape[0]
    w0, n0 = _ws(ws0)
    w1, n1 = _ws(ws1)
    _check("moe_layer_forward_chunked", lib().moe_layer_forward_chunked(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, C.byref(layer.c),
        _ptr(y, "y", _U16, (T, MOE_HIDDEN)), int(chunk), w0, w1, min(n0, n1), _stream(stream)))


class LayerChain:
    """A host array of layer descriptors for moe_chain_forward (kept alive
    with the layers it points to)."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.c = (moe_layer * len(self.layers))(*[L.c for L in self.layers])

    def __len__(self):
        return len(self.layers)


def moe_chain_forward(x, chain: LayerChain, x_out, ws, y_layers=None, path: int = MOE_PATH_AUTO,
                      route_out=None, stream=None) -> None:
    """x_out = the residual stream after every layer of the chain;
    y_layers: optional bf16 [nlayers, T, 2048] per-layer outputs; route_out:
    optional (ids [nlayers,T,8], w [nlayers,T,8], sg [nlayers,T])."""
    T, n = x.shape[0], len(chain)
    wsp, wsn = _ws(ws)
    ri, rw, rs = _route_out(route_out, T, n)
    opt = moe_options(path, None, ri, rw, rs)
    _check("moe_chain_forward", lib().moe_chain_forward(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, chain.c, n,
        _ptr(x_out, "x_out", _U16, (T, MOE_HIDDEN)),
        _ptr(y_layers, "y_layers", _U16, (n, T, MOE_HIDDEN)), wsp, wsn, _stream(stream),
        C.byref(opt)))


def moe_layer_forward(x, layer: DeviceLayer, y, ws, stream=None) -> None:
    T = x.shape[0]
    wsp, wsn = _ws(ws)
    _check("moe_layer_forward", lib().moe_layer_forward(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, C.byref(layer.c),
        _ptr(y, "y", _U16, (T, MOE_HIDDEN)), wsp, wsn, _stream(stream)))


def moe_chain_forward_noalloc(x, chain: LayerChain, x_out, y_layers=None,
                              path: int = MOE_PATH_AUTO, route_out=None, stream=None) -> None:
    """moe_chain_forward with the library's own fixed device workspace (no
    allocation in the call; T <= MOE_NOALLOC_T_MAX)."""
    T, n = x.shape[0], len(chain)
    ri, rw, rs = _route_out(route_out, T, n)
    opt = moe_options(path, None, ri, rw, rs)
    _check("moe_chain_forward_noalloc", lib().moe_chain_forward_noalloc(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, chain.c, n,
        _ptr(x_out, "x_out", _U16, (T, MOE_HIDDEN)),
        _ptr(y_layers, "y_layers", _U16, (n, T, MOE_HIDDEN)), _stream(stream), C.byref(opt)))


def moe_lm_head_argmax(x, w_head, token, ws, stream=None) -> None:
    """token[t] = argmax_v x[t] . w_head[v] (ties to the lower v), on the device."""
    T, V = x.shape[0], w_head.shape[0]
    wsp, wsn = _ws(ws)
    _check("moe_lm_head_argmax", lib().moe_lm_head_argmax(
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), T, _ptr(w_head, "w_head", _U16, (V, MOE_HIDDEN)), V,
        _ptr(token, "token", torch.int32, (T,)), wsp, wsn, _stream(stream)))


def moe_embed(token, emb, x, stream=None) -> None:
    """x[t] = emb[token[t]] (zeros for a token outside the table), on the device."""
    T, V = token.shape[0], emb.shape[0]
    _check("moe_embed", lib().moe_embed(
        _ptr(token, "token", torch.int32, (T,)), T, _ptr(emb, "emb", _U16, (V, MOE_HIDDEN)), V,
        _ptr(x, "x", _U16, (T, MOE_HIDDEN)), _stream(stream)))


def moe_router_transpose(w_router, w_router_t, stream=None) -> None:
    _check("moe_router_transpose", lib().moe_router_transpose(
        _ptr(w_router, "w_router", _U16, (MOE_EXPERTS, MOE_HIDDEN)),
        _ptr(w_router_t, "w_router_t", _U16, (MOE_HIDDEN, MOE_EXPERTS)), _stream(stream)))


def moe_probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    n = src.numel() * src.element_size()
    _check("moe_probe_read", lib().moe_probe_read(
        _ptr(src, "src"), n, _ptr(sink, "sink", torch.float32), _stream(stream)))


def moe_probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    _check("moe_probe_copy", lib().moe_probe_copy(
        _ptr(dst, "dst"), _ptr(src, "src"), n, _stream(stream)))


def moe_gdn_workspace_bytes(T: int, hv: int) -> int:
    return int(lib().moe_gdn_workspace_bytes(T, hv))


def gdn_workspace(T: int, hv: int, device="cuda") -> torch.Tensor:
    """Device scratch of moe_gdn_workspace_bytes(T, hv) bytes for moe_gdn_scan."""
    return torch.empty(max(moe_gdn_workspace_bytes(T, hv), 256), dtype=torch.uint8, device=device)


def moe_gdn_scan(q, k, v, g, beta, o, ws, s0=None, s_out=None, stream=None) -> None:
    """Gated delta rule scan of one sequence: q, k bf16 [T, hk, 128], v bf16
    [T, hv, 128], g and beta fp32 [T, hv], s0 / s_out fp32 [hv, 128, 128]
    (optional), o bf16 [T, hv, 128]."""
    T, hk = k.shape[0], k.shape[1]
    hv = v.shape[1]
    D = MOE_GDN_DIM
    _check("moe_gdn_scan", lib().moe_gdn_scan(
        _ptr(q, "q", _U16, (T, hk, D)), _ptr(k, "k", _U16, (T, hk, D)),
        _ptr(v, "v", _U16, (T, hv, D)), _ptr(g, "g", torch.float32, (T, hv)),
        _ptr(beta, "beta", torch.float32, (T, hv)), T, hk, hv,
        _ptr(s0, "s0", torch.float32, (hv, D, D)), _ptr(o, "o", _U16, (T, hv, D)),
        _ptr(s_out, "s_out", torch.float32, (hv, D, D)), *_ws(ws), _stream(stream)))


def to_device_bits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16/fp16 bit patterns (uint16 numpy) -> int16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def bits_to_numpy(t: torch.Tensor) -> np.ndarray:
    """int16/bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
