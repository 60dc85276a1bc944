"""moe_chain_forward: a chain of distinct layers with residual adds, checked
layer by layer against the oracle on the GPU's own input to each layer."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu

AUTO, DEC, PRE = moe.MOE_PATH_AUTO, moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL


def run_chain(x, nl, path=AUTO, ws=None):
    """Returns x_out, y per layer, (ids, w, sg) per layer (numpy)."""
    T = x.shape[0]
    chain = moe.LayerChain([P.dev_layer(0, l) for l in range(nl)])
    xd = moe.to_device_bits(x)
    xo = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ys = torch.empty((nl, T, 2048), dtype=torch.int16, device="cuda")
    ro = (torch.empty((nl, T, 8), dtype=torch.int32, device="cuda"),
          torch.empty((nl, T, 8), dtype=torch.float32, device="cuda"),
          torch.empty((nl, T), dtype=torch.float32, device="cuda"))
    moe.moe_chain_forward(xd, chain, xo, moe.workspace(T) if ws is None else ws, y_layers=ys,
                          path=path, route_out=ro)
    torch.cuda.synchronize()
    return moe.bits_to_numpy(xo), moe.bits_to_numpy(ys), tuple(t.cpu().numpy() for t in ro)


def check_chain(T, nl, path=AUTO, seed=0):
    P.say(f"chain T={T} layers={nl} path={path}")
    x = synth.make_x(T, seed=seed, step=T)
    xo, ys, (ids, w, sg) = run_chain(x, nl, path)
    o = P.orc()
    xl = x
    for l in range(nl):
        L = P.host_layer(0, l)
        P.check_route(ids[l], w[l], sg[l], o.route(L, xl), f"chain T={T} layer {l} route")
        ref, _ = P.oracle_layer_substituted(L, xl, ids[l])
        P.assert_close(P.bf16_f64(ys[l]), P.bf16_f64(ref.y), f"chain T={T} layer {l} y")
        xl = o.round_bf16(P.bf16_f64(xl) + P.bf16_f64(ys[l]))
    assert np.array_equal(xo, xl), "x_out is not the residual stream of the layers' outputs"


@pytest.mark.parametrize("T,nl", [(1, 4), (2, 3), (5, 3), (8, 3)])
def test_chain_few_token(gpu, T, nl):
    """The fused few-token chain: every layer after the first takes its router
    logits from the previous layer's down kernel."""
    check_chain(T, nl)


@pytest.mark.parametrize("T,nl,path", [(16, 2, DEC), (4, 2, PRE), (100, 2, AUTO)])
def test_chain_other_paths(gpu, T, nl, path):
    check_chain(T, nl, path)


def test_chain_single_layer_equals_layer_call(gpu):
    """A one-layer chain is the layer call: bit-identical y and x_out."""
    for T in (1, 8, 64):
        x = synth.make_x(T, seed=4, step=T)
        xo, ys, _ = run_chain(x, 1)
        y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
        res = torch.empty_like(y)
        moe.moe_layer_forward_ex(moe.to_device_bits(x), P.dev_layer(0, 0), y, moe.workspace(T),
                                 residual_out=res)
        torch.cuda.synchronize()
        assert np.array_equal(ys[0], moe.bits_to_numpy(y)) and np.array_equal(xo, moe.bits_to_numpy(res))


def test_chain_deterministic(gpu):
    """Integer sums make the cross-layer router logits order independent:
    repeated chains are bit-identical, also through a workspace full of
    garbage."""
    x = synth.make_x(3, seed=5, step=9)
    a = run_chain(x, 5)
    ws = torch.full((moe.moe_workspace_bytes(3),), 0x3B, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        b = run_chain(x, 5, ws=ws)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert all(np.array_equal(u, v) for u, v in zip(a[2], b[2]))


def test_chain_graph_replay(gpu):
    """A 6-layer decode chain captured in a HIP graph and replayed several
    times (with eager work in between) matches the eager chain bit for bit."""
    nl = 6
    chain = moe.LayerChain([P.dev_layer(0, l) for l in range(nl)])
    ws = moe.workspace(1)
    x0 = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
    xo = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
    xs = [moe.to_device_bits(synth.make_x(1, seed=0, step=s)) for s in range(4)]
    eager = []
    for s in range(4):
        x0.copy_(xs[s])
        moe.moe_chain_forward(x0, chain, xo, ws)
        eager.append(xo.clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_chain_forward(x0, chain, xo, ws)
    for s in (2, 0, 3, 1):
        x0.copy_(xs[s])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xo, eager[s]), f"replay of step {s} differs from eager"
        y = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
        moe.moe_layer_forward(xs[(s + 1) % 4], P.dev_layer(0, 0), y, ws)
        torch.cuda.synchronize()


def test_router_transpose(gpu):
    """moe_router_transpose is an exact transpose."""
    D = P.dev_layer(0, 0)
    assert torch.equal(D.w_router_t, D.w_router.t().contiguous())


def test_chain_without_transposed_router(gpu):
    """A layer without the transposed router matrix is not fused into the
    layer before it (it runs its own router kernel); the chain stays
    correct and equal to the fully fused chain up to the routing logits'
    summation order."""
    import ctypes as C
    T, nl = 2, 3
    x = synth.make_x(T, seed=6, step=5)
    layers = [P.dev_layer(0, l) for l in range(nl)]
    chain = moe.LayerChain(layers)
    chain.c[1].w_router_t = None
    xd = moe.to_device_bits(x)
    xo = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ys = torch.empty((nl, T, 2048), dtype=torch.int16, device="cuda")
    ro = (torch.empty((nl, T, 8), dtype=torch.int32, device="cuda"),
          torch.empty((nl, T, 8), dtype=torch.float32, device="cuda"),
          torch.empty((nl, T), dtype=torch.float32, device="cuda"))
    moe.moe_chain_forward(xd, chain, xo, moe.workspace(T), y_layers=ys, route_out=ro)
    torch.cuda.synchronize()
    ys, ids = moe.bits_to_numpy(ys), ro[0].cpu().numpy()
    o = P.orc()
    xl = x
    for l in range(nl):
        ref, _ = P.oracle_layer_substituted(P.host_layer(0, l), xl, ids[l])
        P.assert_close(P.bf16_f64(ys[l]), P.bf16_f64(ref.y), f"mixed chain layer {l}")
        xl = o.round_bf16(P.bf16_f64(xl) + P.bf16_f64(ys[l]))
    assert np.array_equal(moe.bits_to_numpy(xo), xl)
