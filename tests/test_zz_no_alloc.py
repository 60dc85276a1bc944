"""moe_chain_forward_noalloc (workspace in the library's fixed device array)
against moe_chain_forward with a caller workspace: bit-identical outputs, on
consecutive calls of decreasing size, eager and graph-captured."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu


def both(x, nl, path=moe.MOE_PATH_AUTO):
    T = x.shape[0]
    chain = moe.LayerChain([P.dev_layer(0, l) for l in range(nl)])
    xd = moe.to_device_bits(x)
    outs = []
    for noalloc in (False, True):
        xo = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
        ys = torch.empty((nl, T, 2048), dtype=torch.int16, device="cuda")
        if noalloc:
            moe.moe_chain_forward_noalloc(xd, chain, xo, y_layers=ys, path=path)
        else:
            moe.moe_chain_forward(xd, chain, xo, moe.workspace(T), y_layers=ys, path=path)
        torch.cuda.synchronize()
        outs.append((moe.bits_to_numpy(xo), moe.bits_to_numpy(ys)))
    return outs


@pytest.mark.parametrize("sizes", [(8, 1), (64, 20), (5, 2)])
def test_noalloc_matches_workspace_call(gpu, sizes):
    """Two calls in a row, the second smaller: each equals the workspace
    call bit for bit (the same kernels on the same layout)."""
    for i, T in enumerate(sizes):
        P.say(f"noalloc T={T} (call {i})")
        x = synth.make_x(T, seed=40 + i, step=T)
        (xa, ya), (xb, yb) = both(x, 3)
        assert np.array_equal(xa, xb) and np.array_equal(ya, yb), f"T={T}"


def test_noalloc_layer_parity(gpu):
    """The no-allocation chain against the oracle, layer by layer."""
    T, nl = 4, 2
    x = synth.make_x(T, seed=44, step=1)
    chain = moe.LayerChain([P.dev_layer(0, l) for l in range(nl)])
    xo = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ys = torch.empty((nl, T, 2048), dtype=torch.int16, device="cuda")
    ids = torch.empty((nl, T, 8), dtype=torch.int32, device="cuda")
    ro = (ids, torch.empty((nl, T, 8), device="cuda"), torch.empty((nl, T), device="cuda"))
    moe.moe_chain_forward_noalloc(moe.to_device_bits(x), chain, xo, y_layers=ys, route_out=ro)
    torch.cuda.synchronize()
    ys, ids = moe.bits_to_numpy(ys), ids.cpu().numpy()
    xl = x
    for l in range(nl):
        ref, _ = P.oracle_layer_substituted(P.host_layer(0, l), xl, ids[l])
        P.assert_close(P.bf16_f64(ys[l]), P.bf16_f64(ref.y), f"noalloc layer {l}")
        xl = P.orc().round_bf16(P.bf16_f64(xl) + P.bf16_f64(ys[l]))
    assert np.array_equal(moe.bits_to_numpy(xo), xl)


def test_noalloc_rejects_large_t(gpu):
    T = moe.MOE_NOALLOC_T_MAX + 1
    chain = moe.LayerChain([P.dev_layer(0, 0)])
    x = torch.zeros((T, 2048), dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_chain_forward_noalloc(x, chain, torch.empty_like(x))
    assert ei.value.status == 1


def test_noalloc_graph_capture(gpu):
    """Captured in a HIP graph (the use it is for), replayed with eager work
    in between: every replay equals the eager call."""
    nl = 3
    chain = moe.LayerChain([P.dev_layer(0, l) for l in range(nl)])
    x0 = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
    xo = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
    xs = [moe.to_device_bits(synth.make_x(1, seed=45, step=s)) for s in range(3)]
    eager = []
    for s in range(3):
        x0.copy_(xs[s])
        moe.moe_chain_forward_noalloc(x0, chain, xo)
        eager.append(xo.clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_chain_forward_noalloc(x0, chain, xo)
    for s in (1, 2, 0):
        x0.copy_(xs[s])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xo, eager[s])
        other = torch.empty((8, 2048), dtype=torch.int16, device="cuda")
        moe.moe_chain_forward_noalloc(moe.to_device_bits(synth.make_x(8, seed=46)), chain, other)
        torch.cuda.synchronize()
