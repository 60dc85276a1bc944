"""moe_layer_forward_chunked: a long prompt through one layer in chunks,
the next chunk's routing and permutation on a second stream while the
current chunk's expert GEMMs run.  The result must equal, bit for bit, the
chunks run one after another on one stream with the grouped-GEMM path, and
match the oracle on sampled tokens of every chunk."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu
PRE = moe.MOE_PATH_PREFILL


def sequential(xd, D, chunk, route=False):
    """The chunks one after another (grouped-GEMM path), one workspace."""
    T = xd.shape[0]
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    sg = torch.empty((T,), dtype=torch.float32, device="cuda")
    ws = moe.workspace(min(chunk, T))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        moe.moe_layer_forward_ex(xd[c0:c1], D, y[c0:c1], ws, path=PRE,
                                 route_out=(ids[c0:c1], w[c0:c1], sg[c0:c1]))
    torch.cuda.synchronize()
    return y, ids


def chunked(xd, D, chunk, fill=None):
    T = xd.shape[0]
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    n = moe.moe_workspace_bytes(chunk)
    ws0 = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws1 = torch.empty(n, dtype=torch.uint8, device="cuda")
    if fill is not None:
        ws0.fill_(fill)
        ws1.fill_(fill ^ 0xFF)
    moe.moe_layer_forward_chunked(xd, D, y, chunk, ws0, ws1)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,chunk,skewed", [
    (1000, 256, False),      # four chunks, the last one ragged (232 tokens)
    (700, 100, True),        # seven chunks
    (300, 1000, False),      # one chunk: the caller's stream alone
    (257, 256, False),       # a one-token last chunk
])
def test_chunked_equals_sequential(gpu, T, chunk, skewed):
    P.say(f"chunked T={T} chunk={chunk} skewed={skewed}")
    D = P.dev_layer(0, 0, skewed)
    xd = moe.to_device_bits(synth.make_x(T, seed=21, layer=T))
    want, _ = sequential(xd, D, chunk)
    got = chunked(xd, D, chunk)
    assert torch.equal(got, want)


def test_chunked_skewed_16384(gpu):
    """The Zipf-biased router over 16384 tokens in four 4096-token chunks:
    bit-identical to the sequential chunks, and the oracle on 12 sampled
    tokens of every chunk."""
    T, C = 16384, 4096
    L, D = P.host_layer(0, 0, True), P.dev_layer(0, 0, True)
    x = synth.make_x(T, seed=13, layer=T)
    xd = moe.to_device_bits(x)
    want, ids = sequential(xd, D, C, route=True)
    got = chunked(xd, D, C, fill=0x3C)
    assert torch.equal(got, want)
    yn = moe.bits_to_numpy(got)
    rng = np.random.default_rng(22)
    rows = np.sort(np.concatenate([c0 + rng.choice(C, 12, replace=False) for c0 in range(0, T, C)]))
    ref, _ = P.oracle_layer_substituted(L, np.ascontiguousarray(x[rows]), ids.cpu().numpy()[rows])
    P.assert_close(P.bf16_f64(yn[rows]), P.bf16_f64(ref.y), "chunked skewed y")


def test_chunked_graph_replay(gpu):
    """The chunked call captured in a HIP graph (the second stream forks from
    and joins the capturing stream) and replayed several times with other
    eager work in between: every replay equals the eager result."""
    T, C = 1000, 256
    D = P.dev_layer(0, 1)
    xs = [moe.to_device_bits(synth.make_x(T, seed=30 + s, layer=T)) for s in range(3)]
    n = moe.moe_workspace_bytes(C)
    ws0 = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws1 = torch.empty(n, dtype=torch.uint8, device="cuda")
    x = torch.empty_like(xs[0])
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    eager = []
    for s in range(3):
        x.copy_(xs[s])
        moe.moe_layer_forward_chunked(x, D, y, C, ws0, ws1)      # (also sets up the stream)
        torch.cuda.synchronize()
        eager.append(y.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_forward_chunked(x, D, y, C, ws0, ws1)
    torch.cuda.synchronize()
    other = torch.empty_like(y)
    for r in range(6):
        s = r % 3
        x.copy_(xs[s])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager[s]), f"replay {r} differs from eager"
        moe.moe_layer_forward(xs[(s + 1) % 3][:64], D, other[:64], moe.workspace(64))
        torch.cuda.synchronize()
