"""moe_layer_forward (whole layer, one stream, no host sync) vs the oracle."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu

AUTO, DEC, PRE = moe.MOE_PATH_AUTO, moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL


def gpu_layer(x, D, path=AUTO, residual=False):
    """One layer call; returns y, the residual output (or None), x on the
    device and the routing the call itself used (ids, w, sg)."""
    T = x.shape[0]
    xd = moe.to_device_bits(x)
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    res = torch.empty_like(y) if residual else None
    ro = (torch.empty((T, 8), dtype=torch.int32, device="cuda"),
          torch.empty((T, 8), dtype=torch.float32, device="cuda"),
          torch.empty((T,), dtype=torch.float32, device="cuda"))
    moe.moe_layer_forward_ex(xd, D, y, moe.workspace(T), path=path, residual_out=res, route_out=ro)
    torch.cuda.synchronize()
    route = tuple(t.cpu().numpy() for t in ro)
    return moe.bits_to_numpy(y), (moe.bits_to_numpy(res) if residual else None), xd, route


def check_layer(T, path, seed=0, skewed=False, sample=None):
    """The layer's y against the oracle on the same input; the oracle takes
    the GPU call's own expert set on (near-tie) tokens where they differ, and
    the call's routing is checked against the oracle's as well."""
    P.say(f"layer T={T} path={path} seed={seed} skewed={skewed}")
    L, D = P.host_layer(0, 0, skewed), P.dev_layer(0, 0, skewed)
    x = synth.make_x(T, seed=seed) if seed == 0 else synth.make_x(T, seed=seed, layer=T)
    y, _, xd, (ids, w, sg) = gpu_layer(x, D, path)
    rows = np.arange(T) if sample is None else sample
    xs = np.ascontiguousarray(x[rows])
    P.check_route(ids[rows], w[rows], sg[rows], P.orc().route(L, xs), f"route of the layer call T={T}")
    ref, diff = P.oracle_layer_substituted(L, xs, ids[rows])
    P.assert_close(P.bf16_f64(y[rows]), P.bf16_f64(ref.y), f"y T={T} path={path}")
    return y


def test_config0_t16_decode(gpu):
    check_layer(16, DEC)


def test_config0_t16_prefill(gpu):
    check_layer(16, PRE)


@pytest.mark.parametrize("T", [1, 2, 8])
def test_decode_auto(gpu, T):
    check_layer(T, AUTO, seed=3)


@pytest.mark.parametrize("T", [9, 64, 100, 129, 512, 513, 896, 897])
def test_prefill_auto(gpu, T):
    check_layer(T, AUTO, seed=4)


@pytest.mark.parametrize("skewed", [False, True])
def test_full_size_t4096(gpu, skewed):
    """The headline prefill size, every token of the [4096, 2048] output."""
    check_layer(4096, AUTO, seed=5, skewed=skewed)


@pytest.mark.parametrize("T", [256, 1024, 2048])
def test_prefill_sweep_sizes(gpu, T):
    """The other sizes of the prefill sweep, every token."""
    check_layer(T, AUTO, seed=16)


def test_residual_output(gpu):
    D = P.dev_layer(0, 0)
    x = synth.make_x(8, seed=6)
    y, res, _, _ = gpu_layer(x, D, residual=True)
    want = P.orc().round_bf16(P.bf16_f64(x) + P.bf16_f64(y))
    assert np.array_equal(res, want)


def test_layer_deterministic(gpu):
    D = P.dev_layer(0, 0)
    for T in (1, 700):
        x = synth.make_x(T, seed=7)
        a = gpu_layer(x, D)[0]
        b = gpu_layer(x, D)[0]
        assert np.array_equal(a, b)


def test_t0_is_noop(gpu):
    D = P.dev_layer(0, 0)
    x = torch.zeros((0, 2048), dtype=torch.int16, device="cuda")
    y = torch.zeros((0, 2048), dtype=torch.int16, device="cuda")
    moe.moe_layer_forward(x, D, y, moe.workspace(0))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [17, 32])
def test_decode_forced_max(gpu, T):
    check_layer(T, DEC, seed=8)


def test_graph_capture_chain(gpu):
    """A 3-layer decode chain captured in a HIP graph and replayed several
    times, with eager work in between, matches the eager chain bit for bit."""
    D = [P.dev_layer(0, l) for l in range(3)]
    ws = moe.workspace(1)
    x0 = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
    bufs = [torch.empty((1, 2048), dtype=torch.int16, device="cuda") for _ in range(2)]
    y = torch.empty((1, 2048), dtype=torch.int16, device="cuda")

    def chain():
        cur = x0
        for l, Dl in enumerate(D):
            moe.moe_layer_forward_ex(cur, Dl, y, ws, residual_out=bufs[l % 2])
            cur = bufs[l % 2]
        return cur

    xs = [moe.to_device_bits(synth.make_x(1, seed=0, step=s)) for s in range(4)]
    eager = []
    for s in range(4):
        x0.copy_(xs[s])
        eager.append(chain().clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = chain()
    for s in range(4):
        x0.copy_(xs[s])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[s]), f"replay {s} differs from eager"
        # unrelated eager work between replays
        moe.moe_layer_forward(xs[(s + 1) % 4], D[0], y, ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [4, 300])
def test_workspace_garbage(gpu, T):
    """The workspace is scratch: one full of garbage gives the same result as a
    fresh one, on each of several calls."""
    D = P.dev_layer(0, 0)
    x = moe.to_device_bits(synth.make_x(T, seed=9))
    want = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    moe.moe_layer_forward(x, D, want, moe.workspace(T))
    ws = torch.full((moe.moe_workspace_bytes(T),), 0xA7, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        y = torch.empty_like(want)
        moe.moe_layer_forward(x, D, y, ws)
        torch.cuda.synchronize()
        assert torch.equal(y, want)
        ws.fill_(0x5C)


@pytest.mark.parametrize("T,path", [(1, AUTO), (8, AUTO), (20, DEC), (100, AUTO), (16, PRE)])
def test_dense_and_expert_layouts_agree(gpu, T, path):
    """The same weights in the dense layout (expert_stride 0) and in the
    expert-major 2 MiB blocks give bit-identical outputs on every path."""
    P.say(f"layouts T={T} path={path}")
    L = P.host_layer(0, 0)
    dense = P.dev_layer(0, 0)
    assert dense.routed.c.expert_stride == 0
    blocked = moe.DeviceLayer(L, layout="expert")
    assert blocked.routed.c.expert_stride == moe.EXPERT_BLOCK
    assert blocked.routed.c.gate_q % moe.EXPERT_BLOCK == 0
    x = synth.make_x(T, seed=9)
    y0 = gpu_layer(x, dense, path)[0]
    y1 = gpu_layer(x, blocked, path)[0]
    assert np.array_equal(y0, y1)


def test_max_t_sampled(gpu):
    """The largest T the library accepts (MOE_T_MAX = 65536 tokens), checked
    against the oracle on sampled tokens (routing is per token, so any subset
    of tokens is a valid oracle input)."""
    rng = np.random.default_rng(11)
    T = moe.MOE_T_MAX
    check_layer(T, AUTO, seed=12, sample=np.sort(rng.choice(T, 32, replace=False)))


@pytest.mark.parametrize("T,nl", [(1, 3), (512, 2)])
def test_chain_layer_by_layer(gpu, T, nl):
    """A chain of distinct layers with residual adds (the decode and the
    T = 512 prefill workloads): every layer's output matches the oracle run
    on the GPU's own input to that layer, and the residual output is exactly
    bf16(x + y)."""
    xd = moe.to_device_bits(synth.make_x(T, seed=0, step=3))
    for l in range(nl):
        P.say(f"chain T={T} layer {l}")
        L, D = P.host_layer(0, l), P.dev_layer(0, l)
        x = moe.bits_to_numpy(xd)
        y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
        res = torch.empty_like(y)
        ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
        ro = (ids, torch.empty((T, 8), device="cuda"), torch.empty((T,), device="cuda"))
        moe.moe_layer_forward_ex(xd, D, y, moe.workspace(T), residual_out=res, route_out=ro)
        torch.cuda.synchronize()
        yn = moe.bits_to_numpy(y)
        ref, _ = P.oracle_layer_substituted(L, x, ids.cpu().numpy())
        P.assert_close(P.bf16_f64(yn), P.bf16_f64(ref.y), f"chain T={T} layer {l}")
        want = P.orc().round_bf16(P.bf16_f64(x) + P.bf16_f64(yn))
        assert np.array_equal(moe.bits_to_numpy(res), want)
        xd = res


def test_skewed_chunked_sampled(gpu):
    """The Zipf-biased router over 16384 tokens in four 4096-token chunks
    sharing one workspace, checked on sampled tokens of every chunk."""
    T, C = 16384, 4096
    L, D = P.host_layer(0, 0, True), P.dev_layer(0, 0, True)
    x = synth.make_x(T, seed=13, layer=T)
    xd = moe.to_device_bits(x)
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    sg = torch.empty((T,), dtype=torch.float32, device="cuda")
    ws = moe.workspace(C)
    for c0 in range(0, T, C):
        c1 = c0 + C
        moe.moe_layer_forward_ex(xd[c0:c1], D, y[c0:c1], ws, route_out=(ids[c0:c1], w[c0:c1], sg[c0:c1]))
    torch.cuda.synchronize()
    yn = moe.bits_to_numpy(y)
    rng = np.random.default_rng(14)
    rows = np.sort(np.concatenate([c0 + rng.choice(C, 12, replace=False) for c0 in range(0, T, C)]))
    ids = ids.cpu().numpy()
    ref, _ = P.oracle_layer_substituted(L, np.ascontiguousarray(x[rows]), ids[rows])
    P.assert_close(P.bf16_f64(yn[rows]), P.bf16_f64(ref.y), "skewed chunked y")


