"""moe_route on the GPU vs the oracle's router (same inputs)."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu


# (33..512 tokens run the router GEMM in 8 K slices, 1024 in 4, 2048 in 2,
# 4096 unsplit)
@pytest.mark.parametrize("T", [1, 8, 16, 32, 33, 100, 129, 512, 1024, 2048, 4096])
def test_route_uniform(gpu, T):
    P.say(f"route T={T} seed=0 layer=0")
    L, D = P.host_layer(0, 0), P.dev_layer(0, 0)
    x = synth.make_x(T, seed=0, layer=T)
    ids, w, sg = P.gpu_route(moe.to_device_bits(x), D)
    ref = P.orc().route(L, x)
    P.check_route(ids, w, sg, ref, f"route T={T}")
    # descending logit order; logits closer than 2^-14 relative (the GPU
    # compares 24-bit logit keys, then the expert index) may come in index
    # order, exact ties always go to the lower index
    lg = ref.logits
    for t in range(T):
        vals = lg[t, ids[t]]
        tol = np.maximum(1e-5, 2.0 ** -14 * np.abs(vals[:-1]))
        assert np.all(np.diff(vals) <= tol)
        eq = np.diff(vals) == 0
        assert np.all(np.diff(ids[t])[eq] > 0), "exact ties must go to the lower index"


@pytest.mark.parametrize("T", [7, 512, 4096])
def test_route_skewed_bias(gpu, T):
    P.say(f"route skewed T={T}")
    L, D = P.host_layer(0, 0, True), P.dev_layer(0, 0, True)
    x = synth.make_x(T, seed=1, layer=3)
    ids, w, sg = P.gpu_route(moe.to_device_bits(x), D)
    P.check_route(ids, w, sg, P.orc().route(L, x), f"route skewed T={T}")


@pytest.mark.parametrize("T", [1, 40])
def test_route_zero_input(gpu, T):
    D = P.dev_layer(0, 0)
    x = torch.zeros((T, 2048), dtype=torch.int16, device="cuda")
    ids, w, sg = P.gpu_route(x, D)
    assert np.all(ids == np.arange(8)) and np.all(w == 0.125) and np.all(sg == 0.5)


def test_route_deterministic(gpu):
    D = P.dev_layer(0, 0)
    x = moe.to_device_bits(synth.make_x(300, seed=2))
    a = P.gpu_route(x, D)
    b = P.gpu_route(x, D)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
