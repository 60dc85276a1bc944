"""Exact logit ties on the GPU: equal logits must go to the lower expert
index (the oracle's rule, pinned on the CPU by pin_topk_ties).

Duplicated router rows give bit-identical logits on both sides, so here the
selected sets must agree EXACTLY (no near-tie allowance).  The ties are
placed across the 8th/9th rank of token 0, once with the copy above the
original index and once below it, and checked through every routing path:
the small-T router GEMV, the fused MFMA router (T > 32) and the decode
layer, whose routing runs inside the gate/up kernel (checked through the
layer output, since the tied experts have different FFN weights)."""
import copy

import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu


def _tie_layer(below: bool):
    L = copy.deepcopy(P.host_layer(0, 0))
    x = synth.make_x(40, seed=5, layer=77)
    lg = P.orc().route(L, x).logits[0]
    order = np.argsort(-lg, kind="stable")
    e8 = int(order[7])
    # a non-selected expert on the wanted side of e8 becomes its exact copy
    pool = [int(e) for e in order[8:] if (e < e8 if below else e > e8)]
    twin = pool[0]
    L.w_router[twin] = L.w_router[e8]
    return L, x, e8, twin


@pytest.mark.parametrize("below", [False, True])
@pytest.mark.parametrize("T", [1, 8, 40])
def test_route_exact_ties(gpu, T, below):
    L, x, e8, twin = _tie_layer(below)
    x = x[:T]
    D = moe.DeviceLayer(L)
    ids, w, sg = P.gpu_route(moe.to_device_bits(x), D)
    ref = P.orc().route(L, x)
    P.say(f"ties T={T} below={below}: e8={e8} twin={twin} token0 gpu={ids[0].tolist()}")
    low, high = min(e8, twin), max(e8, twin)
    assert low in ids[0] and high not in ids[0]
    for t in range(T):
        assert set(ids[t].tolist()) == set(ref.ids[t].tolist()), f"token {t}"
        assert list(ids[t]) == list(ref.ids[t]), f"order of token {t}"


@pytest.mark.parametrize("below", [False, True])
@pytest.mark.parametrize("T", [1, 8])
def test_decode_layer_exact_ties(gpu, T, below):
    L, x, e8, twin = _tie_layer(below)
    x = x[:T]
    D = moe.DeviceLayer(L)
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    moe.moe_layer_forward_ex(moe.to_device_bits(x), D, y, moe.workspace(T), path=moe.MOE_PATH_DECODE)
    torch.cuda.synchronize()
    got = P.bf16_f64(y.cpu().numpy().view(np.uint16))
    ref = P.bf16_f64(P.orc().layer_forward(L, x).y)
    P.assert_close(got, ref, f"decode layer with exact ties T={T} below={below}")
