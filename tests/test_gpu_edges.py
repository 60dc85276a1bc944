"""Edge inputs: activations at the fp16 range limit, on both paths.

The expert kernels carry x and h as fp16.  Inside [2^-14, 65504] the
conversion from bf16 is exact, so a layer whose activations stay in range is
computed as defined; a token whose x or h leaves the range gets a non-finite
output row and the other tokens are unaffected (the routing, computed from
the bf16 x in fp32, is not affected)."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu

SCALE_2M8, BIAS_M7P5_2M8 = 0x1C00, 0xA780      # fp16 2^-8 and -7.5 * 2^-8: w = 2^-9 for code 8


@pytest.fixture(scope="module")
def const_layer():
    L = synth.constant_layer(synth.PROD, 8, SCALE_2M8, BIAS_M7P5_2M8)
    return L, moe.DeviceLayer(L)


def bf16_bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


@pytest.mark.parametrize("path", [moe.MOE_PATH_AUTO, moe.MOE_PATH_PREFILL])
def test_fp16_range_limit(gpu, const_layer, path):
    L, D = const_layer
    T = 4
    x = np.zeros((T, 2048), np.uint16)
    x[0, 5] = bf16_bits(59904.0)                 # largest bf16 below 65504: exact in fp16
    x[1] = synth.make_x(1, seed=3)[0]            # an ordinary token
    x[2, 7] = bf16_bits(65536.0)                 # beyond fp16: that token's row is not finite
    x[3, 100] = bf16_bits(-59904.0)
    xd = moe.to_device_bits(x)
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    moe.moe_layer_forward_ex(xd, D, y, moe.workspace(T), path=path)
    torch.cuda.synchronize()
    g = P.bf16_f64(moe.bits_to_numpy(y))
    keep = np.array([0, 1, 3])
    ref = P.orc().layer_forward(L, np.ascontiguousarray(x[keep]))
    # token 0: g = u = 59904 * 2^-9 = 117, h = bf16(silu(117) * 117) = 13696,
    # d = 13696, y = bf16(1.5 * 13696) = 20480 in every column
    assert np.all(P.bf16_f64(ref.y[0]) == 20480.0)
    P.assert_close(g[keep], P.bf16_f64(ref.y), f"in-range tokens path={path}")
    assert not np.all(np.isfinite(g[2])), "a token beyond the fp16 range must not look finite"
