"""moe_expert_ffn and moe_combine on the GPU vs the oracle, with identical
inputs on both sides (the oracle's permutation of the same ids)."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu

DEC, PRE = moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL


def routed_inputs(T, seed, skewed=False):
    L = P.host_layer(0, 0, skewed)
    x = synth.make_x(T, seed=seed, layer=11)
    r = P.orc().route(L, x)
    pm = P.orc().permute(synth.PROD, r.ids)
    return L, x, r, pm


def gpu_ffn(x, D, pm, T, path):
    out = torch.empty(((8 + 1) * T, 2048), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(moe.to_device_bits(x), D, torch.from_numpy(pm.offsets).cuda(),
                       torch.from_numpy(pm.perm).cuda(), out, moe.workspace(T), path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,path", [(1, DEC), (8, DEC), (16, DEC), (16, PRE), (32, DEC),
                                    (1, PRE), (64, PRE), (200, PRE), (512, PRE), (513, PRE),
                                    (896, PRE), (897, PRE)])
def test_expert_ffn(gpu, T, path):
    P.say(f"expert_ffn T={T} path={path}")
    L, x, r, pm = routed_inputs(T, seed=T)
    got = gpu_ffn(x, P.dev_layer(0, 0), pm, T, path)
    ref = P.orc().expert_ffn(L, x, pm.offsets, pm.perm)
    P.assert_close(got, ref, f"expert_out T={T} path={path}")


@pytest.mark.parametrize("T,skewed", [(4096, False), (4096, True)])
def test_expert_ffn_full_size_sampled(gpu, T, skewed):
    """Full-size prefill launch; the oracle recomputes a sample of rows."""
    P.say(f"expert_ffn sampled T={T} skewed={skewed}")
    L, x, r, pm = routed_inputs(T, seed=7, skewed=skewed)
    got = gpu_ffn(x, P.dev_layer(0, 0, skewed), pm, T, PRE)
    rng = np.random.default_rng(T)
    rows = np.unique(np.concatenate([rng.choice(9 * T, 96, replace=False),
                                     [0, 8 * T - 1, 8 * T, 9 * T - 1]])).astype(np.int32)
    ref = P.orc().expert_ffn(L, x, pm.offsets, pm.perm, rows=rows)
    P.assert_close(got[rows], ref, f"expert_out sampled T={T}")


def test_paths_agree_at_16(gpu):
    L, x, r, pm = routed_inputs(16, seed=99)
    D = P.dev_layer(0, 0)
    a = gpu_ffn(x, D, pm, 16, DEC)
    b = gpu_ffn(x, D, pm, 16, PRE)
    P.assert_close(b, a, "prefill vs decode at T=16")


@pytest.mark.parametrize("T", [1, 5, 16, 300])
def test_combine_within_rounding(gpu, T):
    """Identical fp32 inputs.  The GPU sums nine fp32 products in fp32, the
    oracle in float64; each GPU output must be the bf16 rounding of a value
    within the fp32 summation bound (16 * 2^-24 * sum |terms|) of the exact
    sum, i.e. |y_gpu - y_exact| <= bound + half a bf16 ulp; away from
    cancellation that is at most one bf16 ulp."""
    P.say(f"combine T={T}")
    rng = np.random.default_rng(T)
    ids = np.argsort(rng.random((T, 256)), axis=1)[:, :8].astype(np.int32)
    pm = P.orc().permute(synth.PROD, ids)
    out = (rng.standard_normal((9 * T, 2048)) * 0.2).astype(np.float32)
    w = rng.random((T, 8)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    sg = rng.random(T).astype(np.float32)
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    moe.moe_combine(torch.from_numpy(out).cuda(), torch.from_numpy(pm.inv).cuda(),
                    torch.from_numpy(w).cuda(), torch.from_numpy(sg).cuda(), y)
    torch.cuda.synchronize()
    got = moe.bits_to_numpy(y)
    o64 = out.astype(np.float64)
    ref, y32 = P.orc().combine(synth.PROD, o64, pm.inv, w.astype(np.float64),
                               sg.astype(np.float64))
    terms = np.abs(w.astype(np.float64)[:, :, None] * o64[pm.inv.reshape(T, 8)]).sum(1)
    terms += np.abs(sg.astype(np.float64)[:, None] * o64[8 * T:])
    bound = 16 * 2.0 ** -24 * terms
    g = P.bf16_f64(got)
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(g), np.abs(y32)) + 1e-300)) - 8)
    assert np.all(np.abs(g - y32) <= bound + half_ulp), "combine outside the rounding bound"
    same = np.mean(got == ref)
    P.say(f"  combine T={T}: identical to the oracle's bf16 on {same:.5f} of outputs")
    assert same > 0.999


def test_expert_ffn_max_t_split(gpu):
    """The split FFN at the largest T (65536 tokens, the grouped-GEMM path):
    its fp32 output is 4.83e9 bytes, beyond a 32-bit range, so rows past 2^32
    bytes -- the shared-expert rows 8T .. 9T-1 among them -- must land where
    they belong.  Seeded random routing (any routing is a valid input here);
    sampled rows against the oracle, including the first and last routed and
    shared rows."""
    T = moe.MOE_T_MAX
    P.say(f"expert_ffn split T={T}")
    L = P.host_layer(0, 0)
    rng = np.random.default_rng(65536)
    ids = np.argsort(rng.random((T, 256), dtype=np.float32), axis=1)[:, :8].astype(np.int32)
    pm = P.orc().permute(synth.PROD, ids)
    x = synth.make_x(T, seed=17, layer=5)
    D = P.dev_layer(0, 0)
    out = torch.empty(((8 + 1) * T, 2048), dtype=torch.float32, device="cuda")
    out.fill_(float("nan"))
    moe.moe_expert_ffn(moe.to_device_bits(x), D, torch.from_numpy(pm.offsets).cuda(),
                       torch.from_numpy(pm.perm).cuda(), out, moe.workspace(T), path=PRE)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(9 * T, 60, replace=False),
                                     [0, 1, 8 * T - 1, 8 * T, 8 * T + 1, 9 * T - 1]])).astype(np.int32)
    got = out[torch.from_numpy(rows.astype(np.int64)).cuda()].cpu().numpy().astype(np.float64)
    del out
    assert np.all(np.isfinite(got)), "a sampled row was never written"
    ref = P.orc().expert_ffn(L, x, pm.offsets, pm.perm, rows=rows)
    P.assert_close(got, ref, f"expert_out sampled T={T}")
