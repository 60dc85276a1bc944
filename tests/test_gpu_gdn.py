"""Gated delta rule scan (moe_gdn_scan) against the fp64 oracle.

The kernel computes in chunks of 64 tokens on fp16 MFMA with fp32
accumulation and an fp32 state; the oracle runs the recurrence token by
token in double.  Tolerances (relative L2 over all outputs / over the final
state, and the largest error against the output scale) follow from fp16
operand rounding (relative 2^-11 per operand, a few chained products per
chunk, errors in the state damped by the decay), see the library's
documentation."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import oracle

pytestmark = pytest.mark.gpu

O_REL, S_REL, O_MAX = 5e-3, 5e-3, 2e-2
# Calls of up to MOE_GDN_STEP_T_MAX tokens run token by token in fp32: o
# then differs from the oracle's bf16 rounding only where fp32 error flips a
# last bit (one bf16 ulp, 2^-8 relative, in a small share of elements), the
# state by fp32 rounding over a few dozen steps.
STEP_O_REL, STEP_S_REL, STEP_O_MAX = 1e-3, 1e-5, 8e-3


def _bf(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(x, s0=True, ws=None):
    T, hk = x.k.shape[0], x.k.shape[1]
    hv = x.v.shape[1]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (moe.to_device_bits(a) for a in (x.q, x.k, x.v))
    g, beta = dev(x.g), dev(x.beta)
    s0d = dev(x.s0) if (s0 and x.s0 is not None) else None
    o = torch.empty((T, hv, 128), dtype=torch.int16, device="cuda")
    s_out = torch.empty((hv, 128, 128), dtype=torch.float32, device="cuda")
    ws = moe.gdn_workspace(T, hv) if ws is None else ws
    moe.moe_gdn_scan(q, k, v, g, beta, o, ws, s0=s0d, s_out=s_out)
    torch.cuda.synchronize()
    return moe.bits_to_numpy(o), s_out.cpu().numpy().astype(np.float64)


def _check(x, s0=True, o_rel=O_REL, s_rel=S_REL, o_max=O_MAX):
    o_bits, st = _run(x, s0)
    ref = oracle.load().gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.s0 if s0 else None)
    got, want = _bf(o_bits), _bf(ref.o_bf16)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    mab = np.abs(got - want).max() / np.abs(want).max()
    srel = np.linalg.norm(st - ref.state) / np.linalg.norm(ref.state)
    print(f"T={x.k.shape[0]} hk={x.k.shape[1]} hv={x.v.shape[1]} o relL2={rel:.2e} "
          f"max/scale={mab:.2e} state relL2={srel:.2e}", flush=True)
    assert np.all(np.isfinite(got))
    assert rel <= o_rel and mab <= o_max and srel <= s_rel
    return rel, srel


@pytest.mark.parametrize("T,hk,hv,s0", [(1, 1, 1, True), (1, 1, 2, False), (63, 1, 2, True),
                                        (64, 2, 2, False), (65, 1, 1, True), (130, 2, 4, True),
                                        (300, 4, 8, False), (517, 2, 4, True)])
def test_gdn_small(T, hk, hv, s0):
    _check(synth.make_gdn(T, hk, hv, seed=T + 7 * hv), s0)


def test_gdn_full_size_t2048():
    """The workload of the scan's benchmark: 2048 tokens, 16 key heads, 32
    value heads, a carried-in state; every output and the final state."""
    _check(synth.make_gdn(2048, synth.GDN_HK, synth.GDN_HV, seed=1))


def test_gdn_longest_sequence():
    """MOE_T_MAX tokens (1024 chunk steps) with two value heads over one key
    head: every output and the final state."""
    _check(synth.make_gdn(65536, 1, 2, seed=11))


def test_gdn_most_heads():
    """MOE_GDN_HEADS_MAX value heads over 8 key heads."""
    _check(synth.make_gdn(100, 8, 64, seed=13))


@pytest.mark.parametrize("regime", ["strong_decay", "no_decay"])
def test_gdn_decay_extremes(regime):
    """Strong decay (about e^-1 per token: within a chunk the old state and
    early tokens fall below fp16's range in the scaled operands) and none at
    all (g = 0: nothing is forgotten, the state only changes by the delta
    writes)."""
    x = synth.make_gdn(300, 2, 4, seed=17)
    rng = np.random.default_rng(17)
    if regime == "strong_decay":
        g = (-rng.uniform(0.5, 1.5, x.g.shape)).astype(np.float32)
    else:
        g = np.zeros_like(x.g)
    _check(synth.GdnInputs(x.q, x.k, x.v, g, x.beta, x.s0))


def test_gdn_t0_passes_state():
    x = synth.make_gdn(1, 1, 2, seed=3)
    s0 = torch.from_numpy(x.s0).cuda()
    s_out = torch.full((2, 128, 128), 7.0, dtype=torch.float32, device="cuda")
    z = torch.empty((0, 1, 128), dtype=torch.int16, device="cuda")
    zv = torch.empty((0, 2, 128), dtype=torch.int16, device="cuda")
    zg = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    ws = moe.gdn_workspace(0, 2)
    moe.moe_gdn_scan(z, z, zv, zg, zg, zv, ws, s0=s0, s_out=s_out)
    torch.cuda.synchronize()
    assert np.array_equal(s_out.cpu().numpy(), x.s0)
    moe.moe_gdn_scan(z, z, zv, zg, zg, zv, ws, s0=None, s_out=s_out)
    torch.cuda.synchronize()
    assert not s_out.cpu().numpy().any()


def test_gdn_deterministic_and_workspace_garbage():
    x = synth.make_gdn(200, 2, 4, seed=5)
    ws = moe.gdn_workspace(200, 4)
    ws.fill_(0xA5)
    a = _run(x, ws=ws)
    ws.fill_(0x3C)
    b = _run(x, ws=ws)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gdn_split_matches_oracle():
    """Two calls with the state carried between them (the split falls inside
    a chunk) agree with the oracle's single scan."""
    x = synth.make_gdn(300, 2, 4, seed=9)
    T1 = 137
    first = synth.GdnInputs(x.q[:T1], x.k[:T1], x.v[:T1], x.g[:T1], x.beta[:T1], x.s0)
    o1, st1 = _run(first)
    second = synth.GdnInputs(x.q[T1:], x.k[T1:], x.v[T1:], x.g[T1:], x.beta[T1:],
                             st1.astype(np.float32))
    o2, st2 = _run(second)
    ref = oracle.load().gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.s0)
    got = _bf(np.concatenate([o1, o2]))
    want = _bf(ref.o_bf16)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= O_REL
    assert np.linalg.norm(st2 - ref.state) / np.linalg.norm(ref.state) <= S_REL


@pytest.mark.parametrize("T,hk,hv", [(2, 1, 2), (7, 2, 4), (32, 4, 8), (48, 16, 32)])
def test_gdn_step_path(T, hk, hv):
    """Calls of up to MOE_GDN_STEP_T_MAX tokens (the token-by-token fp32
    kernel) against the oracle, at the tighter fp32 tolerances."""
    assert T <= moe.MOE_GDN_STEP_T_MAX
    _check(synth.make_gdn(T, hk, hv, seed=40 + T), o_rel=STEP_O_REL, s_rel=STEP_S_REL,
           o_max=STEP_O_MAX)


def _call(x, t0, t1, st, o=None):
    """Tokens t0 .. t1 - 1 of x with the state st updated in place."""
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (moe.to_device_bits(a[t0:t1]) for a in (x.q, x.k, x.v))
    g, beta = dev(x.g[t0:t1]), dev(x.beta[t0:t1])
    o = torch.empty((t1 - t0, x.v.shape[1], 128), dtype=torch.int16, device="cuda")
    moe.moe_gdn_scan(q, k, v, g, beta, o, moe.gdn_workspace(t1 - t0, x.v.shape[1]), s0=st, s_out=st)
    return o


def test_gdn_decode_loop_in_place():
    """Twenty single-token calls (decode), the state updated in place
    (s_out = s0), agree with the oracle's scan of the twenty tokens."""
    x = synth.make_gdn(20, 2, 4, seed=21)
    st = torch.from_numpy(x.s0.copy()).cuda()
    outs = [_call(x, t, t + 1, st) for t in range(20)]
    torch.cuda.synchronize()
    ref = oracle.load().gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.s0)
    got = _bf(np.concatenate([moe.bits_to_numpy(o) for o in outs]))
    want = _bf(ref.o_bf16)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    srel = np.linalg.norm(st.cpu().numpy() - ref.state) / np.linalg.norm(ref.state)
    print(f"decode loop: o relL2={rel:.2e} state relL2={srel:.2e}", flush=True)
    assert rel <= STEP_O_REL and srel <= STEP_S_REL


def test_gdn_split_across_paths_in_place():
    """Calls of 1, 5, 64, 30 and 200 tokens (three token by token, two
    chunked), the state updated in place between them, agree with the
    oracle's single scan."""
    x = synth.make_gdn(300, 2, 4, seed=23)
    st = torch.from_numpy(x.s0.copy()).cuda()
    bounds = [0, 1, 6, 70, 100, 300]
    outs = [_call(x, a, b, st) for a, b in zip(bounds, bounds[1:])]
    torch.cuda.synchronize()
    ref = oracle.load().gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.s0)
    got = _bf(np.concatenate([moe.bits_to_numpy(o) for o in outs]))
    want = _bf(ref.o_bf16)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    srel = np.linalg.norm(st.cpu().numpy() - ref.state) / np.linalg.norm(ref.state)
    print(f"split across paths: o relL2={rel:.2e} state relL2={srel:.2e}", flush=True)
    assert rel <= O_REL and srel <= S_REL


def test_gdn_step_state_4_byte_aligned():
    """The state arrays need only be 4-byte aligned: a state one float off a
    16-byte boundary (the token-by-token kernel's per-element path) gives
    exactly what the 16-byte-aligned state gives."""
    x = synth.make_gdn(3, 1, 2, seed=31)
    n = x.s0.size
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (moe.to_device_bits(a) for a in (x.q, x.k, x.v))
    g, beta = dev(x.g), dev(x.beta)
    ws = moe.gdn_workspace(3, 2)
    outs = []
    for off in (0, 1):
        buf = torch.zeros(2 * n + 8, dtype=torch.float32, device="cuda")
        s0 = buf[off:off + n].view(x.s0.shape)
        s0.copy_(dev(x.s0))
        s_out = buf[n + 4 + off:n + 4 + off + n].view(x.s0.shape)
        assert (s0.data_ptr() % 16 == 0) == (off == 0)
        o = torch.empty((3, 2, 128), dtype=torch.int16, device="cuda")
        moe.moe_gdn_scan(q, k, v, g, beta, o, ws, s0=s0, s_out=s_out)
        torch.cuda.synchronize()
        outs.append((moe.bits_to_numpy(o), s_out.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    ref = oracle.load().gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.s0)
    srel = np.linalg.norm(outs[1][1] - ref.state) / np.linalg.norm(ref.state)
    assert srel <= STEP_S_REL
