"""moe_permute on the GPU: bit-exact against the oracle's stable counting
sort, for random, skewed and GPU-produced expert ids."""
import numpy as np
import pytest
import torch

import gemv_router_softmax_amd as moe
from gemv_router_softmax_amd import synth
import parity as P

pytestmark = pytest.mark.gpu


def run_perm(ids_np):
    T = ids_np.shape[0]
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).cuda()
    counts = torch.empty(256, dtype=torch.int32, device="cuda")
    offsets = torch.empty(257, dtype=torch.int32, device="cuda")
    perm = torch.empty(8 * T, dtype=torch.int32, device="cuda")
    inv = torch.empty(8 * T, dtype=torch.int32, device="cuda")
    moe.moe_permute(ids, counts, offsets, perm, inv, moe.workspace(T))
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (counts, offsets, perm, inv)]


def random_ids(T, seed, E=256):
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :8].astype(np.int32)


def check(ids_np):
    got = run_perm(ids_np)
    ref = P.orc().permute(synth.PROD, ids_np)
    for name, g, r in zip(("counts", "offsets", "perm", "inv"), got,
                          (ref.counts, ref.offsets, ref.perm, ref.inv)):
        assert np.array_equal(g, r), f"{name} differs at {np.flatnonzero(g != r)[:5]}"


@pytest.mark.parametrize("T", [1, 2, 7, 8, 16, 31, 32, 33, 127, 128, 129, 511, 512, 513, 4096, 4097, 16384, 65536])
def test_permute_random(gpu, T):
    P.say(f"permute random T={T}")
    check(random_ids(T, T))


@pytest.mark.parametrize("T", [64, 4096, 20000])
def test_permute_skewed(gpu, T):
    # every token picks experts 0..7 (hot experts get all T rows), and a Zipf mix
    P.say(f"permute skewed T={T}")
    check(np.tile(np.arange(8, dtype=np.int32), (T, 1)))
    rng = np.random.default_rng(T)
    w = 1.0 / np.arange(1, 257) ** 1.2
    ids = np.stack([rng.choice(256, 8, replace=False, p=w / w.sum()) for _ in range(T)])
    check(ids.astype(np.int32))


def test_permute_gpu_ids(gpu):
    L = P.dev_layer(0, 0)
    x = moe.to_device_bits(synth.make_x(4096, seed=5))
    ids, _, _ = P.gpu_route(x, L)
    check(ids)


def test_permute_deterministic(gpu):
    ids = random_ids(20000, 3)
    a, b = run_perm(ids), run_perm(ids)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_permute_invalid_ids_skipped(gpu):
    ids = random_ids(100, 4)
    ids[3, 2] = 256
    ids[50, 0] = -1
    counts, offsets, perm, inv = run_perm(ids)
    flat = ids.ravel()
    ok = (flat >= 0) & (flat < 256)
    assert inv[3 * 8 + 2] == -1 and inv[50 * 8] == -1
    assert offsets[256] == ok.sum()
    want = np.flatnonzero(ok)[np.argsort(flat[ok], kind="stable")]
    assert np.array_equal(perm[:ok.sum()], want)
    assert np.array_equal(counts, np.bincount(flat[ok], minlength=256))
