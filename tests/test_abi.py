"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol the header declares, sizes its workspace monotonically and rejects
bad arguments on the host (returning before anything is enqueued).

Every call below is built to FAIL validation (or be a T == 0 no-op): the
fake addresses are never handed to a kernel, so these tests are safe on a
machine with a GPU too."""
import ctypes as C
import os
import re

import pytest

import gemv_router_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, ALIGN, WS = 0, 1, 2, 3
A = 0x100000          # fake, 16-byte aligned "device" address (never dereferenced)
MIS = 0x100004        # fake misaligned address


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(moe_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) == 18, names
    assert sorted(moe.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_header_constants_match_binding():
    src = open(HEADER).read()
    for name in ("MOE_HIDDEN", "MOE_INTER", "MOE_EXPERTS", "MOE_TOPK", "MOE_GROUP", "MOE_T_MAX",
                 "MOE_DECODE_T", "MOE_DECODE_T_MAX", "MOE_NOALLOC_T_MAX", "MOE_NOALLOC_WS_BYTES",
                 "MOE_GDN_DIM", "MOE_GDN_CHUNK", "MOE_GDN_STEP_T_MAX", "MOE_GDN_HEADS_MAX"):
        m = re.search(rf"#define {name} (\d+)", src)
        assert int(m.group(1)) == getattr(moe, name), name


def test_workspace_bytes(L):
    assert moe.moe_workspace_bytes(-1) == 0
    assert moe.moe_workspace_bytes(moe.MOE_T_MAX + 1) == 0
    prev = 0
    for T in [0, 1, 2, 7, 8, 9, 16, 63, 64, 512, 4095, 4096, 4097, 16384, 65536]:
        b = moe.moe_workspace_bytes(T)
        assert b >= prev and b % 256 == 0
        prev = b
    # the split outputs fit: [9T][2048] fp32 scratch is part of it
    assert moe.moe_workspace_bytes(4096) >= 9 * 4096 * 2048 * 4


def test_status_strings():
    assert moe.moe_status_string(0) == "MOE_OK"
    assert moe.moe_status_string(3) == "MOE_ERR_WORKSPACE"
    assert moe.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def _qffn(p=A):
    return moe.moe_qffn(*([p] * 9))


def _layer(p=A):
    return moe.moe_layer(p, None, p, _qffn(p), _qffn(p), None)


def test_route_validation(L):
    big = moe.moe_workspace_bytes(4)
    f = L.moe_route
    assert f(A, -1, A, None, A, A, A, A, A, big, None) == INVALID
    assert f(A, moe.MOE_T_MAX + 1, A, None, A, A, A, A, A, big, None) == INVALID
    assert f(None, 0, None, None, None, None, None, None, None, 0, None) == OK
    assert f(None, 4, A, None, A, A, A, A, A, big, None) == INVALID
    assert f(A, 4, A, None, None, A, A, A, A, big, None) == INVALID
    assert f(MIS, 4, A, None, A, A, A, A, A, big, None) == ALIGN
    assert f(A, 4, A, MIS + 1, A, A, A, A, A, big, None) == ALIGN
    assert f(A, 4, A, None, A, A, A, A, A, big - 1, None) == WS


def test_permute_validation(L):
    big = moe.moe_workspace_bytes(100)
    f = L.moe_permute
    assert f(A, 0, None, None, None, None, None, 0, None) == OK
    assert f(A, 100, A, None, A, A, A, big, None) == INVALID
    assert f(A, 100, A, A, A, A + 2, A, big, None) == ALIGN
    assert f(A, 100, A, A, A, A, A, 16, None) == WS


def test_expert_ffn_validation(L):
    big = moe.moe_workspace_bytes(16)
    f = L.moe_expert_ffn
    q = _qffn()
    assert f(A, 16, None, C.byref(q), A, A, A, A, big, None, None) == INVALID
    bad = _qffn()
    bad.down_b = None
    assert f(A, 16, C.byref(bad), C.byref(q), A, A, A, A, big, None, None) == INVALID
    mis = _qffn()
    mis.up_s = MIS
    assert f(A, 16, C.byref(q), C.byref(mis), A, A, A, A, big, None, None) == ALIGN
    assert f(A, 16, C.byref(q), C.byref(q), A, A, A, A, big - 256, None, None) == WS
    # expert_stride: 0 (dense) or a 256-byte multiple of at least one code matrix
    for st in (-256, 256, (1 << 19) - 256, (1 << 19) + 16, 1 << 32):
        bs = _qffn()
        bs.expert_stride = st
        assert f(A, 16, C.byref(bs), C.byref(q), A, A, A, A, big, None, None) == INVALID, st
    # forcing the decode path above its limit, or an unknown path
    opt = moe.moe_options(moe.MOE_PATH_DECODE, None)
    assert f(A, moe.MOE_DECODE_T_MAX + 1, C.byref(q), C.byref(q), A, A, A, A, 1 << 40, None,
             C.byref(opt)) == INVALID
    opt = moe.moe_options(7, None)
    assert f(A, 16, C.byref(q), C.byref(q), A, A, A, A, big, None, C.byref(opt)) == INVALID


def test_combine_validation(L):
    f = L.moe_combine
    assert f(None, None, None, None, 0, None, None) == OK
    assert f(A, A, A, None, 3, A, None) == INVALID
    assert f(A, A, A, A, 3, MIS, None) == ALIGN


def test_layer_forward_validation(L):
    big = moe.moe_workspace_bytes(64)
    f = L.moe_layer_forward_ex
    lay = _layer()
    assert f(A, 0, None, None, None, 0, None, None) == OK
    assert f(A, 64, None, A, A, big, None, None) == INVALID
    assert f(A, -3, C.byref(lay), A, A, big, None, None) == INVALID
    assert f(A, 64, C.byref(lay), A, A, big - 1, None, None) == WS
    assert f(A, 64, C.byref(lay), MIS, A, big, None, None) == ALIGN
    opt = moe.moe_options(moe.MOE_PATH_PREFILL, MIS)
    assert f(A, 64, C.byref(lay), A, A, big, None, C.byref(opt)) == ALIGN
    # route outputs: all three or none, 4-byte aligned
    for ids, w, sg, want in [(A, None, None, INVALID), (A, A, None, INVALID),
                             (A, A, A + 2, ALIGN)]:
        opt = moe.moe_options(moe.MOE_PATH_AUTO, None, ids, w, sg)
        assert f(A, 64, C.byref(lay), A, A, big, None, C.byref(opt)) == want, (ids, w, sg)
    lb = _layer()
    lb.router_bias = A + 2
    assert f(A, 64, C.byref(lb), A, A, big, None, None) == ALIGN
    lz = _layer()
    lz.w_router = None
    assert L.moe_layer_forward(A, 64, C.byref(lz), A, A, big, None) == INVALID
    lt = _layer()
    lt.w_router_t = MIS
    assert f(A, 64, C.byref(lt), A, A, big, None, None) == ALIGN


def test_chunked_validation(L):
    big = moe.moe_workspace_bytes(256)
    f = L.moe_layer_forward_chunked
    lay = _layer()
    B = A + (1 << 30)             # a second fake workspace far from the first
    assert f(A, 0, C.byref(lay), A, 256, A, B, big, None) == OK          # T = 0: no-op
    assert f(A, 1000, C.byref(lay), A, 0, A, B, big, None) == INVALID    # chunk < 1
    assert f(A, 1000, C.byref(lay), A, moe.MOE_T_MAX + 1, A, B, big, None) == INVALID
    assert f(A, moe.MOE_T_MAX + 1, C.byref(lay), A, 256, A, B, big, None) == INVALID
    assert f(A, 1000, None, A, 256, A, B, big, None) == INVALID
    assert f(A, 1000, C.byref(lay), A, 256, A, None, big, None) == INVALID
    assert f(A, 1000, C.byref(lay), A, 256, A, B, big - 1, None) == WS   # sized by the chunk
    assert f(A, 1000, C.byref(lay), A, 256, A, A + big - 256, big, None) == INVALID   # overlap
    assert f(A, 1000, C.byref(lay), A, 256, A, B + 4, big, None) == ALIGN
    assert f(MIS, 1000, C.byref(lay), A, 256, A, B, big, None) == ALIGN


def test_chain_forward_validation(L):
    big = moe.moe_workspace_bytes(4)
    f = L.moe_chain_forward
    arr = (moe.moe_layer * 3)(_layer(), _layer(), _layer())
    assert f(A, 0, arr, 3, A, None, A, big, None, None) == OK           # T = 0: no-op
    assert f(A, 4, arr, 0, A, None, A, big, None, None) == OK           # no layers: no-op
    assert f(A, 4, arr, -1, A, None, A, big, None, None) == INVALID
    assert f(A, 4, None, 3, A, None, A, big, None, None) == INVALID
    assert f(A, 4, arr, 3, None, None, A, big, None, None) == INVALID
    assert f(A, 4, arr, 3, A, MIS, A, big, None, None) == ALIGN
    assert f(A, 4, arr, 3, A, None, A, big - 1, None, None) == WS
    bad = (moe.moe_layer * 3)(_layer(), _layer(), _layer())
    bad[2].shared.down_s = MIS                                            # checked in every layer
    assert f(A, 4, bad, 3, A, None, A, big, None, None) == ALIGN
    opt = moe.moe_options(moe.MOE_PATH_AUTO, A)                           # residual_out: not for chains
    assert f(A, 4, arr, 3, A, None, A, big, None, C.byref(opt)) == INVALID
    opt = moe.moe_options(moe.MOE_PATH_DECODE, None)
    assert f(A, moe.MOE_DECODE_T_MAX + 1, arr, 3, A, None, A, 1 << 40, None, C.byref(opt)) == INVALID


def test_buffer_ranges_fit_32bit_offsets():
    """The kernels address their buffers with 32-bit buffer-resource ranges
    and offsets.  At the largest T every whole-buffer range they use must stay
    below 2^32; the fp32 expert output of the split call does not (9 * 65536
    rows of 8 KB = 4.83e9 B), which is why the grouped GEMM bases each item's
    output range at the item's first row (at most 160 rows)."""
    T, H, I = moe.MOE_T_MAX, moe.MOE_HIDDEN, moe.MOE_INTER
    whole = {
        "x rows of the gate/up GEMM (fp16)": T * H * 2,
        "h rows of the down GEMM (fp16)": 9 * T * I * 2,
        "router input x (bf16)": T * H * 2,
        "permutation entries": 8 * T * 4,
        "fp16 weighted down rows of the fused layer": 9 * T * H * 2,
    }
    for what, n in whole.items():
        assert n < 2 ** 32, what
    assert 9 * T * H * 4 >= 2 ** 32          # the split call's output: per-item ranges needed
    assert 160 * H * 4 < 2 ** 31             # one item's rows: far inside the range
    # the largest row offset inside any whole-buffer range, as the kernels form it
    assert (9 * T - 1) * I * 2 + (I * 2 - 16) < 2 ** 32


def test_chain_noalloc_validation(L):
    f = L.moe_chain_forward_noalloc
    arr = (moe.moe_layer * 2)(_layer(), _layer())
    assert f(A, 0, arr, 2, A, None, None, None) == OK                      # T = 0: no-op
    assert f(A, moe.MOE_NOALLOC_T_MAX + 1, arr, 2, A, None, None, None) == INVALID
    assert f(A, -1, arr, 2, A, None, None, None) == INVALID
    assert moe.moe_workspace_bytes(moe.MOE_NOALLOC_T_MAX) <= moe.MOE_NOALLOC_WS_BYTES


def test_greedy_validation(L):
    big = moe.moe_workspace_bytes(8)
    f = L.moe_lm_head_argmax
    assert f(A, 0, A, 100, A, A, big, None) == INVALID
    assert f(A, moe.MOE_DECODE_T + 1, A, 100, A, A, 1 << 40, None) == INVALID
    assert f(A, 1, A, 0, A, A, big, None) == INVALID
    assert f(A, 1, None, 100, A, A, big, None) == INVALID
    assert f(MIS, 1, A, 100, A, A, big, None) == ALIGN
    assert f(A, 1, A, 100, A, A, 16, None) == WS
    g = L.moe_embed
    assert g(A, 0, A, 100, A, None) == OK
    assert g(A, 3, A, 0, A, None) == INVALID
    assert g(A, 3, None, 100, A, None) == INVALID
    assert g(A, 3, A, 100, MIS, None) == ALIGN


def test_router_transpose_validation(L):
    assert L.moe_router_transpose(None, A, None) == INVALID
    assert L.moe_router_transpose(A, None, None) == INVALID
    assert L.moe_router_transpose(A, MIS, None) == ALIGN


def test_probe_validation(L):
    assert L.moe_probe_read(A, 0, A, None) == INVALID
    assert L.moe_probe_read(A, 17, A, None) == INVALID
    assert L.moe_probe_copy(A, MIS, 32, None) == ALIGN


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "gemv_router_softmax_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), fn
                assert "moe_oracle" not in src and "libmoe_oracle" not in src, fn


def test_gdn_workspace_bytes(L):
    assert moe.moe_gdn_workspace_bytes(-1, 4) == 0
    assert moe.moe_gdn_workspace_bytes(10, 0) == 0
    assert moe.moe_gdn_workspace_bytes(10, moe.MOE_GDN_HEADS_MAX + 1) == 0
    assert moe.moe_gdn_workspace_bytes(moe.MOE_T_MAX + 1, 4) == 0
    assert moe.moe_gdn_workspace_bytes(0, 4) == 0
    prev = 0
    for T in [1, 63, 64, 65, 2048, 65536]:
        b = moe.moe_gdn_workspace_bytes(T, 32)
        assert b >= prev and b % 256 == 0
        assert b == moe.moe_gdn_workspace_bytes(1, 32) * ((T + 63) // 64)
        prev = b


def test_gdn_rejects_bad_arguments(L):
    """moe_gdn_scan(q, k, v, g, beta, T, hk, hv, s0, o, s_out, ws, ws_bytes, stream)."""
    f = L.moe_gdn_scan
    big = 1 << 40
    ok = dict(q=A, k=A, v=A, g=A, beta=A, T=100, hk=2, hv=4, s0=None, o=A, s_out=None, ws=A,
              ws_bytes=big)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["T"], a["hk"], a["hv"], a["s0"],
                 a["o"], a["s_out"], a["ws"], a["ws_bytes"], None)
    assert call(hv=3) == INVALID                       # hv not a multiple of hk
    assert call(hk=0) == INVALID
    assert call(hv=moe.MOE_GDN_HEADS_MAX + 2, hk=2) == INVALID
    assert call(T=-1) == INVALID
    assert call(T=moe.MOE_T_MAX + 1) == INVALID
    assert call(q=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(k=MIS) == ALIGN
    assert call(ws=A + 16) == ALIGN                    # workspace must be 256-byte aligned
    assert call(s_out=A + 2) == ALIGN
    assert call(ws_bytes=moe.moe_gdn_workspace_bytes(100, 4) - 1) == WS
    assert call(T=0, s_out=None) == OK                 # nothing to do
