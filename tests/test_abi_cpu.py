"""The C ABI on the host: the library loads, exports every declared symbol and
rejects bad arguments before anything reaches the device (no GPU needed)."""

import ctypes as C
import os
import re

import pytest

from dense_long_context_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlc.h")

OK, E_INVAL, E_DTYPE, E_SHAPE, E_WORKSPACE, E_HIP, E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
P = 0x1000  # a fake, 256-byte aligned pointer: never dereferenced, validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
        assert n in binding.SIGNATURES, f"binding lacks {n}"


def test_version_and_status_strings(L):
    assert L.dlc_abi_version() == 1
    assert binding.status_str(E_WORKSPACE) == "DLC_E_WORKSPACE"
    assert binding.status_str(12345) == "DLC_E_UNKNOWN"


def _csa_compress(L, **kw):
    a = dict(dtype=BF16, B=1, n=16, c=8, m=4, Za=P, Zb=P, Ca=P, Cb=P, ld=8, bs=128, Ba=None, Bb=None,
             i0=0, i1=4, out=P, cap=4)
    a.update(kw)
    return L.csa_compress(a["dtype"], a["B"], a["n"], a["c"], a["m"], a["Za"], a["Zb"], a["Ca"], a["Cb"],
                          a["ld"], a["bs"], a["Ba"], a["Bb"], a["i0"], a["i1"], a["out"], a["cap"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), E_DTYPE),
    (dict(m=0), E_INVAL),
    (dict(c=0), E_INVAL),
    (dict(B=0), E_INVAL),
    (dict(Za=None), E_INVAL),
    (dict(out=None), E_INVAL),
    (dict(Zb=None), E_INVAL),          # CSA needs the b-streams
    (dict(ld=4), E_SHAPE),             # ld < c
    (dict(B=2, bs=64), E_SHAPE),       # sequences overlap
    (dict(i1=5), E_SHAPE),             # i_end > n/m
    (dict(i0=3, i1=2), E_SHAPE),
    (dict(i0=-1), E_SHAPE),
    (dict(cap=3), E_SHAPE),            # cap < i_end
    (dict(i0=2, i1=2), OK),            # empty range: nothing to do, nothing launched
])
def test_csa_compress_validation(L, kw, status):
    assert _csa_compress(L, **kw) == status
    if status:
        assert binding.last_error().startswith("csa_compress")


def test_hca_compress_validation(L):
    assert L.hca_compress(BF16, 1, 12, 8, 3, P, P, 8, 96, None, 0, 5, P, 5, None) == E_SHAPE
    assert L.hca_compress(BF16, 1, 12, 8, 3, P, None, 8, 96, None, 0, 4, P, 4, None) == E_INVAL
    assert L.hca_compress(BF16, 1, 12, 8, 3, P, P, 8, 96, None, 0, 0, P, 4, None) == OK


def _topk(L, **kw):
    a = dict(dtype=BF16, B=1, n_q=1, n_hI=4, cI=64, m=4, k=8, qI=P, wI=P, KI=P, cap=16, t=P, t_max=64,
             idx=P, count=P, scores=None, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return L.csa_index_topk(a["dtype"], a["B"], a["n_q"], a["n_hI"], a["cI"], a["m"], a["k"], a["qI"],
                            a["wI"], a["KI"], a["cap"], a["t"], a["t_max"], a["idx"], a["count"],
                            a["scores"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), E_DTYPE),
    (dict(k=0), E_UNSUPPORTED),
    (dict(k=8193), E_UNSUPPORTED),
    (dict(n_hI=128, cI=128), E_UNSUPPORTED),
    (dict(m=0), E_INVAL),
    (dict(t_max=68), E_SHAPE),          # floor(68/4) = 17 > cap
    (dict(qI=None), E_INVAL),
    (dict(idx=None), E_INVAL),
    (dict(ws=None), E_WORKSPACE),
    (dict(ws_bytes=16), E_WORKSPACE),
    (dict(ws=P + 8), E_WORKSPACE),      # misaligned
])
def test_index_topk_validation(L, kw, status):
    assert _topk(L, **kw) == status


def _topk_fp4(L, **kw):
    a = dict(dtype=BF16, B=1, n_q=1, n_hI=4, cI=128, m=4, k=8, qI=P, wI=P, KIc=P, KIs=P, cap=16, t=P,
             t_max=64, idx=P, count=P, scores=None, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return L.csa_index_topk_fp4(a["dtype"], a["B"], a["n_q"], a["n_hI"], a["cI"], a["m"], a["k"], a["qI"],
                                a["wI"], a["KIc"], a["KIs"], a["cap"], a["t"], a["t_max"], a["idx"], a["count"],
                                a["scores"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), E_DTYPE),
    (dict(cI=64), E_UNSUPPORTED),
    (dict(cI=96), E_UNSUPPORTED),
    (dict(n_hI=65), E_UNSUPPORTED),
    (dict(k=0), E_UNSUPPORTED),
    (dict(m=0), E_INVAL),
    (dict(t_max=68), E_SHAPE),          # floor(68/4) = 17 > cap
    (dict(KIs=None), E_INVAL),
    (dict(qI=P + 4), E_INVAL),          # misaligned query
    (dict(KIs=P + 2), E_INVAL),         # misaligned key scales
    (dict(ws_bytes=16), E_WORKSPACE),
])
def test_index_topk_fp4_validation(L, kw, status):
    assert _topk_fp4(L, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((BF16, 1, 4, 48, P, 192, P, 96, P, 6), E_SHAPE),      # width not a multiple of 32
    ((7, 1, 4, 64, P, 256, P, 128, P, 8), E_DTYPE),
    ((BF16, 1, 4, 64, None, 256, P, 128, P, 8), E_INVAL),
    ((BF16, 2, 4, 64, P, 128, P, 128, P, 8), E_SHAPE),     # batch stride shorter than the rows
    ((BF16, 1, 4, 64, P + 2, 256, P, 128, P, 8), E_INVAL),  # misaligned source
    ((BF16, 1, 0, 64, None, 0, None, 0, None, 0), OK),      # no rows: nothing to do
])
def test_mxfp4_quantize_validation(L, args, status):
    assert L.mxfp4_quantize(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((1, 0, 8, P, P, P), E_INVAL),          # n_h = 0
    ((1, 4, 0, P, P, P), E_INVAL),          # c = 0
    ((1, 4, 8, None, P, P), E_INVAL),
    ((1, 4, 8, P, P, None), E_INVAL),
    ((1, 4, 8, P + 4, P, P), E_INVAL),      # misaligned output
    ((0, 4, 8, None, None, None), OK),      # no rows: nothing to do
])
def test_attend_sink_validation(L, args, status):
    assert L.attend_sink(*args, None) == status


def test_fp4_workspace_query(L):
    base = L.csa_index_topk_ws(4, 1, 262144, 1024)
    w = L.csa_index_topk_fp4_ws(4, 1, 64, 128, 262144, 1024)
    assert w >= base + 4 * 64 * (64 + 4) and w % 256 == 0
    assert L.csa_index_topk_fp4_ws(0, 1, 64, 128, 10, 1) == 0


def test_workspace_queries(L):
    w1 = L.csa_index_topk_ws(4, 1, 262144, 1024)
    assert w1 > 262144 * 4 * 4
    assert L.csa_index_topk_ws(4, 2, 262144, 1024) > w1
    assert L.csa_index_topk_ws(0, 1, 10, 1) == 0
    assert L.csa_attend_ws(1, 1, 1, 2, 1) == 0           # one split: no partials
    big = L.hca_attend_ws(16, 1, 128, 512, 8192)
    assert big > 0 and big % 256 == 0
    assert L.hca_attend_ws(16, 1, 128, 512, 16384) >= big


def test_prefill_workspace_does_not_grow_with_the_cache(L):
    """Query-tiled calls (64 or more queries a sequence) run the cache in
    ranges: their workspace depends on the queries and k, not on cap; decode
    calls keep one array per entry."""
    sizes = [L.csa_index_topk_ws(4, 256, cap, 1024) for cap in (40000, 262144, 1 << 20, (1 << 22) + 3)]
    assert len(set(sizes)) == 1, sizes
    assert L.csa_index_topk_ws(4, 256, 20000, 1024) <= sizes[0]  # a cache shorter than one range
    fp4 = [L.csa_index_topk_fp4_ws(4, 256, 64, 128, cap, 1024) for cap in (40000, 1 << 20)]
    assert fp4[0] == fp4[1]
    assert L.csa_index_topk_ws(4, 1, 1 << 20, 1024) > L.csa_index_topk_ws(4, 1, 1 << 18, 1024)


def test_attend_validation(L):
    args = lambda **kw: dict(dict(dtype=BF16, B=1, n_q=1, n_h=4, c=128, k=8, q=P, C=P, cap=16, idx=P,  # noqa
                                  count=P, out=P, lse=None, ws=None, wsb=0), **kw)
    def csa(**kw):
        a = args(**kw)
        return L.csa_attend(a["dtype"], a["B"], a["n_q"], a["n_h"], a["c"], a["k"], a["q"], a["C"], a["cap"],
                            a["idx"], a["count"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"], None)
    assert csa(dtype=9) == E_DTYPE
    assert csa(k=0) == E_INVAL
    assert csa(idx=None) == E_INVAL
    assert csa(q=P + 2) == E_INVAL                       # MFMA path needs 16-byte alignment
    assert csa(dtype=F32, c=2048) == E_UNSUPPORTED
    assert csa(B=4, n_h=128, c=512, k=1024) == E_WORKSPACE
    # the c = 512 kernel lists a split's gathered rows in LDS: at most 256
    # splits of 2048 keys, refused beyond that before anything is launched
    assert csa(n_h=128, c=512, k=256 * 2048 + 1, ws=P, wsb=1 << 40) == E_UNSUPPORTED
    assert L.hca_attend(BF16, 1, 1, 4, 128, 128, P, P, 4, P, 1024, 0.0, P, None, None, 0, None) == E_SHAPE
    assert L.hca_attend(BF16, 1, 1, 4, 128, 0, P, P, 4, P, 100, 0.0, P, None, None, 0, None) == E_INVAL


def test_window_validation(L):
    def win(**kw):
        a = dict(dict(dtype=BF16, B=1, n_q=1, n_h=4, c=128, n_win=128, q=P, C=P, ring=128, t=P, t_max=10,
                      o_in=None, lse_in=None, out=P, lse=None, ws=None, wsb=0), **kw)
        return L.window_attend(a["dtype"], a["B"], a["n_q"], a["n_h"], a["c"], a["n_win"], a["q"], a["C"],
                               a["ring"], a["t"], a["t_max"], 0.0, a["o_in"], a["lse_in"], a["out"], a["lse"],
                               a["ws"], a["wsb"], None)
    assert win(dtype=7) == E_DTYPE
    assert win(n_win=0) == E_INVAL
    assert win(t=None) == E_INVAL
    assert win(ring=64) == E_SHAPE                       # ring smaller than the window
    assert win(o_in=P) == E_INVAL                        # o_in without lse_in
    assert win(o_in=P, lse_in=P) == E_WORKSPACE          # joining needs the partial buffers
    assert L.window_attend_ws(4, 1, 128, 512, 128) > 0
    assert L.window_attend_ws(4, 1, 128, 512, 0) == 0


def _csa_fused(L, **kw):
    a = dict(dtype=BF16, B=1, n=256, d=64, c=64, m=4, H=P, ldh=64, hbs=256 * 64, W=P, ldw=64, Ba=None, Bb=None,
             i0=0, i1=64, out=P, cap=64)
    a.update(kw)
    return L.csa_project_compress(a["dtype"], a["B"], a["n"], a["d"], a["c"], a["m"], a["H"], a["ldh"], a["hbs"],
                                  a["W"], a["W"], a["W"], a["W"], a["ldw"], a["Ba"], a["Bb"], a["i0"], a["i1"],
                                  a["out"], a["cap"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=F32), E_UNSUPPORTED),  # the fused pass is bf16 only
    (dict(m=0), E_INVAL),
    (dict(H=None), E_INVAL),
    (dict(W=None), E_INVAL),
    (dict(c=48), E_UNSUPPORTED),       # channels come in groups of 32
    (dict(m=3), E_UNSUPPORTED),        # the ratio must divide the 128-row tile
    (dict(m=128, i1=2), E_UNSUPPORTED),  # CSA needs a tile of more than one block
    (dict(d=60, ldh=64, ldw=64), E_UNSUPPORTED),  # K rows in whole 16-byte vectors
    (dict(ldh=32), E_SHAPE),           # ldh < d
    (dict(B=2, hbs=64), E_SHAPE),      # sequences overlap
    (dict(i1=65), E_SHAPE),            # i_end > n/m
    (dict(cap=63), E_SHAPE),
    (dict(i0=5, i1=5), OK),            # empty range: nothing launched
])
def test_project_compress_validation(L, kw, status):
    assert _csa_fused(L, **kw) == status
    if status:
        assert binding.last_error().startswith("csa_project_compress")


def test_hca_project_compress_validation(L):
    args = lambda **kw: dict(dict(c=128, m=128, i1=2, cap=2), **kw)  # noqa: E731
    fused = lambda a: L.hca_project_compress(BF16, 1, 256, 64, a["c"], a["m"], P, 64, 256 * 64, P, P, 64,  # noqa: E731
                                             None, 0, a["i1"], P, a["cap"], None)
    assert fused(args(c=96)) == E_UNSUPPORTED   # channels come in groups of 64
    assert fused(args(m=256, i1=1)) == E_UNSUPPORTED
    assert fused(args(i1=3)) == E_SHAPE
    assert fused(args(i1=0)) == OK
    assert L.hca_project_compress(BF16, 1, 256, 64, 128, 128, P, 64, 256 * 64, P, None, 64, None, 0, 2, P, 2,
                                  None) == E_INVAL


def test_bandwidth_references_validation(L):
    assert L.dlc_copy(P, P, 1000, None) == E_INVAL        # not a multiple of 16 bytes
    assert L.dlc_read(P, 1000, 0, None) == E_INVAL        # direct-to-LDS form: not a multiple of 1 KB
    assert L.dlc_read(P, 1024, 1, None) == E_INVAL        # tile form: not a multiple of 4 KB
    assert L.dlc_read(P, 4096, 2, None) == E_INVAL        # no such form
    assert L.dlc_read(None, 1024, 0, None) == E_INVAL
    assert L.dlc_read(P, 0, 0, None) == OK
    assert L.dlc_read(P, 0, 1, None) == OK


def test_timing_arm_stages(L):
    for stage in range(1, 8):  # DLC_STAGE_INDEX_SCORES .. DLC_STAGE_READ
        assert L.dlc_timing_arm(stage, None, None) == OK  # NULL events: disarmed
    assert L.dlc_timing_arm(0, None, None) == E_INVAL
    assert L.dlc_timing_arm(8, None, None) == E_INVAL


def test_project_validation(L):
    assert L.dlc_project(BF16, 4, 4, 0, P, 8, P, 8, P, 4, BF16, None, 0, None) == E_INVAL
    assert L.dlc_project(BF16, 4, 4, 8, P, 4, P, 8, P, 4, BF16, None, 0, None) == E_SHAPE
    assert L.dlc_project(F32, 4, 4, 8, P, 8, P, 8, P, 4, BF16, None, 0, None) == E_DTYPE
    assert L.dlc_project(BF16, 0, 4, 8, P, 8, P, 8, P, 4, BF16, None, 0, None) == OK
    # the row path's k-split workspace: used where N is small and K large, never above 16 rows
    need = L.dlc_project_ws(BF16, 4, 512, 7168)
    assert need >= 32 * 8 * 1024                                   # 32 column tiles, 8 slices of 1 KB each
    assert L.dlc_project_ws(BF16, 4, 65536, 512) == 0              # enough column tiles already
    assert L.dlc_project_ws(BF16, 17, 512, 7168) == 0              # the 128-row tile path
    assert L.dlc_project_ws(F32, 4, 512, 7168) == 0
    assert L.dlc_project(BF16, 4, 512, 7168, P, 7168, P, 7168, P, 512, BF16, P, need - 1, None) == E_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        binding.lib()


def test_attend_gather_limit(L):
    """csa_attend's c = 512 kernel lists a split's gathered rows in LDS: more
    keys than 256 splits x 2048 rows is refused, not run."""
    big = 256 * 2048 + 1
    rc = L.csa_attend(BF16, 1, 1, 128, 512, big, P, P, 1 << 20, P, P, 0.0, P, None, P, 1 << 40, None)
    assert rc == E_UNSUPPORTED
    assert "gathered keys" in binding.last_error()
    rc = L.csa_attend_window(BF16, 1, 1, 128, 512, big - 128, P, P, 1 << 20, P, P, P, 256, 129, P, 10, 0.0, P,
                             None, P, 1 << 40, None)
    assert rc == E_UNSUPPORTED


def test_binding_rejects_host_tensors():
    """Tensors the kernels would dereference must be on the CUDA device: a host
    tensor is refused by the binding before any call reaches the library."""
    import torch

    import dense_long_context_amd as dlc

    bf = torch.bfloat16
    qI, wI = torch.zeros((1, 1, 4, 64), dtype=bf), torch.zeros((1, 1, 4))
    KI, t = torch.zeros((1, 16, 64), dtype=bf), torch.tensor([[64]])
    q, C = torch.zeros((1, 1, 4, 128), dtype=bf), torch.zeros((1, 16, 128), dtype=bf)
    idx, cnt = torch.zeros((1, 1, 8), dtype=torch.int32), torch.zeros((1, 1), dtype=torch.int32)
    S = torch.zeros((1, 16, 8), dtype=bf)
    calls = [
        lambda: dlc.csa_index_topk(qI, wI, KI, t, 64, 4, 8),
        lambda: dlc.csa_attend(q, C, idx, cnt),
        lambda: dlc.hca_attend(q, C, t, 64, 4),
        lambda: dlc.window_attend(q, C, t, 64, 16),
        lambda: dlc.csa_compress(S, S, S, S, 4, torch.zeros((1, 4, 8), dtype=bf)),
        lambda: dlc.hca_compress(S, S, 4, torch.zeros((1, 4, 8), dtype=bf)),
        lambda: dlc.dlc_project(torch.zeros((4, 8), dtype=bf), torch.zeros((4, 8), dtype=bf)),
        lambda: dlc.mxfp4_quantize(torch.zeros((4, 64), dtype=bf)),
        lambda: dlc.attend_sink(torch.zeros((1, 4, 8)), torch.zeros((1, 4)), torch.zeros(4)),
    ]
    for f in calls:
        with pytest.raises(ValueError, match="CUDA device"):
            f()
