"""Stage parity on the GPU: every C-ABI call against the fp64 oracle on the
same seeded inputs, at sizes that span several tiles with ragged tails, plus
the degenerate cases (nothing visible, k >= visible, ties, masked indices).

Tolerances (derived in the design notes): fp32 outputs 1e-5 row-relative;
bf16-stored outputs 8e-3 row-relative (one bf16 rounding of an fp32 result);
fp32 attention outputs from bf16 inputs 2e-2 row-relative (the target bar);
top-k per the tie rule in devtools.check_topk (the target band: ties within
1e-4 relative at the k-th score), and exactly the selection rule applied to the
device's own fp32 scores; scores within their fp32 bound (devtools.score_bound).
"""

import math

import numpy as np
import pytest
import torch

import dense_long_context_amd as dlc
from dense_long_context_amd import binding
import oracle as O
import synth
from devtools import DEV, FlipTally, assert_rows_close, check_scores, check_topk, f64, need_gpu, score_bound

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL_STORE = {"f32": 1e-5, "bf16": 8e-3}
TOL_ATT = {"f32": 1e-5, "bf16": 2e-2}


def setup_module():
    need_gpu()


def _streams(B, n, c, dtype, seed, nstreams=4, ld=None, scale=1.0):
    """Streams [B][n][c] drawn as one [B][n][ld] buffer (ld >= c), returned as views."""
    ld = ld or c
    full = synth.normal((nstreams, B, n, ld), seed, std=scale, dtype=dtype)
    return [full[i] for i in range(nstreams)], full


# ------------------------------------------------------------------ compress

@pytest.mark.parametrize("dtype,B,n,c,m,ld,bias", [
    ("f32", 1, 6, 2, 2, 2, False),        # the worked example's shape
    ("f32", 2, 37, 5, 3, 7, True),        # generic path, ragged tail, strided rows
    ("f32", 3, 64, 12, 4, 12, True),      # fp32 vector path
    ("bf16", 2, 130, 6, 4, 6, True),      # bf16 generic path (c not a multiple of 8)
    ("bf16", 2, 1000, 128, 4, 136, True), # bf16 vector path, strided rows
    ("bf16", 1, 4096, 512, 4, 512, False),
    ("bf16", 2, 515, 64, 1, 64, True),    # m = 1
])
def test_csa_compress(dtype, B, n, c, m, ld, bias):
    seed = 100 + n
    (Za, Zb, Ca, Cb), full = _streams(B, n, ld, dtype, seed, scale=2.0)
    Za, Zb, Ca, Cb = (x[:, :, :c] for x in (Za, Zb, Ca, Cb))
    Ba = synth.normal((m, c), seed + 1, dtype="f32") if bias else None
    Bb = synth.normal((m, c), seed + 2, dtype="f32") if bias else None
    cap = n // m + 3
    dev = lambda x: None if x is None else x.to(DEV)  # noqa: E731
    # same strides on the device: move the full buffer and slice it
    dfull = full.to(DEV)
    dZa, dZb, dCa, dCb = (dfull[i][:, :, :c] for i in range(4))
    out = torch.full((B, cap, c), 7.0, dtype=TD[dtype], device=DEV)
    nent = n // m
    mid = nent // 3
    # two calls (entries [0, mid) then [mid, n/m)) must equal the definition
    dlc.csa_compress(dZa, dZb, dCa, dCb, m, out, 0, mid, dev(Ba), dev(Bb))
    dlc.csa_compress(dZa, dZb, dCa, dCb, m, out, mid, nent, dev(Ba), dev(Bb))
    torch.cuda.synchronize()
    got = out.cpu()
    for b in range(B):
        ref = O.csa_compress(Za[b], Zb[b], Ca[b], Cb[b], m, Ba, Bb)
        assert_rows_close(got[b, :nent], O.store_as(ref, dtype), TOL_STORE[dtype], f"csa b={b}")
        assert (got[b, nent:].float() == 7.0).all(), "entries past i_end must be untouched"


@pytest.mark.parametrize("dtype,B,n,c,mp,bias", [
    ("f32", 1, 6, 2, 3, False),
    ("f32", 2, 100, 9, 7, True),
    ("bf16", 3, 1000, 64, 128, True),
    ("bf16", 2, 8 * 128 + 50, 512, 128, False),
    ("bf16", 1, 77, 16, 1, True),
])
def test_hca_compress(dtype, B, n, c, mp, bias):
    seed = 300 + n
    (Z, Cs), full = _streams(B, n, c, dtype, seed, nstreams=2, scale=2.0)
    Bh = synth.normal((mp, c), seed + 1, dtype="f32") if bias else None
    cap = n // mp
    dfull = full.to(DEV)
    out = torch.empty((B, cap, c), dtype=TD[dtype], device=DEV)
    dlc.hca_compress(dfull[0], dfull[1], mp, out, bias=None if Bh is None else Bh.to(DEV))
    torch.cuda.synchronize()
    got = out.cpu()
    for b in range(B):
        ref = O.hca_compress(Z[b], Cs[b], mp, Bh)
        assert_rows_close(got[b], O.store_as(ref, dtype), TOL_STORE[dtype], f"hca b={b}")


@pytest.mark.parametrize("dtype,c,m,n", [
    ("bf16", 128, 4, 515),      # few entries: the lanes-per-chunk path
    ("bf16", 128, 4, 16400),    # full-pass path (one thread per entry pair and column group)
    ("f32", 12, 4, 44003),
    ("bf16", 64, 2, 301),
])
def test_compress_neg_inf_logits(dtype, c, m, n):
    """-inf logits, the page's padding device ("DeepSeek-V4 Hybrid Attention:
    CSA and HCA from Scratch", §4, block i = 0): a fully masked b-block (every
    b-row bias -inf, so a whole chunk of -inf logits) leaves the a-rows' softmax
    alone, scattered -inf biases drop their rows, and an HCA block whose first
    rows are all -inf pools over the rest."""
    B = 2
    seed = 4242 + c + n
    (Za, Zb, Ca, Cb), full = _streams(B, n, c, dtype, seed, scale=2.0)
    dfull = full.to(DEV)
    g = np.random.default_rng(seed)
    Ba = synth.normal((m, c), seed + 1, dtype="f32")
    mask = g.random((m, c)) < 0.3
    mask[0] = False                                   # every column keeps at least one a-row
    Ba[torch.from_numpy(mask)] = float("-inf")
    Bb_all = torch.full((m, c), float("-inf"))
    Bb_some = synth.normal((m, c), seed + 2, dtype="f32")
    Bb_some[torch.from_numpy(g.random((m, c)) < 0.5)] = float("-inf")
    cap = n // m
    for Bb, nm in ((Bb_all, "b-block masked"), (Bb_some, "scattered")):
        out = torch.full((B, cap, c), 7.0, dtype=TD[dtype], device=DEV)
        dlc.csa_compress(dfull[0], dfull[1], dfull[2], dfull[3], m, out, 0, cap, Ba.to(DEV), Bb.to(DEV))
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.isfinite(got.float()).all(), f"csa {nm}: non-finite entries"
        for b in range(B):
            ref = O.csa_compress(Za[b], Zb[b], Ca[b], Cb[b], m, Ba, Bb)
            assert_rows_close(got[b], O.store_as(ref, dtype), TOL_STORE[dtype], f"csa {nm} b={b}")
    # HCA: the first chunk of rows of every block fully masked, plus scattered -inf
    mp = 16
    Bh = synth.normal((mp, c), seed + 3, dtype="f32")
    Bh[:4] = float("-inf")
    Bh[4:][torch.from_numpy(g.random((mp - 4, c)) < 0.4)] = float("-inf")
    Bh[mp - 1] = 0.0                                   # every column keeps one row
    out = torch.empty((B, n // mp, c), dtype=TD[dtype], device=DEV)
    dlc.hca_compress(dfull[0], dfull[2], mp, out, bias=Bh.to(DEV))
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.isfinite(got.float()).all(), "hca: non-finite entries"
    for b in range(B):
        ref = O.hca_compress(Za[b], Ca[b], mp, Bh)
        assert_rows_close(got[b], O.store_as(ref, dtype), TOL_STORE[dtype], f"hca -inf b={b}")


# ------------------------------------------------------------ indexer, top-k

@pytest.mark.parametrize("dtype,B,n_q,n_hI,cI,m,k,cap,ts", [
    ("f32", 1, 1, 1, 2, 2, 1, 3, [5]),                      # worked-example shape
    ("f32", 2, 2, 3, 5, 4, 7, 50, [200, 37, 3, 150]),       # VALU path, ragged
    ("bf16", 1, 1, 4, 64, 4, 64, 2048, [8192]),             # decode-8k indexer shape
    ("bf16", 2, 3, 64, 128, 4, 100, 5000, [20000, 19999, 4, 333, 8000, 0]),
    ("bf16", 1, 2, 16, 32, 4, 1024, 1500, [6000, 4100]),    # k >= visible for one query
    ("bf16", 2, 1, 20, 64, 2, 300, 4000, [8000, 7777]),     # head padding (20 -> 32)
    ("bf16", 1, 1, 64, 256, 4, 16, 600, [2400]),
    ("bf16", 1, 2, 64, 128, 4, 8192, 20000, [80000, 40003]),  # the largest k the ABI takes
    ("bf16", 1, 1, 64, 128, 4, 2048, 200000, [800000]),     # 447 chunks of 448 entries
    # 3.2M visible entries: 65 or 66 tiles a wave, past the 64 whose scores a
    # wave keeps in LDS, so these waves store each tile's scores as they go
    ("bf16", 1, 1, 64, 128, 4, 1024, 3200000, [12800000]),
])
def test_index_topk(dtype, B, n_q, n_hI, cI, m, k, cap, ts):
    seed = 500 + cap
    qI = synth.normal((B, n_q, n_hI, cI), seed, dtype=dtype)
    wI = synth.normal((B, n_q, n_hI), seed + 1, dtype="f32")
    KI = synth.normal((B, cap, cI), seed + 2, dtype=dtype)
    t = torch.tensor(ts, dtype=torch.int64).reshape(B, n_q)
    t_max = int(t.max())
    scores = torch.full((B, n_q, cap), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt = dlc.csa_index_topk(qI.to(DEV), wI.to(DEV), KI.to(DEV), t.to(DEV), t_max, m, k, scores=scores)
    torch.cuda.synchronize()
    idx, cnt, sc = idx.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy()
    tally = FlipTally(f"index_topk {dtype} cap={cap}")
    for b in range(B):
        for j in range(n_q):
            tt = int(t[b, j])
            ref = O.index_scores(qI[b, j], wI[b, j], KI[b], tt, m)
            nv = len(ref)
            check_scores(sc[b, j, :nv], ref, score_bound(qI[b, j], wI[b, j], KI[b, :nv]), f"scores b={b} q={j}")
            tally.add(check_topk(idx[b, j], cnt[b, j], ref, k, dev_scores=sc[b, j, :nv]))
    tally.report()


@pytest.mark.parametrize("B,n_q,n_hI,cI,m,k,cap,seed", [
    (2, 100, 64, 128, 4, 100, 3000, 1),      # two query tiles (64 + 36), mixed visibilities
    (1, 64, 20, 128, 2, 50, 700, 2),         # 20 heads, one full tile
    (3, 70, 64, 128, 4, 1024, 2000, 3),      # k >= visible for most queries
    (2, 66, 64, 128, 4, 200, 1001, 4),       # cap % 4 != 0: score rows not 16-byte aligned (scalar head and tail)
    (1, 64, 64, 128, 4, 512, 70001, 5),      # three ranges of 32768 entries folded into a running top-k
    (1, 64, 32, 128, 4, 8192, 36000, 6),     # the largest k across two ranges
    # c^I other than 128: the per-query MFMA scores kernel runs range by range
    # (its rows counted from each range's first entry)
    (1, 64, 64, 64, 4, 300, 40000, 7),
    (1, 64, 32, 256, 4, 100, 33000, 8),      # c^I = 256: two tiles in flight per wave
])
def test_index_topk_prefill(B, n_q, n_hI, cI, m, k, cap, seed):
    """Many queries per sequence: the query-tiled MFMA scores kernel and the
    histogram pass (c^I = 128), or the per-query MFMA scores kernel (other
    widths), against the oracle for every query.  These calls run the cache
    in ranges of 32768 entries, each range's top-k folded into a running one,
    so a cache past 32768 entries crosses ranges."""
    qI = synth.normal((B, n_q, n_hI, cI), 700 + seed, dtype="bf16")
    wI = synth.normal((B, n_q, n_hI), 701 + seed, dtype="f32")
    KI = synth.normal((B, cap, cI), 702 + seed, dtype="bf16")
    rng = np.random.default_rng(seed)
    t = torch.from_numpy(rng.integers(0, m * cap + 1, size=(B, n_q))).to(torch.int64)
    t[0, 0], t[0, 1] = 0, m * cap          # nothing visible / everything visible
    t_max = int(t.max())
    scores = torch.full((B, n_q, cap), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt = dlc.csa_index_topk(qI.to(DEV), wI.to(DEV), KI.to(DEV), t.to(DEV), t_max, m, k, scores=scores)
    torch.cuda.synchronize()
    idx, cnt, sc = idx.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy()
    tally = FlipTally(f"index_topk prefill seed={seed}")
    for b in range(B):
        for j in range(n_q):
            tt = int(t[b, j])
            ref = O.index_scores(qI[b, j], wI[b, j], KI[b], tt, m)
            nv = len(ref)
            check_scores(sc[b, j, :nv], ref, score_bound(qI[b, j], wI[b, j], KI[b, :nv]), f"scores b={b} q={j}")
            assert np.isnan(sc[b, j, nv:]).all(), f"entries past the visible range written b={b} q={j}"
            tally.add(check_topk(idx[b, j], cnt[b, j], ref, k, dev_scores=sc[b, j, :nv]))
    tally.report()


def test_index_topk_ties_pick_smallest_indices():
    # every score equal (zero keys): the k smallest indices, in order
    B, cap, k = 1, 3000, 100
    qI = synth.normal((B, 1, 64, 128), 1, dtype="bf16")
    wI = synth.normal((B, 1, 64), 2, dtype="f32")
    KI = torch.zeros((B, cap, 128), dtype=torch.bfloat16)
    t = torch.tensor([[4 * cap]])
    idx, cnt = dlc.csa_index_topk(qI.to(DEV), wI.to(DEV), KI.to(DEV), t.to(DEV), 4 * cap, 4, k)
    assert int(cnt[0, 0]) == k
    assert idx[0, 0].cpu().tolist() == list(range(k))


def test_index_topk_duplicate_rows_break_ties_by_index():
    # 2001 exact copies of the best-scoring row: the top-512 are all tied at the
    # maximum, so the tie rule alone decides them: the 512 smallest indices
    cap, k = 4096, 512
    KI = synth.normal((1, cap, 64), 7, dtype="bf16")
    qI = synth.normal((1, 1, 8, 64), 8, dtype="bf16")
    wI = torch.ones((1, 1, 8))
    best = int(np.argmax(O.index_scores(qI[0, 0], wI[0, 0], KI[0], 4 * cap, 4)))
    KI[0, 1000:3000] = KI[0, best]
    ties = sorted(set(range(1000, 3000)) | {best})
    t = torch.tensor([[4 * cap]])
    idx, cnt = dlc.csa_index_topk(qI.to(DEV), wI.to(DEV), KI.to(DEV), t.to(DEV), 4 * cap, 4, k)
    assert int(cnt[0, 0]) == k
    assert idx[0, 0].cpu().tolist() == ties[:k]


def test_index_topk_workspace_reuse():
    """One workspace through several calls: garbage on entry (the selection
    then counts the first-digit histogram again from the scores), then the
    state each call leaves behind, for two queries and for one.  Every result
    against the oracle, a repeated call bit-identical, and the histogram area
    (the first B*n_q*2048 words) zero after every call."""
    n_hI, cI, m, k, cap = 64, 128, 4, 512, 30000
    qI = synth.normal((2, 1, n_hI, cI), 41, dtype="bf16")
    wI = synth.normal((2, 1, n_hI), 42, dtype="f32")
    KI = synth.normal((2, cap, cI), 43, dtype="bf16")
    ws = torch.full((dlc.csa_index_topk_ws(2, 1, cap, k),), 0xA5, dtype=torch.uint8, device=DEV)
    ws[: 2 * 2048 * 4].view(torch.float32).fill_(float("nan"))  # rows of equal words: their sum wraps to 0
    tally = FlipTally("index_topk workspace reuse")
    runs = []
    for B, ts in ((2, [120000, 90001]), (2, [120000, 90001]), (1, [50003]), (2, [7, 119999])):
        t = torch.tensor(ts, dtype=torch.int64).reshape(B, 1)
        scores = torch.empty((B, 1, cap), dtype=torch.float32, device=DEV)
        idx, cnt = dlc.csa_index_topk(qI[:B].to(DEV), wI[:B].to(DEV), KI[:B].to(DEV), t.to(DEV), int(t.max()), m, k,
                                      scores=scores, ws=ws)
        torch.cuda.synchronize()
        assert not ws[: B * 2048 * 4].any(), "histogram area not cleared"
        runs.append(idx.cpu())
        for b in range(B):
            ref = O.index_scores(qI[b, 0], wI[b, 0], KI[b], ts[b], m)
            nv = len(ref)
            tally.add(check_topk(idx[b, 0].cpu().numpy(), int(cnt[b, 0]), ref, k,
                                 dev_scores=scores[b, 0, :nv].cpu().numpy()))
    assert torch.equal(runs[0], runs[1])
    tally.report()


def test_index_topk_nothing_visible():
    qI = synth.normal((2, 1, 4, 64), 3, dtype="bf16")
    wI = synth.normal((2, 1, 4), 4, dtype="f32")
    KI = synth.normal((2, 10, 64), 5, dtype="bf16")
    t = torch.tensor([[3], [0]])
    idx, cnt = dlc.csa_index_topk(qI.to(DEV), wI.to(DEV), KI.to(DEV), t.to(DEV), 3, 4, 8)
    assert cnt.cpu().tolist() == [[0], [0]]
    assert (idx.cpu() == -1).all()


# ---------------------------------------------------------------- attention

def _random_selection(B, n_q, k, cap, seed, counts):
    g = torch.Generator().manual_seed(seed)
    idx = torch.full((B, n_q, k), -1, dtype=torch.int32)
    for b in range(B):
        for j in range(n_q):
            c = counts[b * n_q + j]
            sel = torch.randperm(cap, generator=g)[:c].sort().values
            idx[b, j, :c] = sel.to(torch.int32)
    cnt = torch.tensor(counts, dtype=torch.int32).reshape(B, n_q)
    return idx, cnt


@pytest.mark.parametrize("dtype,B,n_q,n_h,c,k,cap,counts", [
    ("f32", 1, 1, 1, 2, 1, 3, [1]),                          # worked-example shape
    ("f32", 2, 1, 3, 10, 9, 40, [9, 4]),                     # VALU path
    ("bf16", 1, 1, 16, 128, 64, 2048, [64]),                 # decode-8k shape
    ("bf16", 2, 2, 128, 512, 1024, 32768, [1024, 1000, 77, 0]),
    ("bf16", 1, 1, 48, 256, 300, 900, [299]),                # heads not a multiple of 32
    ("bf16", 1, 3, 128, 512, 40, 5000, [40, 33, 1]),
    ("bf16", 2, 1, 40, 512, 300, 2000, [300, 129]),           # c = 512 split partials, last head block partial
    # several head groups and a split count that is not a multiple of 8 (the
    # c = 512 grid runs splits in chunks of 8 per head group): 64-head groups
    # (4 groups, 5 splits), then 128-head groups (2 groups, 5 splits)
    ("bf16", 1, 1, 256, 512, 300, 2000, [300]),
    ("bf16", 4, 4, 256, 512, 300, 3000, [300, 299, 1, 0, 300, 150, 64, 65, 300, 300, 33, 257, 300, 2, 100, 200]),
    # the largest k: more gathered keys than one split holds in LDS (2048)
    ("bf16", 1, 2, 128, 512, 8192, 9000, [8192, 5000]),
])
def test_csa_attend(dtype, B, n_q, n_h, c, k, cap, counts):
    seed = 700 + cap + k
    q = synth.normal((B, n_q, n_h, c), seed, dtype=dtype)
    C = synth.normal((B, cap, c), seed + 1, dtype=dtype)
    idx, cnt = _random_selection(B, n_q, k, cap, seed + 2, counts)
    out, lse = dlc.csa_attend(q.to(DEV), C.to(DEV), idx.to(DEV), cnt.to(DEV))
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        for j in range(n_q):
            sel = idx[b, j, :counts[b * n_q + j]].numpy()
            o_ref, l_ref = O.csa_attend(q[b, j], C[b], sel)
            if len(sel) == 0:
                assert (out[b, j] == 0).all() and torch.isneginf(lse[b, j]).all()
                continue
            assert_rows_close(out[b, j], o_ref, TOL_ATT[dtype], f"csa o b={b} q={j}")
            assert np.abs(f64(lse[b, j]) - l_ref).max() <= 1e-3 + 1e-5 * np.abs(l_ref).max()


def test_csa_attend_ignores_invalid_indices():
    B, k, cap, c, n_h = 1, 16, 100, 128, 32
    q = synth.normal((B, 1, n_h, c), 11, dtype="bf16")
    C = synth.normal((B, cap, c), 12, dtype="bf16")
    idx = torch.tensor([[[3, 7, -1, 250, 9, 11, 5000, 2] + [-1] * 8]], dtype=torch.int32)
    cnt = torch.tensor([[10]], dtype=torch.int32)  # count beyond the valid run: padding ignored too
    out, lse = dlc.csa_attend(q.to(DEV), C.to(DEV), idx.to(DEV), cnt.to(DEV))
    o_ref, l_ref = O.csa_attend(q[0, 0], C[0], [3, 7, 9, 11, 2])
    assert_rows_close(out[0, 0].cpu(), o_ref, 2e-2, "masked indices")


@pytest.mark.parametrize("dtype,B,n_q,n_h,c,mp,cap,ts", [
    ("f32", 1, 1, 1, 2, 3, 2, [5]),                          # worked-example shape
    ("f32", 2, 1, 2, 16, 4, 30, [100, 7]),
    ("bf16", 1, 1, 16, 128, 128, 64, [8192]),                # decode-8k shape
    ("bf16", 3, 1, 128, 512, 128, 700, [700 * 128, 3 * 128 + 5, 100]),
    ("bf16", 2, 2, 40, 256, 16, 513, [513 * 16, 16 * 500 + 3, 31, 16 * 64]),
    ("bf16", 2, 1, 24, 512, 128, 3000, [3000 * 128, 128 * 777 + 5]),  # c = 512, 24 heads: one partial head block
])
def test_hca_attend(dtype, B, n_q, n_h, c, mp, cap, ts):
    seed = 900 + cap
    q = synth.normal((B, n_q, n_h, c), seed, dtype=dtype)
    C = synth.normal((B, cap, c), seed + 1, dtype=dtype)
    t = torch.tensor(ts, dtype=torch.int64).reshape(B, n_q)
    out, lse = dlc.hca_attend(q.to(DEV), C.to(DEV), t.to(DEV), int(t.max()), mp)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for b in range(B):
        for j in range(n_q):
            o_ref, l_ref = O.hca_attend(q[b, j], C[b], int(t[b, j]), mp)
            if not np.isfinite(l_ref).any():
                assert (out[b, j] == 0).all() and torch.isneginf(lse[b, j]).all()
                continue
            assert_rows_close(out[b, j], o_ref, TOL_ATT[dtype], f"hca o b={b} q={j}")
            assert np.abs(f64(lse[b, j]) - l_ref).max() <= 1e-3 + 1e-5 * np.abs(l_ref).max()


@pytest.mark.parametrize("n_q,n_h,mp,cap,seed,sample", [
    (256, 120, 16, 1100, 1, (0, 1, 2, 77, 128, 255)),  # one split per query (fp32 output), a partial head block
    (16, 128, 4, 16400, 2, (0, 1, 9)),                  # 16 splits of 1056 keys: bf16 partials, empty splits, combine
])
def test_hca_attend_long_splits(n_q, n_h, mp, cap, seed, sample):
    """Splits of at least 1024 keys run the c = 512 kernel in its HD form (the
    softmax per head, P exchanged through LDS, O split by dims): sampled
    queries against the oracle, with an empty query, a full one and ragged
    key counts."""
    c = 512
    q = synth.normal((1, n_q, n_h, c), 1700 + seed, dtype="bf16")
    C = synth.normal((1, cap, c), 1710 + seed, dtype="bf16")
    rng = np.random.default_rng(seed)
    t = torch.from_numpy(rng.integers(1024 * mp, cap * mp + 1, size=(1, n_q))).to(torch.int64)
    t[0, 0], t[0, 1] = mp - 1, cap * mp  # no key; every key
    out, lse = dlc.hca_attend(q.to(DEV), C.to(DEV), t.to(DEV), int(t.max()), mp)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for j in sample:
        o_ref, l_ref = O.hca_attend(q[0, j], C[0], int(t[0, j]), mp)
        if not np.isfinite(l_ref).any():
            assert (out[0, j] == 0).all() and torch.isneginf(lse[0, j]).all()
            continue
        assert_rows_close(out[0, j], o_ref, TOL_ATT["bf16"], f"hca long splits q={j}")
        assert np.abs(f64(lse[0, j]) - l_ref).max() <= 1e-3 + 1e-5 * np.abs(l_ref).max()


def test_hca_attend_window_long_splits():
    """The window branch joined to HCA with 256 consecutive queries of one
    sequence (one split of >= 1024 keys each: the HD form with the window's
    keys as the tail of the key list)."""
    n_q, n_h, c, mp, cap, ring, n_win = 256, 128, 512, 16, 1100, 512, 128
    q = synth.normal((1, n_q, n_h, c), 1750, dtype="bf16")
    Ch = synth.normal((1, cap, c), 1751, dtype="bf16")
    R = _ring(1, ring, c, "bf16", 1752)
    t = (cap * mp - n_q + torch.arange(n_q, dtype=torch.int64)).reshape(1, n_q)
    o, lse = dlc.hca_attend_window(q.to(DEV), Ch.to(DEV), t.to(DEV), int(t.max()), mp, R.to(DEV), n_win)
    torch.cuda.synchronize()
    for j in (0, 100, 255):
        o1, l1 = O.hca_attend(q[0, j], Ch[0], int(t[0, j]), mp)
        o2, l2 = _window_ref(q[0, j], R[0], t[0, j], n_win)
        o_r, l_r = O.merge_lse(o1, l1, o2, l2)
        assert_rows_close(o[0, j], o_r, TOL_ATT["bf16"], f"hca+window long splits q={j}")
        assert np.abs(lse[0, j].cpu().numpy() - l_r).max() <= TOL_ATT["bf16"]


# --------------------------------------------------------------- projection

@pytest.mark.parametrize("dtype,M,N,K,out_dtype", [
    ("f32", 6, 2, 2, "f32"),
    ("f32", 33, 70, 19, "f32"),
    ("bf16", 300, 260, 1024, "bf16"),
    ("bf16", 129, 64, 72, "f32"),
    ("bf16", 1, 8192, 512, "bf16"),     # row-vector path (M <= 16) from here on: one wave per column tile
    ("bf16", 4, 1000, 520, "f32"),      # ragged column tiles, K % 32 = 8 (last step partly masked), 4 waves a tile
    ("bf16", 3, 70, 40, "f32"),         # two steps, the second with one lane group in range
    ("bf16", 7, 512, 7168, "bf16"),     # the query down-projection's shape, 16 waves a tile
    ("bf16", 16, 64, 7168, "f32"),      # M = 16, four column tiles
    ("bf16", 17, 300, 256, "f32"),      # M = 17: back on the 128-row tile path
    ("bf16", 4, 64, 7168, "f32"),       # the indexer weight projection's shape: 4 tiles, k split 8 ways
    ("bf16", 2, 200, 968, "bf16"),      # 13 tiles (last one ragged), k split 4 ways into slices of 8, 8, 8, 7 steps
])
def test_project(dtype, M, N, K, out_dtype):
    A = synth.normal((M, K), 41, dtype=dtype)
    W = synth.normal((K, N), 42, std=K ** -0.5, dtype=dtype)
    dA, dW = A.to(DEV), W.t().contiguous().to(DEV)
    ref = O.project(A, W)
    want = O.store_as(ref, out_dtype) if out_dtype == "bf16" else ref
    tol = 1e-5 if out_dtype == "f32" else 8e-3
    out = dlc.dlc_project(dA, dW, out_dtype=TD[out_dtype])
    assert_rows_close(out.cpu(), want, tol, "project")
    again = dlc.dlc_project(dA, dW, out_dtype=TD[out_dtype])
    assert torch.equal(out, again), "dlc_project must give the same bits on a repeated call"
    # with a workspace: the row path may split the k-range over workgroups
    ws = dlc.project_workspace(M, N, K, DEV, TD[dtype])
    if ws is not None:
        split = dlc.dlc_project(dA, dW, out_dtype=TD[out_dtype], ws=ws)
        assert_rows_close(split.cpu(), want, tol, "project, k split over workgroups")
        assert int(ws.count_nonzero()) == 0, "the workspace is left all zero"
        again = dlc.dlc_project(dA, dW, out_dtype=TD[out_dtype], ws=ws)
        assert torch.equal(split, again), "the k-split result must be the same bits on a reused workspace"


@pytest.mark.gpu
def test_project_workspace_shared():
    """One workspace for calls of different shapes (each leaves it zeroed): the
    query down-projection, the indexer weights and a wide projection in turn."""
    shapes = [(4, 512, 7168), (4, 64, 7168), (4, 8192, 512), (3, 200, 968), (4, 512, 7168)]
    ws = torch.zeros(max(dlc.dlc_project_ws(M, N, K) for M, N, K in shapes), dtype=torch.uint8, device=DEV)
    for i, (M, N, K) in enumerate(shapes):
        A = synth.normal((M, K), 60 + i, dtype="bf16")
        W = synth.normal((K, N), 70 + i, std=K ** -0.5, dtype="bf16")
        out = dlc.dlc_project(A.to(DEV), W.t().contiguous().to(DEV), out_dtype=torch.float32, ws=ws)
        assert_rows_close(out.cpu(), O.project(A, W), 1e-5, f"project {M}x{N}x{K}, shared workspace")
        assert int(ws.count_nonzero()) == 0


# ------------------------------------------------------------ sliding window

def _ring(B, ring, c, dtype, seed):
    return synth.normal((B, ring, c), seed, dtype=dtype)


def _window_ref(q, R, t, n_win):
    """Oracle window attention of one query: the window's positions, their rows
    read from the ring (token p at row p % ring)."""
    pos = O.window_positions(int(t), n_win)
    rows = f64(R)[pos % R.shape[0]]
    return O.mqa_attend(q, rows)


@pytest.mark.parametrize("dtype,B,n_q,n_h,c,n_win,ring,ts", [
    ("f32", 1, 1, 3, 5, 4, 4, [2]),                                   # VALU path, partial window
    ("f32", 2, 1, 2, 8, 4, 4, [10, 3]),                               # wrap-around
    ("bf16", 2, 1, 16, 128, 128, 128, [300, 50]),                     # c = 128 MFMA path
    ("bf16", 4, 1, 128, 512, 128, 128, [(1 << 20) + 5, (1 << 20) + 200, 127, 0]),  # V4-Pro shape, t = 0
    ("bf16", 1, 3, 128, 512, 128, 130, [1000, 999, 998]),             # prefill chunk, ring > n_win
])
def test_window_attend(dtype, B, n_q, n_h, c, n_win, ring, ts):
    seed = 900 + c + ring
    q = synth.normal((B, n_q, n_h, c), seed, dtype=dtype)
    R = _ring(B, ring, c, dtype, seed + 1)
    t = torch.tensor(ts, dtype=torch.int64).reshape(B, n_q)
    o, lse = dlc.window_attend(q.to(DEV), R.to(DEV), t.to(DEV), int(t.max()), n_win)
    torch.cuda.synchronize()
    for b in range(B):
        for j in range(n_q):
            o_r, l_r = _window_ref(q[b, j], R[b], t[b, j], n_win)
            assert_rows_close(o[b, j], o_r, TOL_ATT[dtype], f"window b={b} q={j}")
            assert np.abs(lse[b, j].cpu().numpy() - l_r).max() <= TOL_ATT[dtype]


@pytest.mark.parametrize("dtype,B,n_h,c,k,cap,counts", [
    ("bf16", 4, 128, 512, 1024, 262208, [1024, 1024, 7, 0]),  # V4-Pro shape; one empty compressed part
    ("bf16", 2, 40, 512, 200, 3000, [200, 64]),              # c = 512, 40 heads: the merge with a partial head block
    ("f32", 2, 4, 16, 8, 40, [5, 8]),
])
def test_window_joins_compressed_branch_in_place(dtype, B, n_h, c, k, cap, counts):
    """csa_attend, then window_attend with the CSA output as o_in and out: the
    attention over the union of the selected entries and the window."""
    seed = 950 + c
    n_win, ring = 128, 128
    q = synth.normal((B, 1, n_h, c), seed, dtype=dtype)
    Cc = synth.normal((B, cap, c), seed + 1, dtype=dtype)
    R = _ring(B, ring, c, dtype, seed + 2)
    g = torch.Generator().manual_seed(seed + 3)
    idx = torch.full((B, 1, k), -1, dtype=torch.int32)
    for b, n in enumerate(counts):
        idx[b, 0, :n] = torch.sort(torch.randperm(cap, generator=g)[:n])[0].to(torch.int32)
    cnt = torch.tensor(counts, dtype=torch.int32).reshape(B, 1)
    t = torch.tensor([4 * cap + 3 + b for b in range(B)], dtype=torch.int64).reshape(B, 1)
    qd, Rd = q.to(DEV), R.to(DEV)
    o, lse = dlc.csa_attend(qd, Cc.to(DEV), idx.to(DEV), cnt.to(DEV))
    dlc.window_attend(qd, Rd, t.to(DEV), int(t.max()), n_win, o_in=o, lse_in=lse, out=o, lse=lse)
    torch.cuda.synchronize()
    for b in range(B):
        sel = idx[b, 0, :counts[b]].numpy().astype(np.int64)
        o1, l1 = O.csa_attend(q[b, 0], Cc[b], sel)
        o2, l2 = _window_ref(q[b, 0], R[b], t[b, 0], n_win)
        o_r, l_r = O.merge_lse(o1, l1, o2, l2)
        assert_rows_close(o[b, 0], o_r, TOL_ATT[dtype], f"joined b={b}")
        assert np.abs(lse[b, 0].cpu().numpy() - l_r).max() <= TOL_ATT[dtype]


@pytest.mark.parametrize("dtype,B,n_h,c,k,cap,counts,ring", [
    ("bf16", 4, 128, 512, 1024, 262208, [1024, 1024, 7, 0], 128),  # V4-Pro shape; one empty compressed part
    ("bf16", 2, 16, 128, 64, 2048, [64, 30], 200),                 # c = 128 MFMA path, ring > n_win
    ("f32", 2, 4, 16, 8, 40, [5, 8], 128),                          # VALU path
])
def test_csa_attend_window(dtype, B, n_h, c, k, cap, counts, ring):
    """One attention over the selected entries followed by the window: the
    oracle's merge of the two parts (pinned to the concatenated attention)."""
    seed = 970 + c
    n_win = 128
    q = synth.normal((B, 1, n_h, c), seed, dtype=dtype)
    Cc = synth.normal((B, cap, c), seed + 1, dtype=dtype)
    R = _ring(B, ring, c, dtype, seed + 2)
    g = torch.Generator().manual_seed(seed + 3)
    idx = torch.full((B, 1, k), -1, dtype=torch.int32)
    for b, n in enumerate(counts):
        idx[b, 0, :n] = torch.sort(torch.randperm(cap, generator=g)[:n])[0].to(torch.int32)
    cnt = torch.tensor(counts, dtype=torch.int32).reshape(B, 1)
    t = torch.tensor([4 * cap + 3 + 5 * b for b in range(B)], dtype=torch.int64).reshape(B, 1)
    t[-1, 0] = 60                                                   # a window shorter than n_win
    o, lse = dlc.csa_attend_window(q.to(DEV), Cc.to(DEV), idx.to(DEV), cnt.to(DEV), R.to(DEV), t.to(DEV),
                                   int(t.max()), n_win)
    torch.cuda.synchronize()
    for b in range(B):
        sel = idx[b, 0, :counts[b]].numpy().astype(np.int64)
        o1, l1 = O.csa_attend(q[b, 0], Cc[b], sel)
        o2, l2 = _window_ref(q[b, 0], R[b], t[b, 0], n_win)
        o_r, l_r = O.merge_lse(o1, l1, o2, l2)
        assert_rows_close(o[b, 0], o_r, TOL_ATT[dtype], f"csa+window b={b}")
        assert np.abs(lse[b, 0].cpu().numpy() - l_r).max() <= TOL_ATT[dtype]


@pytest.mark.parametrize("dtype,B,n_h,c,mp,cap,ts,ring", [
    ("bf16", 4, 128, 512, 128, 8194, [(1 << 20) + 3, (1 << 20) + 130, 200, 5], 384),  # HCA empty for t < m'
    ("f32", 2, 3, 8, 4, 30, [50, 2], 16),
])
def test_hca_attend_window(dtype, B, n_h, c, mp, cap, ts, ring):
    seed = 990 + c
    n_win = 128 if ring >= 128 else 16
    q = synth.normal((B, 1, n_h, c), seed, dtype=dtype)
    Ch = synth.normal((B, cap, c), seed + 1, dtype=dtype)
    R = _ring(B, ring, c, dtype, seed + 2)
    t = torch.tensor(ts, dtype=torch.int64).reshape(B, 1)
    o, lse = dlc.hca_attend_window(q.to(DEV), Ch.to(DEV), t.to(DEV), int(t.max()), mp, R.to(DEV), n_win)
    torch.cuda.synchronize()
    for b in range(B):
        o1, l1 = O.hca_attend(q[b, 0], Ch[b], int(t[b, 0]), mp)
        o2, l2 = _window_ref(q[b, 0], R[b], t[b, 0], n_win)
        o_r, l_r = O.merge_lse(o1, l1, o2, l2)
        assert_rows_close(o[b, 0], o_r, TOL_ATT[dtype], f"hca+window b={b}")
        assert np.abs(lse[b, 0].cpu().numpy() - l_r).max() <= TOL_ATT[dtype]


# ------------------------------------------------------------------ copy kernel

@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 48, (1 << 20) + 16 * 37])
def test_copy_kernel(nbytes):
    """dlc_copy moves every byte: one 16-byte element per thread and pass,
    ragged last block (the bandwidth reference also copies the benchmark's
    caches)."""
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
    buf = torch.full((nbytes + 4096,), 7, dtype=torch.uint8, device=DEV)
    dst = buf[:nbytes]                      # the bytes after it must stay untouched
    binding.dlc_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert (buf[nbytes:] == 7).all()
