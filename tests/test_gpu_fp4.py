"""FP4 (MXFP4) indexer on the GPU against the oracle.

mxfp4_quantize must reproduce the oracle's codes and block exponents bit for
bit (the encoding is integer work on exact inputs).  csa_index_topk_fp4's
scores are exact products summed in fp32, so they match the oracle's exact
fp64 scores on the dequantized operands within the fp32 accumulation bound;
the selected sets follow the tie rule of devtools.check_topk.
"""

import numpy as np
import pytest
import torch

import dense_long_context_amd as dlc
import oracle as O
import synth
from devtools import DEV, FlipTally, check_scores, check_topk, f64, need_gpu, score_bound

pytestmark = pytest.mark.gpu


def setup_module():
    need_gpu()


def unpack(codes, scales):
    """device bytes -> (codes 0..15 per element, block exponents)"""
    c = codes.cpu().numpy().astype(np.int64)
    el = np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[:-1] + (2 * c.shape[-1],))
    return el, scales.cpu().numpy().astype(np.int64) - 127


def _tie_rows(rng, rows, width):
    """rows built from the grid midpoints (exact ties) and grid values, times 2^e"""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 3.0, 6.0, 0.1, 7.5])
    x = rng.choice(mids, size=(rows, width)) * rng.choice([-1.0, 1.0], size=(rows, width))
    blocks = x.reshape(rows, width // 32, 32)
    blocks[..., 0] = 4.0                     # block max in [4, 8): exponent 0 before scaling
    return (blocks * np.exp2(rng.integers(-20, 20, size=(rows, width // 32, 1)))).reshape(rows, width)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,width", [(1, 32), (37, 128), (1000, 256), (3, 64)])
def test_mxfp4_quantize_bit_exact(dtype, rows, width):
    rng = np.random.default_rng(rows + width)
    x = rng.standard_normal((rows, width)) * np.exp2(rng.integers(-30, 30, size=(rows, 1)))
    x[0, :32] = 0.0                                       # an all-zero block
    if rows > 2:
        x[1] = _tie_rows(rng, 1, width)[0]                # exact midpoints
        x[2, :32] = 2.0 ** -126                           # block max below 2^-125: exponent clamps to -127
        x[2, 3] = 1.5 * 2.0 ** -126
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xt = torch.from_numpy(x).to(tdt)
    codes, scales = dlc.mxfp4_quantize(xt.to(DEV))
    torch.cuda.synchronize()
    got_c, got_e = unpack(codes, scales)
    ref_c, ref_e = O.mxfp4_quantize(f64(xt))
    assert np.array_equal(got_e, ref_e)
    assert np.array_equal(got_c, ref_c)


def test_mxfp4_quantize_cache_ranges_and_batches():
    # a [B][cap][cI] cache quantized in two row ranges through the raw ABI
    B, cap, cI = 3, 50, 128
    K = synth.normal((B, cap, cI), 21, dtype="bf16")
    Kd = K.to(DEV)
    codes = torch.zeros((B, cap, cI // 2), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((B, cap, cI // 32), dtype=torch.uint8, device=DEV)
    L = dlc.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for r0, r1 in ((0, 17), (17, cap)):
        rc = L.mxfp4_quantize(1, B, r1 - r0, cI, Kd.data_ptr() + r0 * cI * 2, cap * cI,
                              codes.data_ptr() + r0 * cI // 2, cap * cI // 2,
                              scales.data_ptr() + r0 * cI // 32, cap * cI // 32, stream)
        assert rc == 0
    torch.cuda.synchronize()
    got_c, got_e = unpack(codes, scales)
    ref_c, ref_e = O.mxfp4_quantize(f64(K))
    assert np.array_equal(got_e, ref_e) and np.array_equal(got_c, ref_c)


def _bound_fp4(qI, wI, KI):
    """fp32 bound of the device scores, on the dequantized operands"""
    return score_bound(O.mxfp4_dequantize(*O.mxfp4_quantize(qI)), wI, O.mxfp4_dequantize(*O.mxfp4_quantize(KI)))


@pytest.mark.parametrize("dtype,B,n_q,n_hI,cI,m,k,cap,ts", [
    ("bf16", 2, 3, 64, 128, 4, 100, 5000, [20000, 19999, 4, 333, 8000, 0]),   # ragged, 1 and 0 visible
    ("bf16", 1, 1, 64, 128, 4, 1024, 70000, [280000]),                        # many chunks
    ("f32", 1, 2, 20, 256, 2, 300, 4000, [8000, 7777]),                       # head padding, c^I = 256
    ("bf16", 1, 2, 16, 128, 4, 1024, 1500, [6000, 4100]),                     # k >= visible for one query
])
def test_index_topk_fp4(dtype, B, n_q, n_hI, cI, m, k, cap, ts):
    seed = 900 + cap
    qI = synth.normal((B, n_q, n_hI, cI), seed, dtype=dtype)
    wI = synth.normal((B, n_q, n_hI), seed + 1, dtype="f32")
    KI = synth.normal((B, cap, cI), seed + 2, dtype="bf16")
    KIc, KIs = dlc.mxfp4_quantize(KI.to(DEV))
    t = torch.tensor(ts, dtype=torch.int64).reshape(B, n_q)
    t_max = int(t.max())
    scores = torch.full((B, n_q, cap), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt = dlc.csa_index_topk_fp4(qI.to(DEV), wI.to(DEV), KIc, KIs, t.to(DEV), t_max, m, k, scores=scores)
    torch.cuda.synchronize()
    idx, cnt, sc = idx.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy()
    tally = FlipTally(f"index_topk_fp4 cap={cap}")
    for b in range(B):
        for j in range(n_q):
            tt = int(t[b, j])
            ref = O.index_scores_fp4(qI[b, j], wI[b, j], KI[b], tt, m)
            nv = len(ref)
            if nv:
                check_scores(sc[b, j, :nv], ref, _bound_fp4(qI[b, j], wI[b, j], KI[b, :nv]), f"scores b={b} q={j}")
            tally.add(check_topk(idx[b, j], cnt[b, j], ref, k, dev_scores=sc[b, j, :nv]))
    tally.report()


@pytest.mark.parametrize("B,n_q,n_hI,m,k,cap,seed", [
    (2, 100, 64, 4, 100, 3000, 1),      # two query tiles (64 + 36), mixed visibilities
    (1, 64, 20, 2, 50, 700, 2),         # 20 heads: a head group padded at zero weight
    (2, 66, 64, 4, 200, 1001, 4),       # cap % 4 != 0: score rows not 16-byte aligned
    (1, 64, 64, 4, 700, 66000, 5),      # three ranges of 32768 entries folded into a running top-k
])
def test_index_topk_fp4_prefill(B, n_q, n_hI, m, k, cap, seed):
    """Many queries per sequence: the query-tiled FP4 kernel (32x32x64 MXFP4
    MFMA) against the oracle's FP4 scores, every query."""
    cI = 128
    qI = synth.normal((B, n_q, n_hI, cI), 950 + seed, dtype="bf16")
    wI = synth.normal((B, n_q, n_hI), 951 + seed, dtype="f32")
    KI = synth.normal((B, cap, cI), 952 + seed, dtype="bf16")
    KIc, KIs = dlc.mxfp4_quantize(KI.to(DEV))
    rng = np.random.default_rng(seed)
    t = torch.from_numpy(rng.integers(0, m * cap + 1, size=(B, n_q))).to(torch.int64)
    t[0, 0], t[0, 1] = 0, m * cap
    t_max = int(t.max())
    scores = torch.full((B, n_q, cap), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt = dlc.csa_index_topk_fp4(qI.to(DEV), wI.to(DEV), KIc, KIs, t.to(DEV), t_max, m, k, scores=scores)
    torch.cuda.synchronize()
    idx, cnt, sc = idx.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy()
    Kd = [O.mxfp4_dequantize(*O.mxfp4_quantize(KI[b])) for b in range(B)]
    tally = FlipTally(f"index_topk_fp4 prefill seed={seed}")
    for b in range(B):
        for j in range(n_q):
            tt = int(t[b, j])
            nv = tt // m
            qd = O.mxfp4_dequantize(*O.mxfp4_quantize(qI[b, j]))
            ref = O.index_scores(qd, wI[b, j], Kd[b], tt, m)
            check_scores(sc[b, j, :nv], ref, score_bound(qd, wI[b, j], Kd[b][:nv]), f"scores b={b} q={j}")
            assert np.isnan(sc[b, j, nv:]).all(), f"entries past the visible range written b={b} q={j}"
            tally.add(check_topk(idx[b, j], cnt[b, j], ref, k, dev_scores=sc[b, j, :nv]))
    tally.report()


def test_index_topk_fp4_ties_pick_smallest_indices():
    # zero keys: every score is 0, so the k smallest indices win, in order
    B, cap, k = 1, 3000, 100
    qI = synth.normal((B, 1, 64, 128), 1, dtype="bf16")
    wI = synth.normal((B, 1, 64), 2, dtype="f32")
    KIc, KIs = dlc.mxfp4_quantize(torch.zeros((B, cap, 128), dtype=torch.bfloat16, device=DEV))
    t = torch.tensor([[4 * cap]])
    idx, cnt = dlc.csa_index_topk_fp4(qI.to(DEV), wI.to(DEV), KIc, KIs, t.to(DEV), 4 * cap, 4, k)
    assert int(cnt[0, 0]) == k
    assert idx[0, 0].cpu().tolist() == list(range(k))


def test_index_topk_fp4_nothing_visible():
    qI = synth.normal((2, 1, 4, 128), 3, dtype="bf16")
    wI = synth.normal((2, 1, 4), 4, dtype="f32")
    KIc, KIs = dlc.mxfp4_quantize(synth.normal((2, 10, 128), 5, dtype="bf16").to(DEV))
    t = torch.tensor([[3], [0]])
    idx, cnt = dlc.csa_index_topk_fp4(qI.to(DEV), wI.to(DEV), KIc, KIs, t.to(DEV), 3, 4, 8)
    assert cnt.cpu().tolist() == [[0], [0]]
    assert (idx.cpu() == -1).all()


def test_index_topk_fp4_unstaged_waves():
    """3.2M visible entries: every wave of the FP4 decode scores kernel has 65
    tiles, past the 64 whose scores it keeps in LDS, so it stores each tile's
    scores as they come.  The selection must equal the rule applied to the
    device's own scores exactly; the scores of 20000 sampled entries are
    checked against the oracle (the oracle's quantizer over all 3.2M rows
    would take minutes)."""
    B, n_q, n_hI, cI, m, k, cap = 1, 1, 64, 128, 4, 1024, 3200000
    t_q = 4 * cap
    qI = synth.normal((B, n_q, n_hI, cI), 990, dtype="bf16")
    wI = synth.normal((B, n_q, n_hI), 991, dtype="f32")
    KI = synth.normal((B, cap, cI), 992, dtype="bf16")
    KIc, KIs = dlc.mxfp4_quantize(KI.to(DEV))
    t = torch.tensor([[t_q]], dtype=torch.int64)
    scores = torch.full((B, n_q, cap), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt = dlc.csa_index_topk_fp4(qI.to(DEV), wI.to(DEV), KIc, KIs, t.to(DEV), t_q, m, k, scores=scores)
    torch.cuda.synchronize()
    idx, cnt, sc = idx.cpu().numpy(), cnt.cpu().numpy(), scores.cpu().numpy()
    assert np.isfinite(sc[0, 0]).all(), "every visible entry's score is written"
    rows = np.sort(np.random.default_rng(3).choice(cap, 20000, replace=False))
    Ks = KI[0, rows]
    ref = O.index_scores_fp4(qI[0, 0], wI[0, 0], Ks, 4 * len(rows), m)
    check_scores(sc[0, 0, rows], ref, _bound_fp4(qI[0, 0], wI[0, 0], Ks), "sampled fp4 scores")
    exact = O.topk_select(sc[0, 0], k)
    assert int(cnt[0, 0]) == k and np.array_equal(idx[0, 0], exact)
