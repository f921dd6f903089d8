"""The fused projection + pooling calls on the GPU.

csa_project_compress / hca_project_compress take hidden rows and the stream
weights and write the compressed caches in one pass.  Each case checks the
result twice: bit for bit against dlc_project of every stream followed by
csa_compress / hca_compress (the same arithmetic, so the same bits), and
against the oracle's compressor applied to the oracle's projections stored in
bf16, at the bf16-storage tolerance of the stage tests.
"""

import numpy as np
import pytest
import torch

import dense_long_context_amd as dlc
import oracle as O
import synth
from devtools import DEV, assert_rows_close, need_gpu

pytestmark = pytest.mark.gpu

TOL_STORE = 8e-3  # one bf16 rounding of an fp32 result (and of the streams), row-relative


def setup_module():
    need_gpu()


def _hidden(B, n, d, seed, ld=None):
    """H [B][n][d] bf16 as a view of a [B][n][ld] buffer (ld >= d)."""
    ld = ld or d
    full = synth.normal((B, n, ld), seed, dtype="bf16")
    return full[:, :, :d], full


def _weights(k, c, d, seed):
    return [synth.normal((c, d), seed + i, std=d ** -0.5, dtype="bf16") for i in range(k)]


def _unfused_streams(dH, dWs):
    """dlc_project of every stream: [B][n][c] bf16 each."""
    B, n, _ = dH.shape
    out = []
    for W in dWs:
        S = torch.empty((B, n, W.shape[0]), dtype=torch.bfloat16, device=DEV)
        for b in range(B):
            dlc.dlc_project(dH[b], W, out=S[b])
        out.append(S)
    return out


def _oracle_streams(H, Ws):
    """The oracle's projections, stored in bf16 as the device stores them."""
    return [np.stack([O.store_as(O.project(H[b], W.t()), "bf16") for b in range(H.shape[0])]) for W in Ws]


@pytest.mark.parametrize("B,n,d,c,m,ld,bias,rng", [
    (2, 1000, 256, 64, 4, 256, True, None),       # 8 row tiles of 31 entries, ragged last tile
    (1, 600, 128, 32, 4, 136, False, (37, 150)),  # strided rows, a range starting inside a tile
    (1, 515, 64, 128, 2, 64, True, None),         # m = 2: 63 entries a tile; four channel groups
    (2, 333, 128, 64, 8, 128, True, (0, 1)),      # m = 8, only entry 0 (no b-rows)
    (1, 4096, 512, 64, 1, 512, False, None),      # m = 1: 127 entries a tile
])
def test_csa_project_compress(B, n, d, c, m, ld, bias, rng):
    seed = 900 + n
    H, full = _hidden(B, n, d, seed, ld)
    Ws = _weights(4, c, d, seed + 10)
    Ba = synth.normal((m, c), seed + 20, dtype="f32") if bias else None
    Bb = synth.normal((m, c), seed + 21, dtype="f32") if bias else None
    if bias:
        Bb[m - 1, ::5] = -np.inf  # masked positions, the page's padding device
    i0, i1 = rng or (0, n // m)
    cap = n // m + 2
    dH = full.to(DEV)[:, :, :d]
    dWs = [W.to(DEV) for W in Ws]
    dBa = None if Ba is None else Ba.to(DEV)
    dBb = None if Bb is None else Bb.to(DEV)
    fused = torch.full((B, cap, c), 3.0, dtype=torch.bfloat16, device=DEV)
    dlc.csa_project_compress(dH, *dWs, m, fused, i0, i1, Ba=dBa, Bb=dBb)
    Za, Zb, Ca, Cb = _unfused_streams(dH, dWs)
    ref = torch.full((B, cap, c), 3.0, dtype=torch.bfloat16, device=DEV)
    dlc.csa_compress(Za, Zb, Ca, Cb, m, ref, i0, i1, dBa, dBb)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref), "the fused pass must equal dlc_project + csa_compress bit for bit"
    got = fused.cpu()
    oZa, oZb, oCa, oCb = _oracle_streams(H, Ws)
    for b in range(B):
        want = O.csa_compress(oZa[b], oZb[b], oCa[b], oCb[b], m, Ba, Bb, i0, i1)
        assert_rows_close(got[b, i0:i1], O.store_as(want, "bf16"), TOL_STORE, f"csa fused b={b}")
        assert (got[b, :i0].float() == 3.0).all() and (got[b, i1:].float() == 3.0).all(), "entries outside written"


@pytest.mark.parametrize("B,n,d,c,mp,bias", [
    (2, 1000, 256, 128, 128, True),   # 7 entries, one a tile, two channel groups
    (1, 700, 128, 64, 32, False),     # 4 entries a tile, ragged last tile
    (1, 300, 64, 64, 1, True),        # m' = 1: every row its own entry
])
def test_hca_project_compress(B, n, d, c, mp, bias):
    seed = 950 + n
    H, full = _hidden(B, n, d, seed)
    Ws = _weights(2, c, d, seed + 10)
    Bh = synth.normal((mp, c), seed + 20, dtype="f32") if bias else None
    cap = n // mp
    dH = full.to(DEV)
    dWs = [W.to(DEV) for W in Ws]
    dBh = None if Bh is None else Bh.to(DEV)
    fused = torch.empty((B, cap, c), dtype=torch.bfloat16, device=DEV)
    dlc.hca_project_compress(dH, *dWs, mp, fused, bias=dBh)
    Z, Cs = _unfused_streams(dH, dWs)
    ref = torch.empty_like(fused)
    dlc.hca_compress(Z, Cs, mp, ref, bias=dBh)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref), "the fused pass must equal dlc_project + hca_compress bit for bit"
    got = fused.cpu()
    oZ, oC = _oracle_streams(H, Ws)
    for b in range(B):
        want = O.hca_compress(oZ[b], oC[b], mp, Bh)
        assert_rows_close(got[b], O.store_as(want, "bf16"), TOL_STORE, f"hca fused b={b}")


def test_fused_decode8k_caches():
    """The decode8k layer's three caches (CSA entries, indexer keys, HCA
    entries over 8192 tokens, d = 1024) from the fused calls equal the
    two-pass build exactly."""
    cfg = synth.get_config("decode8k")
    n, d, c, cI, m, mp = cfg.t, cfg.d, cfg.c, cfg.cI, cfg.m, cfg.m_prime
    H, full = _hidden(1, n, d, 77)
    dH = full.to(DEV)
    for width, ratio, k, overlap in ((c, m, 4, True), (cI, m, 4, True), (c, mp, 2, False)):
        dWs = [W.to(DEV) for W in _weights(k, width, d, 700 + width + ratio)]
        cap = n // ratio
        fused = torch.empty((1, cap, width), dtype=torch.bfloat16, device=DEV)
        ref = torch.empty_like(fused)
        streams = _unfused_streams(dH, dWs)
        if overlap:
            dlc.csa_project_compress(dH, *dWs, ratio, fused)
            dlc.csa_compress(*streams, ratio, ref)
        else:
            dlc.hca_project_compress(dH, *dWs, ratio, fused)
            dlc.hca_compress(*streams, ratio, ref)
        torch.cuda.synchronize()
        assert torch.equal(fused, ref), f"width {width} ratio {ratio}"
