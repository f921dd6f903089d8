"""Page variants on the GPU against the oracle.

* Sink logits (attend_sink): applied to the outputs of hca_attend and
  csa_attend, compared with the oracle's direct definition (one extra logit
  with a zero value), including a query that sees no entry.
* The [Evolution] derivation of the indexer inputs: keys projected from the
  device's compressed entries with dlc_project, queries projected from hidden
  states, then csa_index_topk; stage-wise, each stage against the oracle on
  the device's stored inputs.
"""

import numpy as np
import pytest
import torch

import dense_long_context_amd as dlc
import oracle as O
import synth
from devtools import DEV, assert_rows_close, check_topk, f64, need_gpu

pytestmark = pytest.mark.gpu


def setup_module():
    need_gpu()


@pytest.mark.parametrize("B,n_h,c,mp,cap,ts", [
    (2, 128, 512, 128, 300, [300 * 128, 100]),     # the second query sees nothing
    (1, 16, 128, 4, 50, [150]),
])
def test_attend_sink_on_hca(B, n_h, c, mp, cap, ts):
    q = synth.normal((B, 1, n_h, c), 61, dtype="bf16")
    C = synth.normal((B, cap, c), 62, dtype="bf16")
    z = synth.normal((n_h,), 63, std=3.0, dtype="f32")
    t = torch.tensor(ts, dtype=torch.int64).reshape(B, 1)
    out, lse = dlc.hca_attend(q.to(DEV), C.to(DEV), t.to(DEV), int(t.max()), mp)
    dlc.attend_sink(out, lse, z.to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        nv = min(int(t[b, 0]) // mp, cap)
        o_r, l_r = O.mqa_attend_with_sink(q[b, 0], C[b, :nv], z)
        assert_rows_close(out[b, 0].cpu(), o_r, 2e-2, f"sink b={b}")
        np.testing.assert_allclose(lse[b, 0].cpu().numpy(), l_r, rtol=2e-2, atol=2e-2)


def test_attend_sink_on_csa_fp32():
    B, n_h, c, cap, k = 2, 3, 8, 40, 6
    q = synth.normal((B, 2, n_h, c), 71, dtype="f32")
    C = synth.normal((B, cap, c), 72, dtype="f32")
    z = synth.normal((n_h,), 73, dtype="f32")
    idx = torch.tensor([[[0, 3, 9, 20, 33, 39], [1, 2, -1, -1, -1, -1]],
                        [[5, 6, 7, 8, 9, 10], [0, -1, -1, -1, -1, -1]]], dtype=torch.int32)
    cnt = torch.tensor([[6, 2], [6, 0]], dtype=torch.int32)
    out, lse = dlc.csa_attend(q.to(DEV), C.to(DEV), idx.to(DEV), cnt.to(DEV))
    dlc.attend_sink(out, lse, z.to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        for j in range(2):
            sel = idx[b, j, :int(cnt[b, j])].numpy().astype(np.int64)
            o_r, l_r = O.mqa_attend_with_sink(q[b, j], C[b, sel], z)
            assert_rows_close(out[b, j].cpu(), o_r, 1e-5, f"sink csa b={b} j={j}")
            np.testing.assert_allclose(lse[b, j].cpu().numpy(), l_r, rtol=1e-5, atol=1e-5)


def test_evolution_indexer_inputs():
    B, n, c, cI, m, n_hI, d, k = 2, 2048, 512, 128, 4, 64, 256, 64
    seed = 80
    full = synth.normal((4, B, n, c), seed, std=2.0, dtype="bf16")
    Za, Zb, Ca, Cb = (full[i] for i in range(4))
    dfull = full.to(DEV)
    cap = n // m
    Cc = torch.empty((B, cap, c), dtype=torch.bfloat16, device=DEV)
    dlc.csa_compress(dfull[0], dfull[1], dfull[2], dfull[3], m, Cc)
    W_k = synth.normal((c, cI), seed + 1, std=c ** -0.5, dtype="bf16")
    W_q = synth.normal((d, n_hI * cI), seed + 2, std=d ** -0.5, dtype="bf16")
    h = synth.normal((B, d), seed + 3, dtype="bf16")
    w = synth.normal((B, 1, n_hI), seed + 4, dtype="f32")
    KI = dlc.dlc_project(Cc.reshape(B * cap, c), W_k.t().contiguous().to(DEV)).reshape(B, cap, cI)
    qI = dlc.dlc_project(h.to(DEV), W_q.t().contiguous().to(DEV)).reshape(B, 1, n_hI, cI)
    t = torch.tensor([[n], [n - 37]], dtype=torch.int64)
    idx, cnt = dlc.csa_index_topk(qI, w.to(DEV), KI, t.to(DEV), n, m, k)
    torch.cuda.synchronize()
    for b in range(B):
        # the entries themselves, then each projection on the device's stored inputs
        assert_rows_close(Cc[b].cpu(), O.store_as(O.csa_compress(Za[b], Zb[b], Ca[b], Cb[b], m), "bf16"), 8e-3,
                          f"entries b={b}")
        kI_ref = O.store_as(O.evolution_indexer_keys(Cc[b].cpu(), W_k), "bf16")
        assert_rows_close(KI[b].cpu(), kI_ref, 8e-3, f"keys b={b}")
        qI_ref = O.store_as(O.evolution_indexer_queries(h[b], W_q, n_hI, cI), "bf16")
        assert_rows_close(qI[b, 0].cpu(), qI_ref, 8e-3, f"queries b={b}")
        tt = int(t[b, 0])
        ref = O.index_scores(qI[b, 0].cpu(), w[b, 0], KI[b].cpu(), tt, m)
        check_topk(idx[b, 0].cpu().numpy().astype(np.int64), int(cnt[b, 0]), ref, k)
