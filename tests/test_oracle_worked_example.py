"""Pin the oracle to the hand-traced six-token example of the page
"DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch" (§3-§10).

Printed values (three decimals) are compared at abs 2.5e-3; closed forms
derived from the same example at 1e-12 relative.
"""

import math

import numpy as np
import pytest

import oracle as O

E = math.e
PRINTED = 2.5e-3


def _w(golden):
    w = {k: np.array(v, dtype=np.float64) for k, v in golden["weights"].items()
         if not k.startswith("_") and not k.endswith("_reuses")}
    return w


def _streams(golden):
    H = np.array(golden["setup"]["H"], dtype=np.float64)
    w = _w(golden)
    return H, {s: O.project(H, w[n]) for s, n in
               (("Ca", "aKV"), ("Cb", "bKV"), ("Za", "aZ"), ("Zb", "bZ"))}


def test_streams_match_printed(golden):
    _, st = _streams(golden)
    for name in ("Ca", "Cb", "Za", "Zb"):
        np.testing.assert_array_equal(st[name], np.array(golden["streams"][name], dtype=float))


def test_csa_weights_printed_and_closed_form(golden):
    _, st = _streams(golden)
    m = golden["setup"]["m"]
    g = golden["csa_weights"]
    for i in (0, 1):
        Sa, Sb = O.csa_window_weights(st["Za"], st["Zb"], m, i)
        for col in (0, 1):
            got = np.concatenate([Sa[:, col], Sb[:, col]])
            np.testing.assert_allclose(got, g[f"block{i}_col{col}"], atol=PRINTED)
            assert abs(got.sum() - 1.0) < 1e-12
    # closed forms
    Sa, Sb = O.csa_window_weights(st["Za"], st["Zb"], m, 0)
    np.testing.assert_allclose(np.concatenate([Sa[:, 0], Sb[:, 0]]),
                               [E / (E + 1), 1 / (E + 1), 0, 0], rtol=1e-12)
    Sa, Sb = O.csa_window_weights(st["Za"], st["Zb"], m, 1)
    den = 2 * E * E + E + 1
    np.testing.assert_allclose(np.concatenate([Sa[:, 0], Sb[:, 0]]),
                               [E * E / den, E / den, 1 / den, E * E / den], rtol=1e-12)


def test_csa_entries_printed_and_closed_form(golden):
    _, st = _streams(golden)
    m = golden["setup"]["m"]
    C = O.csa_compress(st["Za"], st["Zb"], st["Ca"], st["Cb"], m)
    assert C.shape == (3, 2)  # n/m = 3 entries
    np.testing.assert_allclose(C[0], golden["csa_entries"]["C0"], atol=PRINTED)
    np.testing.assert_allclose(C[1], golden["csa_entries"]["C1"], atol=PRINTED)
    np.testing.assert_allclose(C[0], [E / (E + 1), 1.0], rtol=1e-12)
    np.testing.assert_allclose(C[1], [(4 * E * E + E) / (2 * E * E + E + 1), 0.75], rtol=1e-12)
    # C_2 is "analogous" on the page: a-rows 4,5 and b-rows 2,3
    np.testing.assert_allclose(C[2], [3 * E / (1 + 3 * E), 1.0], rtol=1e-12)


def test_indexer_and_topk_printed(golden):
    s, w, ix = golden["setup"], _w(golden), golden["indexer"]
    H = np.array(s["H"], dtype=float)
    Q = O.queries_from_hidden(H[s["t"]], w["DQ"], w["IUQ"], w["w"], w["UQ"], w["UQ"],
                              s["n_h"], s["c"], s["n_hI"], s["cI"])
    np.testing.assert_array_equal(Q["cQ"], ix["cQ"])
    np.testing.assert_array_equal(Q["qI"][0], ix["qI"])
    assert Q["wI"][0] == ix["wI"]
    KI = np.array(ix["KI_assumed"])
    sc = O.index_scores(Q["qI"], Q["wI"], KI, s["t"], s["m"])
    assert O.csa_visible(s["t"], s["m"]) == ix["visible"]
    np.testing.assert_allclose(sc, ix["scores"], rtol=1e-15)
    np.testing.assert_array_equal(O.topk_select(sc, s["k"]), ix["top1"])


def test_full_chain_outputs(golden):
    s, w = golden["setup"], _w(golden)
    H = np.array(s["H"], dtype=float)
    W = dict(aKV=w["aKV"], bKV=w["bKV"], aZ=w["aZ"], bZ=w["bZ"],
             IaKV=w["aKV"], IbKV=w["bKV"], IaZ=w["aZ"], IbZ=w["bZ"],
             KV=w["aKV"], Z=w["aZ"], DQ=w["DQ"], IUQ=w["IUQ"], w=w["w"], UQ=w["UQ"],
             UQ_hca=w["UQ"])
    r = O.decode_chain(H, W, s["t"], s["m"], s["m_prime"], s["k"], s["n_h"], s["c"],
                       s["n_hI"], s["cI"], KI_override=golden["indexer"]["KI_assumed"])
    np.testing.assert_array_equal(r["idx"], [1])
    # k = 1: a softmax over one key is [1], so the output is the value itself (§8)
    np.testing.assert_allclose(r["o_csa"][0], golden["csa_output"]["o"], atol=PRINTED)
    np.testing.assert_allclose(r["o_csa"][0], r["Ccomp"][1], rtol=1e-15)
    np.testing.assert_allclose(r["Chca"][0], golden["hca"]["C0"], atol=PRINTED)
    np.testing.assert_allclose(r["o_hca"][0], golden["hca"]["o"], atol=PRINTED)
    np.testing.assert_allclose(r["o_hca"][0], r["Chca"][0], rtol=1e-15)
    # the lse of a one-key softmax is that key's scaled logit
    q = r["q"][0]
    np.testing.assert_allclose(r["lse_csa"][0], q @ r["Ccomp"][1] / math.sqrt(2), rtol=1e-15)


def test_hca_printed_and_closed_form(golden):
    H = np.array(golden["setup"]["H"], dtype=float)
    w, g = _w(golden), golden["hca"]
    mp = golden["setup"]["m_prime"]
    C, Z = O.project(H, w["aKV"]), O.project(H, w["aZ"])  # the page reuses W^{aKV}, W^{aZ}
    S0 = O.hca_window_weights(Z, mp, 0)
    np.testing.assert_allclose(S0[:, 0], g["block0_col0"], atol=PRINTED)
    np.testing.assert_allclose(S0[:, 1], g["block0_col1"], rtol=1e-12)
    S1 = O.hca_window_weights(Z, mp, 1)
    np.testing.assert_allclose(S1[:, 0], g["block1_col0"], atol=PRINTED)
    Ch = O.hca_compress(Z, C, mp)
    assert Ch.shape == (2, 2)
    np.testing.assert_allclose(Ch[0], g["C0"], atol=PRINTED)
    np.testing.assert_allclose(Ch[1], g["C1"], atol=PRINTED)
    np.testing.assert_allclose(Ch[0], [(E + 2 * E * E) / (1 + E + E * E), 1.0], rtol=1e-12)
    np.testing.assert_allclose(Ch[1], [2 * E / (2 * E + 1), 2.0 / 3.0], rtol=1e-12)
    assert O.hca_visible(golden["setup"]["t"], mp) == g["visible"]


@pytest.mark.parametrize("t,m,expect", [(5, 2, 2), (3, 2, 1), (1, 2, 0), (8192, 4, 2048),
                                        (5, 3, 1), (2, 3, 0), (1 << 20, 128, 8192)])
def test_visibility(t, m, expect):
    assert O.csa_visible(t, m) == expect == O.hca_visible(t, m)
