"""Pins of the oracle's sliding-window branch ([Evolution] §6.1 and §6.2):
the window set, the window attention against torch's SDPA, and the LSE merge
against one attention over the concatenated key sets, which is how the pages
join the window entries to the compressed ones."""

import numpy as np
import pytest
import torch

import oracle as O


@pytest.mark.parametrize("t,n_win,expect", [
    (0, 128, [0]),
    (5, 128, list(range(0, 6))),
    (127, 128, list(range(0, 128))),
    (128, 128, list(range(1, 129))),
    (1000, 4, [997, 998, 999, 1000]),
    (7, 1, [7]),
])
def test_window_positions(t, n_win, expect):
    assert O.window_positions(t, n_win).tolist() == expect


@pytest.mark.parametrize("n,t,n_win,nh,c", [(300, 299, 128, 4, 16), (50, 20, 128, 2, 8), (10, 9, 3, 3, 5)])
def test_window_attend_is_sdpa_over_recent_rows(n, t, n_win, nh, c):
    rng = np.random.default_rng(n + t)
    C = rng.standard_normal((n, c))
    q = rng.standard_normal((nh, c))
    o, lse = O.window_attend(q, C, t, n_win)
    lo = max(0, t - n_win + 1)
    K = torch.tensor(C[lo:t + 1])
    qt = torch.tensor(q)
    ref = torch.nn.functional.scaled_dot_product_attention(qt[None], K[None], K[None])[0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    logits = (q @ C[lo:t + 1].T) / np.sqrt(c)
    np.testing.assert_allclose(lse, np.log(np.exp(logits).sum(axis=1)), rtol=1e-12)


@pytest.mark.parametrize("trial", range(6))
def test_merge_equals_attention_over_concatenation(trial):
    rng = np.random.default_rng(100 + trial)
    nh, c = 3, 7
    A = rng.standard_normal((int(rng.integers(1, 20)), c)) * (1 + trial)
    Bk = rng.standard_normal((int(rng.integers(1, 20)), c))
    q = rng.standard_normal((nh, c))
    o1, l1 = O.mqa_attend(q, A)
    o2, l2 = O.mqa_attend(q, Bk)
    o, lse = O.merge_lse(o1, l1, o2, l2)
    oc, lc = O.mqa_attend(q, np.vstack([A, Bk]))
    np.testing.assert_allclose(o, oc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lc, rtol=1e-12)


def test_merge_with_empty_parts():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 4))
    o1, l1 = O.mqa_attend(q, rng.standard_normal((5, 4)))
    oe, le = O.mqa_attend(q, np.zeros((0, 4)))
    o, lse = O.merge_lse(o1, l1, oe, le)
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(lse, l1)
    o, lse = O.merge_lse(oe, le, o1, l1)
    np.testing.assert_allclose(o, o1, rtol=1e-15)
    o, lse = O.merge_lse(oe, le, oe, le)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_csa_with_window_is_one_attention_over_both_sets():
    # selected compressed entries and window entries, joined as the pages do
    rng = np.random.default_rng(11)
    nh, c, n, n_win, t = 4, 8, 64, 16, 63
    Ccomp = rng.standard_normal((n // 4, c))
    Cwin = rng.standard_normal((n, c))
    q = rng.standard_normal((nh, c))
    sel = np.array([1, 5, 9])
    o1, l1 = O.csa_attend(q, Ccomp, sel)
    o2, l2 = O.window_attend(q, Cwin, t, n_win)
    o, lse = O.merge_lse(o1, l1, o2, l2)
    oc, lc = O.mqa_attend(q, np.vstack([Ccomp[sel], Cwin[t - n_win + 1:t + 1]]))
    np.testing.assert_allclose(o, oc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lc, rtol=1e-12)
