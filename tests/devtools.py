"""Helpers shared by the GPU parity tests: device inputs and comparisons."""

import numpy as np
import pytest
import torch

import oracle as O

DEV = "cuda:0"

# unit roundoff of fp32 with round-to-nearest
U_F32 = 2.0 ** -24


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def f64(x):
    return O.f64(x)


def row_rel_err(got, ref):
    """max over rows of max_j |got - ref| / max_j |ref| (rows = all but the last axis)."""
    g = f64(got).reshape(-1, np.shape(ref)[-1])
    r = f64(ref).reshape(-1, np.shape(ref)[-1])
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max()) if r.size else 0.0


def assert_rows_close(got, ref, tol, what=""):
    err = row_rel_err(got, ref)
    assert err <= tol, f"{what}: row-relative error {err:.3e} > {tol:.1e}"
    return err


def score_bound(qI, wI, KI):
    """Per-entry bound on the fp32 rounding error of the device indexer scores.

    I_s = sum_h w_h ReLU(sum_j q_hj K_sj) ("DeepSeek-V4 Hybrid Attention: CSA
    and HCA from Scratch", §6.4).  The operands are bf16 (or MXFP4, decoded to
    exact values), so every product q_hj K_sj is exact in fp32; the c^I-term
    dot product, the weight product and the n_h^I-term head sum are rounded in
    fp32.  The recursive-summation bound then gives, to first order in u,
        |I_dev - I| <= (n_h^I + c^I) u sum_h |w_h| sum_j |q_hj| |K_sj|,
    u = 2^-24, whatever order the sums take.  qI [n_hI][cI], wI [n_hI],
    KI [n][cI]; returns [n]."""
    q, w, K = f64(qI), f64(wI), f64(KI)
    n_h, c = q.shape
    mag = np.abs(K) @ np.abs(q).T @ np.abs(w)
    return (n_h + c) * U_F32 * mag + 1e-30


def check_scores(got, ref, bound, what=""):
    """Every device score within its arithmetic bound of the oracle's."""
    g, r = f64(got), f64(ref)
    bad = np.flatnonzero(np.abs(g - r) > bound)
    assert bad.size == 0, (f"{what}: {bad.size} scores beyond the fp32 bound, first at {bad[:4]}: "
                           f"got {g[bad[:4]]}, want {r[bad[:4]]}, bound {np.asarray(bound)[bad[:4]]}")


def check_topk(idx_row, count, scores_ref, k, rel_tie=1e-4, dev_scores=None):
    """Top-k parity for one query, at the target tie band (1e-4 relative at s_k).

    The device set must have k_eff = min(k, n) members, ascending, distinct,
    each visible, padded with -1.  It must equal the oracle's set (score
    descending, then index ascending), except that a member of the symmetric
    difference is accepted when its oracle score lies within rel_tie * |s_k| of
    the oracle's k-th score s_k (for s_k = 0, only an exact zero).  Returns the
    size of the symmetric difference (the flips), which is also checked against
    the number of oracle entries inside that band.

    dev_scores (the device's own fp32 scores of the same query, when the call
    returned them): the selection is an integer decision on those fp32 keys,
    so the device set must then equal the selection rule applied to them,
    exactly.
    """
    n = len(scores_ref)
    k_eff = min(k, n)
    assert count == k_eff, f"count {count} != k_eff {k_eff}"
    got = np.asarray(idx_row[:k_eff], dtype=np.int64)
    assert (np.asarray(idx_row[k_eff:]) == -1).all(), "padding must be -1"
    if k_eff == 0:
        return 0
    assert (np.diff(got) > 0).all(), "indices must be ascending and distinct"
    assert got.min() >= 0 and got.max() < n, "index outside the visible range"
    if dev_scores is not None:
        exact = O.topk_select(np.asarray(dev_scores, dtype=np.float32), k)
        assert np.array_equal(got, exact), "the set differs from the selection rule on the device's own scores"
    want = O.topk_select(scores_ref, k)
    diff = np.setxor1d(got, want)
    if diff.size == 0:
        return 0
    s = f64(scores_ref)
    sk = np.sort(s)[::-1][k_eff - 1]
    band = rel_tie * max(abs(sk), 1e-30)
    bad = diff[np.abs(s[diff] - sk) > band]
    assert bad.size == 0, (f"{bad.size} selected entries differ beyond the tie band {band:.3e} at "
                           f"s_k={sk:.6e}: {bad[:8]} (scores {s[bad[:8]]})")
    in_band = int(np.count_nonzero(np.abs(s - sk) <= band))
    assert diff.size <= in_band, f"{diff.size} flips but only {in_band} entries inside the tie band"
    return int(diff.size)


class FlipTally:
    """Top-k flips over the queries of one test (each flip already inside the
    tie band); the test prints the total and asserts it."""

    def __init__(self, what):
        self.what, self.flips, self.queries = what, 0, 0

    def add(self, flips):
        self.flips += int(flips)
        self.queries += 1

    def report(self, max_flips=None):
        print(f"[top-k] {self.what}: {self.flips} flips inside the tie band over {self.queries} queries", flush=True)
        if max_flips is not None:
            assert self.flips <= max_flips, f"{self.what}: {self.flips} flips > {max_flips}"
        return self.flips
