"""Helpers shared by the GPU parity tests: device inputs and comparisons."""

import numpy as np
import pytest
import torch

import oracle as O

DEV = "cuda:0"


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


def check_topk(idx_row, count, scores_ref, k, rel_tie=1e-4, abs_slack=None):
    """Top-k parity for one query (R9 of the design notes).

    The device set must have k_eff = min(k, n) members, ascending, distinct,
    each visible, padded with -1.  It must equal the oracle's set, except that
    members of the symmetric difference may differ when their oracle scores lie
    within rel_tie * |s_k| (+ abs_slack, the scores' arithmetic error bound) of
    the oracle's k-th score s_k.
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
    want = O.topk_select(scores_ref, k)
    diff = np.setxor1d(got, want)
    if diff.size == 0:
        return 0
    s = f64(scores_ref)
    sk = np.sort(s)[::-1][k_eff - 1]
    slack = rel_tie * max(abs(sk), 1e-30) + (abs_slack if abs_slack is not None else 0.0)
    bad = diff[np.abs(s[diff] - sk) > slack]
    assert bad.size == 0, f"{bad.size} selected entries differ beyond the tie band: {bad[:8]}"
    return int(diff.size)
