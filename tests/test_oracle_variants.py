"""Pins of the oracle's page variants (no GPU).

* The [Evolution] derivation of the indexer key, k^I = c^comp W^I_k ("From
  MHA, GQA to MLA, DSA, HCA/CSA", §6.2): because an entry is a convex
  combination of its window's rows with column-wise softmax weights, the
  projection of an entry is NOT in general the compression of the projected
  rows (the weights differ per column), but it is when every column of the
  window shares one weight vector; both facts are checked, so the variant is
  pinned to the compressor rather than to itself.
* Sink logits ("DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch",
  §12 names them): the direct definition (one extra logit, zero value) is
  checked against the closed form applied to a finished attention, against
  the limits z -> -inf (no sink) and z -> +inf (all mass on the sink), and
  against SDPA with an explicit zero key/value row whose logit is forced.
"""

import math

import numpy as np
import torch

from oracle import dlc_oracle as o


def test_evolution_keys_equal_compressing_projected_rows_when_weights_are_shared():
    rng = np.random.default_rng(0)
    m, c, cI, n = 4, 16, 8, 32
    Ca, Cb = rng.standard_normal((n, c)), rng.standard_normal((n, c))
    # logits constant across columns: every column of a window shares one weight vector
    za, zb = rng.standard_normal((n, 1)), rng.standard_normal((n, 1))
    Za, Zb = np.repeat(za, c, axis=1), np.repeat(zb, c, axis=1)
    W = rng.standard_normal((c, cI))
    kI = o.evolution_indexer_keys(o.csa_compress(Za, Zb, Ca, Cb, m), W)
    Za2, Zb2 = np.repeat(za, cI, axis=1), np.repeat(zb, cI, axis=1)
    kI2 = o.csa_compress(Za2, Zb2, Ca @ W, Cb @ W, m)
    np.testing.assert_allclose(kI, kI2, rtol=1e-12, atol=1e-12)


def test_evolution_keys_differ_from_compressing_projected_rows_in_general():
    rng = np.random.default_rng(1)
    m, c, cI, n = 4, 16, 8, 32
    Za, Zb, Ca, Cb = (rng.standard_normal((n, c)) for _ in range(4))
    W = rng.standard_normal((c, cI))
    kI = o.evolution_indexer_keys(o.csa_compress(Za, Zb, Ca, Cb, m), W)
    # per-column weights do not commute with the projection: the pages' two derivations differ
    Z2a, Z2b = Za @ np.abs(W) / c, Zb @ np.abs(W) / c
    kI2 = o.csa_compress(Z2a, Z2b, Ca @ W, Cb @ W, m)
    assert np.abs(kI - kI2).max() > 1e-3


def test_evolution_queries_are_head_slices_of_one_projection():
    rng = np.random.default_rng(2)
    d, n_hI, cI = 24, 3, 8
    h = rng.standard_normal(d)
    W = rng.standard_normal((d, n_hI * cI))
    q = o.evolution_indexer_queries(h, W, n_hI, cI)
    for j in range(n_hI):
        np.testing.assert_allclose(q[j], h @ W[:, j * cI:(j + 1) * cI], rtol=1e-13)


def _case(seed, nh=4, n=9, c=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((nh, c)), rng.standard_normal((n, c)), rng.standard_normal(nh)


def test_sink_direct_equals_closed_form_on_finished_attention():
    q, KV, z = _case(3)
    o_s, l_s = o.mqa_attend_with_sink(q, KV, z)
    o0, l0 = o.mqa_attend(q, KV)
    o2, l2 = o.apply_sink(o0, l0, z)
    np.testing.assert_allclose(o_s, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l_s, l2, rtol=1e-12)


def test_sink_limits():
    q, KV, _ = _case(4)
    o0, l0 = o.mqa_attend(q, KV)
    o_lo, l_lo = o.mqa_attend_with_sink(q, KV, np.full(q.shape[0], -800.0))
    np.testing.assert_allclose(o_lo, o0, rtol=1e-12)
    np.testing.assert_allclose(l_lo, l0, rtol=1e-12)
    o_hi, l_hi = o.mqa_attend_with_sink(q, KV, np.full(q.shape[0], 800.0))
    assert np.abs(o_hi).max() < 1e-300 and np.allclose(l_hi, 800.0)


def test_sink_against_sdpa_with_a_zero_value_row():
    q, KV, z = _case(5, nh=3, n=7, c=8)
    c = q.shape[1]
    scale = 1.0 / math.sqrt(c)
    # one extra key row whose logit equals z_h for every head: key = z_h / scale * q_h / |q_h|^2 per head
    outs = []
    for h in range(q.shape[0]):
        qh = torch.tensor(q[h][None, None, None, :])
        key_sink = z[h] / scale * q[h] / (q[h] @ q[h])
        K = torch.tensor(np.concatenate([KV, key_sink[None]], 0)[None, None])
        V = torch.tensor(np.concatenate([KV, np.zeros((1, c))], 0)[None, None])
        outs.append(torch.nn.functional.scaled_dot_product_attention(qh, K, V, scale=scale)[0, 0, 0].numpy())
    o_s, _ = o.mqa_attend_with_sink(q, KV, z)
    np.testing.assert_allclose(o_s, np.stack(outs), rtol=1e-10, atol=1e-12)


def test_sink_on_an_empty_key_set():
    o2, l2 = o.apply_sink(np.zeros((2, 4)), np.full(2, -np.inf), np.array([0.5, -1.0]))
    assert (o2 == 0).all() and np.allclose(l2, [0.5, -1.0])
