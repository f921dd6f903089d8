"""Pin the oracle with invariants, closed forms, special cases that reduce to
a library routine, and brute force on tiny inputs.

Each test names the passage of "DeepSeek-V4 Hybrid Attention: CSA and HCA
from Scratch" ([Scratch]) that fixes the property.  Together they fail on
the plausible slips: a dropped b-stream term, a separate instead of joint
softmax, a wrong block offset, bias indexed by token instead of position,
a missing ReLU or scale, a transposed operand, an off-by-one visibility.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(12345)


def _streams(n, c, scale=1.0, rng=RNG):
    return [rng.standard_normal((n, c)) * scale for _ in range(4)]


# ---------------------------------------------------------------- compressor

@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_csa_weights_sum_to_one_and_nonnegative(m):
    Za, Zb, _, _ = _streams(6 * m, 5, 3.0)
    for i in range(6):
        Sa, Sb = O.csa_window_weights(Za, Zb, m, i)
        np.testing.assert_allclose(Sa.sum(0) + Sb.sum(0), 1.0, rtol=1e-14)  # [Scratch] §4 check
        assert (Sa >= 0).all() and (Sb >= 0).all()
        if i == 0:
            assert (Sb == 0).all()  # padded positions get exactly 0 (exp(-inf))


@pytest.mark.parametrize("m", [2, 4])
def test_csa_output_is_convex_combination(m):
    # [Scratch] §5 range check: each coordinate lies within the window's min/max
    Za, Zb, Ca, Cb = _streams(8 * m, 7, 2.0)
    C = O.csa_compress(Za, Zb, Ca, Cb, m)
    for i in range(8):
        vals = Ca[m * i:m * (i + 1)] if i == 0 else np.vstack([Ca[m * i:m * (i + 1)], Cb[m * (i - 1):m * i]])
        assert (C[i] >= vals.min(0) - 1e-12).all() and (C[i] <= vals.max(0) + 1e-12).all()


def test_csa_constant_logits_give_window_mean():
    # [Scratch] §4: all-equal logits give uniform weights 1/(2m) (1/m for i = 0)
    m, n, c = 4, 32, 6
    _, _, Ca, Cb = _streams(n, c)
    Z = np.full((n, c), 0.7)
    C = O.csa_compress(Z, Z, Ca, Cb, m)
    np.testing.assert_allclose(C[0], Ca[:m].mean(0), rtol=1e-13)
    for i in range(1, n // m):
        ref = (Ca[m * i:m * (i + 1)].sum(0) + Cb[m * (i - 1):m * i].sum(0)) / (2 * m)
        np.testing.assert_allclose(C[i], ref, rtol=1e-13, atol=1e-15)


def test_csa_shift_invariance():
    # one softmax per column: adding the same constant to every logit changes nothing
    m = 4
    Za, Zb, Ca, Cb = _streams(40, 3)
    C0 = O.csa_compress(Za, Zb, Ca, Cb, m)
    C1 = O.csa_compress(Za + 11.5, Zb + 11.5, Ca, Cb, m)
    np.testing.assert_allclose(C0, C1, rtol=1e-12, atol=1e-14)


def test_csa_joint_softmax_not_separate():
    # raising only the b-logits moves weight from the a-block to the b-block; with two
    # separate block softmaxes it would change nothing.  (The printed block-1 weights of
    # [Scratch] §4 already sum to one jointly; this pins the same reading on random data.)
    m = 2
    Za, Zb, Ca, Cb = _streams(8, 3)
    Cb = Cb + 10.0
    lo = O.csa_compress(Za, Zb, Ca, Cb, m)
    hi = O.csa_compress(Za, Zb + 5.0, Ca, Cb, m)
    assert (hi[1:] > lo[1:]).all()
    np.testing.assert_allclose(hi[0], lo[0], rtol=1e-14)  # entry 0 has no b-rows


def test_csa_m1_with_excluded_b_is_identity():
    # m = 1 and B^b = -inf leave a one-element softmax over the a-row: C^Comp_i = C^a_i
    Za, Zb, Ca, Cb = _streams(9, 4)
    C = O.csa_compress(Za, Zb, Ca, Cb, 1, Ba=np.zeros((1, 4)), Bb=np.full((1, 4), -np.inf))
    np.testing.assert_allclose(C, Ca, rtol=0, atol=0)


def test_csa_b_rows_come_from_previous_block():
    # with the a-block silenced (B^a = -inf) entry i is a softmax over b-rows m(i-1)..mi-1 only
    m, c = 3, 4
    Za, Zb, Ca, Cb = _streams(6 * m, c)
    C = O.csa_compress(Za, Zb, Ca, Cb, m, Ba=np.full((m, c), -1e300),
                       Bb=np.zeros((m, c)))
    for i in range(1, 6):
        S = O.column_softmax(Zb[m * (i - 1):m * i])
        np.testing.assert_allclose(C[i], (S * Cb[m * (i - 1):m * i]).sum(0), rtol=1e-13)


def test_bias_is_indexed_by_position_in_block():
    # [Scratch] §4: B in R^{m x c}, row r added to the r-th row of every window.
    # Z = 0 and B^a_r = log p_r give a-weights p_r / sum p (entry 0 has no b-rows).
    m, c, n = 4, 3, 16
    p = np.array([1.0, 2.0, 3.0, 4.0])
    Ba = np.log(p)[:, None].repeat(c, 1)
    Bb = np.full((m, c), -1e300)  # silence the b-rows
    Z = np.zeros((n, c))
    _, _, Ca, Cb = _streams(n, c)
    C = O.csa_compress(Z, Z, Ca, Cb, m, Ba=Ba, Bb=Bb)
    for i in range(n // m):
        np.testing.assert_allclose(C[i], (p[:, None] * Ca[m * i:m * (i + 1)]).sum(0) / p.sum(),
                                   rtol=1e-13)


@pytest.mark.parametrize("split", [0, 1, 3, 7, 8])
def test_csa_split_calls_equal_one_call(split):
    # compressing [0, s) then [s, N) equals one call, including the overlap across s
    m = 4
    Za, Zb, Ca, Cb = _streams(32, 5)
    full = O.csa_compress(Za, Zb, Ca, Cb, m)
    a = O.csa_compress(Za, Zb, Ca, Cb, m, i_begin=0, i_end=split)
    b = O.csa_compress(Za, Zb, Ca, Cb, m, i_begin=split, i_end=8)
    np.testing.assert_array_equal(np.vstack([a, b]), full)


def test_hca_m1_is_identity_and_mean_for_constant_logits():
    Z, C, _, _ = _streams(12, 3)
    np.testing.assert_allclose(O.hca_compress(Z, C, 1), C, rtol=0, atol=0)
    Ch = O.hca_compress(np.zeros_like(Z), C, 4)
    np.testing.assert_allclose(Ch, C.reshape(3, 4, 3).mean(1), rtol=1e-13)


def test_hca_blocks_do_not_overlap():
    # changing a row of block 1 changes entry 1 only
    Z, C, _, _ = _streams(12, 3)
    a = O.hca_compress(Z, C, 4)
    C2 = C.copy()
    C2[5] += 3.0
    b = O.hca_compress(Z, C2, 4)
    np.testing.assert_array_equal(a[[0, 2]], b[[0, 2]])
    assert (a[1] != b[1]).all()


def test_round_bf16_matches_torch_conversion():
    # library routine: torch converts fp32 to bf16 with round-to-nearest-even
    x32 = (RNG.standard_normal(20000) * 10.0 ** RNG.integers(-5, 6, 20000)).astype(np.float32)
    x32 = np.concatenate([x32, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e-3])])
    want = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(O.round_bf16(x32.astype(np.float64)), want)


# ------------------------------------------------------------------ indexer

def test_index_score_picks_coordinate():
    # one head, w = 1, q = e_j: I_s = ReLU(K_s[j]) (a closed form of [Scratch] §6.4)
    K = RNG.standard_normal((20, 6))
    for j in range(6):
        q = np.zeros((1, 6))
        q[0, j] = 1.0
        sc = O.index_scores(q, np.ones(1), K, t=20 * 3, m=3)
        np.testing.assert_array_equal(sc, np.maximum(K[:, j], 0.0))


def test_index_scores_relu_and_sign():
    nh, cI, N, m = 5, 8, 40, 4
    q = RNG.standard_normal((nh, cI))
    w = RNG.standard_normal(nh)
    K = RNG.standard_normal((N, cI))
    t = N * m
    s1 = O.index_scores(q, w, K, t, m)
    # linear in w, odd in w
    np.testing.assert_allclose(O.index_scores(q, 2 * w, K, t, m), 2 * s1, rtol=1e-14)
    np.testing.assert_allclose(O.index_scores(q, -w, K, t, m), -s1, rtol=1e-14, atol=0)
    # keys anti-aligned with every head's query contribute nothing: score exactly +0.0
    qpos = np.abs(q)
    Kneg = -np.abs(K) - 0.1
    z = O.index_scores(qpos, w, Kneg, t, m)
    assert (z == 0).all() and not np.signbit(z).any()
    # positive head weights and positive dots: the score is the weighted dot sum (no scale)
    zpos = O.index_scores(qpos, np.abs(w), np.abs(K), t, m)
    np.testing.assert_allclose(zpos, np.abs(K) @ qpos.T @ np.abs(w), rtol=1e-13)


def test_index_scores_respect_visibility():
    K = RNG.standard_normal((10, 4))
    q, w = RNG.standard_normal((2, 4)), RNG.standard_normal(2)
    for t in range(0, 41):
        assert O.index_scores(q, w, K, t, 4).shape == (t // 4,)


def _brute_topk(scores, k):
    # rank = number of entries that beat this one: a larger score, or an equal score
    # with a smaller index.  The set is the entries of rank < k.
    n = len(scores)
    ranks = [sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
             for i in range(n)]
    return sorted(i for i in range(n) if ranks[i] < k)


@pytest.mark.parametrize("trial", range(40))
def test_topk_brute_force(trial):
    rng = np.random.default_rng(trial)
    n = int(rng.integers(0, 30))
    k = int(rng.integers(1, 35))
    s = rng.integers(-3, 4, n).astype(float) * (0.5 if trial % 2 else 1.0)  # many ties
    if trial % 3 == 0:
        s = rng.standard_normal(n)
    got = O.topk_select(s, k)
    assert list(got) == _brute_topk(list(s), k)
    assert len(got) == min(k, n) and (np.diff(got) > 0).all()


def test_topk_signed_zero_ties_by_index():
    s = np.array([0.0, -0.0, 0.0, -0.0, -1.0])
    assert list(O.topk_select(s, 3)) == [0, 1, 2]


def test_topk_monotone_invariance():
    # [Scratch] §6.4: a ranking is invariant to monotone transforms; scaling w by a > 0
    nh, cI, N, m = 4, 8, 64, 4
    q, w, K = RNG.standard_normal((nh, cI)), RNG.standard_normal(nh), RNG.standard_normal((N, cI))
    a = O.topk_select(O.index_scores(q, w, K, N * m, m), 9)
    b = O.topk_select(O.index_scores(q, 3.75 * w, K, N * m, m), 9)
    np.testing.assert_array_equal(a, b)


def test_topk_never_picks_invisible():
    # the largest raw score sits in an entry the query may not see yet
    K = np.vstack([np.full((5, 2), 0.1), np.full((3, 2), 9.0)])
    q, w = np.ones((1, 2)), np.ones(1)
    t = 5 * 4 + 3  # floor(23/4) = 5 visible
    sel = O.topk_select(O.index_scores(q, w, K, t, 4), 2)
    assert sel.max() < 5


# --------------------------------------------------------------- attention

def _sdpa(q, KV, scale):
    # library routine: torch SDPA on CPU in fp64, key = value = KV, one KV head
    Q = torch.from_numpy(q)[None, None]                              # [1][1][nh][c]: heads as query rows
    K = torch.from_numpy(KV)[None, None]                             # [1][1][N][c]
    return torch.nn.functional.scaled_dot_product_attention(Q, K, K, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("N,nh,c", [(1, 1, 2), (7, 3, 8), (64, 16, 32), (300, 4, 128)])
def test_attend_with_k_covering_all_equals_sdpa(N, nh, c):
    # k >= floor(t/m) keeps every visible entry: CSA attention is dense MQA over them
    m = 4
    t = N * m + 2
    C = RNG.standard_normal((N + 3, c))  # 3 entries past the visible range
    q = RNG.standard_normal((nh, c))
    idx = O.topk_select(RNG.standard_normal(O.csa_visible(t, m)), k=N + 10)
    assert len(idx) == N
    o, lse = O.csa_attend(q, C, idx)
    np.testing.assert_allclose(o, _sdpa(q, C[:N], 1 / math.sqrt(c)), rtol=1e-12, atol=1e-13)
    ref_lse = np.log(np.exp(q @ C[:N].T / math.sqrt(c)).sum(1))
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_hca_m1_unit_logits_is_textbook_mqa_over_raw_tokens():
    # m' = 1 makes every token its own entry (C^HCA = C), so HCA attention at query t is
    # ordinary MQA over raw tokens s < t
    n, c, nh = 50, 16, 4
    C = RNG.standard_normal((n, c))
    Ch = O.hca_compress(np.zeros((n, c)), C, 1)
    q = RNG.standard_normal((nh, c))
    for t in (1, 17, 49):
        o, _ = O.hca_attend(q, Ch, t, 1)
        np.testing.assert_allclose(o, _sdpa(q, C[:t], 1 / math.sqrt(c)), rtol=1e-12, atol=1e-13)


def test_attend_one_key_and_equal_logits():
    C = RNG.standard_normal((10, 6))
    q = RNG.standard_normal((3, 6))
    o, lse = O.csa_attend(q, C, [4])
    np.testing.assert_array_equal(o, np.repeat(C[4][None], 3, 0))
    np.testing.assert_allclose(lse, q @ C[4] / math.sqrt(6), rtol=1e-15)
    # a query orthogonal to all keys: uniform weights, lse = log N
    o, lse = O.mqa_attend(np.zeros((2, 6)), C)
    np.testing.assert_allclose(o, np.repeat(C.mean(0)[None], 2, 0), rtol=1e-13)
    np.testing.assert_allclose(lse, math.log(10), rtol=1e-15)


def test_attend_permutation_invariance_and_empty():
    C = RNG.standard_normal((30, 8))
    q = RNG.standard_normal((5, 8))
    idx = np.array([3, 9, 14, 27, 2])
    o1, l1 = O.csa_attend(q, C, idx)
    o2, l2 = O.csa_attend(q, C, idx[::-1])
    np.testing.assert_allclose(o1, o2, rtol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    o, lse = O.csa_attend(q, C, np.zeros(0, dtype=np.int64))
    assert (o == 0).all() and np.isneginf(lse).all()
    o, lse = O.hca_attend(q, C, t=3, m_prime=4)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_attend_scale_is_inverse_sqrt_c():
    # [Scratch] §8: logits are q.C / sqrt(c); doubling c's scale by hand matches scale=...
    C = RNG.standard_normal((12, 16))
    q = RNG.standard_normal((2, 16))
    o_def, _ = O.mqa_attend(q, C)
    o_exp, _ = O.mqa_attend(q, C, scale=0.25)
    np.testing.assert_allclose(o_def, o_exp, rtol=1e-15)
    o_other, _ = O.mqa_attend(q, C, scale=1.0)
    assert not np.allclose(o_def, o_other)
