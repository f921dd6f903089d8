"""Pins of the oracle's MXFP4 indexer path (no GPU).

The pages say the lightning indexer's products run in FP4 ("DeepSeek-V4
Hybrid Attention: CSA and HCA from Scratch", §6.4 and §12) but not which FP4
format; the oracle reads it as OCP MXFP4 (E2M1 elements, one E8M0 scale per 32
elements).  These tests pin that reading to the format's own definition:
the E2M1 value table, round-to-nearest-even on that grid, the shared-exponent
rule that puts a block's maximum in E2M1's top binade [4, 8), exactness on
representable inputs, and the error bound that rounding on the grid implies.
"""

import numpy as np
import pytest

from oracle import dlc_oracle as o

# E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit): the eight
# magnitudes written out from the bit fields, independently of the oracle
def e2m1_from_bits(code):
    e, mbit = (code >> 1) & 3, code & 1
    return mbit * 0.5 if e == 0 else (1.0 + 0.5 * mbit) * 2.0 ** (e - 1)


def test_e2m1_table_matches_bit_fields():
    assert tuple(e2m1_from_bits(c) for c in range(8)) == o.E2M1_MAGNITUDES


def _q1(values):
    """quantize one 32-element block whose other elements are 0"""
    x = np.zeros((1, 32))
    x[0, : len(values)] = values
    codes, shared = o.mxfp4_quantize(x)
    return codes[0, : len(values)], int(shared[0, 0])


def test_hand_block_ties_to_even_and_saturation():
    # block max 7.9 -> floor(log2 7.9) = 2 -> shared exponent 0, so the
    # values are rounded as they are:
    #   6 -> 6 (code 7); 3 -> 3 (code 5); 0.25 is halfway 0|0.5 -> even code 0;
    #   0.75 halfway 0.5|1 -> code 2 (1.0); -5 halfway 4|6 -> code 6, negative (14);
    #   7.9 saturates to 6 (code 7); 1.25 halfway 1|1.5 -> code 2; 1.75 halfway
    #   1.5|2 -> code 4; 2.5 halfway 2|3 -> code 4; 3.5 halfway 3|4 -> code 6;
    #   0.3 -> 0.5 (code 1); -0.2 -> 0, stored as +0 (code 0)
    codes, shared = _q1([6, 3, 0.25, 0.75, -5, 7.9, 1.25, 1.75, 2.5, 3.5, 0.3, -0.2])
    assert shared == 0
    assert codes.tolist() == [7, 5, 0, 2, 14, 7, 2, 4, 4, 6, 1, 0]


def test_hand_block_scaled():
    # block max 0.1: floor(log2 0.1) = -4 -> shared -6, unit 2^-6 = 1/64;
    # 0.1 * 64 = 6.4 -> 6 (code 7); 0.03 * 64 = 1.92 -> 2 (code 4);
    # -0.01 * 64 = -0.64 -> 0.5 (code 9)
    codes, shared = _q1([0.1, 0.03, -0.01])
    assert shared == -6
    assert codes.tolist() == [7, 4, 9]
    deq = o.mxfp4_dequantize(*o.mxfp4_quantize(np.array([[0.1, 0.03, -0.01] + [0.0] * 29])))
    assert deq[0, :3].tolist() == [6 / 64, 2 / 64, -0.5 / 64]


def test_zero_block():
    codes, shared = o.mxfp4_quantize(np.zeros((2, 64)))
    assert (codes == 0).all() and (shared == -127).all()


def test_shared_exponent_puts_block_max_in_top_binade():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128)) * np.exp2(rng.integers(-20, 20, size=(50, 1)))
    _, shared = o.mxfp4_quantize(x)
    amax = np.abs(x.reshape(50, 4, 32)).max(-1)
    r = amax / np.exp2(shared)
    assert (r >= 4).all() and (r < 8).all()


def test_representable_values_round_trip():
    rng = np.random.default_rng(2)
    rows, blocks = 40, 4
    mags = rng.integers(0, 8, size=(rows, blocks, 32))
    mags[..., 0] = rng.integers(6, 8, size=(rows, blocks))      # block max 4 or 6: shared exponent as drawn
    signs = rng.integers(0, 2, size=(rows, blocks, 32)) * (mags > 0)
    exps = rng.integers(-30, 30, size=(rows, blocks))
    vals = np.asarray([e2m1_from_bits(c) for c in range(8)])[mags] * np.where(signs, -1.0, 1.0)
    x = (vals * np.exp2(exps)[..., None]).reshape(rows, blocks * 32)
    codes, shared = o.mxfp4_quantize(x)
    assert (shared == exps).all()
    assert (codes == (mags + 8 * signs).reshape(rows, -1)).all()
    assert (o.mxfp4_dequantize(codes, shared) == x).all()


def test_error_bound_of_grid_rounding():
    # on the grid the spacing is 0.5 below 2, 1 in [2, 4), 2 in [4, 6]: the
    # rounding error is at most half of it; above 6 the value saturates
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 64)) * 3.0
    codes, shared = o.mxfp4_quantize(x)
    y = x / np.repeat(np.exp2(shared), 32, axis=-1)
    dq = o.mxfp4_dequantize(codes, shared) / np.repeat(np.exp2(shared), 32, axis=-1)
    a = np.abs(y)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.where(a > 6, a - 6, half)
    assert (np.abs(dq - y) <= bound + 1e-15).all()
    assert (np.sign(dq) * np.sign(y) >= 0).all()


def test_rounding_is_nearest_with_even_ties_everywhere_on_the_grid():
    grid = list(o.E2M1_MAGNITUDES)
    for i in range(7):
        lo, hi = grid[i], grid[i + 1]
        mid = (lo + hi) / 2
        eps = (hi - lo) * 1e-3
        # keep the block's shared exponent at 0 with a 4 in the block
        c, s = _q1([4.0, mid - eps, mid, mid + eps, -(mid - eps), -(mid + eps)])
        assert s == 0
        assert c[1] == i and c[3] == i + 1
        assert c[2] == (i if i % 2 == 0 else i + 1)
        assert c[4] == (i + 8 if i > 0 else 0) and c[5] == i + 1 + 8


def test_fp4_scores_equal_exact_scores_on_representable_inputs():
    rng = np.random.default_rng(4)
    n_hI, cI, nk, m, t = 8, 64, 40, 4, 160

    def representable(shape):
        mags = rng.integers(0, 8, size=shape + (cI // 32, 32))
        mags[..., 0] = 7
        v = np.asarray(o.E2M1_MAGNITUDES)[mags] * rng.choice([-1.0, 1.0], size=mags.shape)
        return (v * np.exp2(rng.integers(-6, 6, size=shape + (cI // 32, 1)))).reshape(shape + (cI,))

    qI, KI = representable((n_hI,)), representable((nk,))
    wI = rng.standard_normal(n_hI)
    assert np.array_equal(o.index_scores_fp4(qI, wI, KI, t, m), o.index_scores(qI, wI, KI, t, m))


def test_fp4_scores_track_exact_scores():
    rng = np.random.default_rng(5)
    n_hI, cI, nk = 16, 128, 300
    qI, KI = rng.standard_normal((n_hI, cI)), rng.standard_normal((nk, cI))
    wI = np.abs(rng.standard_normal(n_hI))
    exact = o.index_scores(qI, wI, KI, 4 * nk, 4)
    fp4 = o.index_scores_fp4(qI, wI, KI, 4 * nk, 4)
    assert np.corrcoef(exact, fp4)[0, 1] > 0.97
    assert np.linalg.norm(fp4 - exact) / np.linalg.norm(exact) < 0.25
