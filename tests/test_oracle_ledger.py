"""Pin the oracle's ledger to the printed figures of "DeepSeek-V4 Hybrid
Attention: CSA and HCA from Scratch", §1 and §12."""

import oracle as O


def test_gqa_baseline(golden):
    g = golden["ledger"]
    assert O.gqa_kv_bytes_per_token_layer(8, 128, 2) == g["gqa8_bytes_per_token_layer"]
    total = 10 ** 6 * 61 * O.gqa_kv_bytes_per_token_layer()
    assert abs(total - g["request_bytes_1e6_tokens_61_layers"]) / total < 0.005  # "~2.5e11"
    assert total == 249_856_000_000


def test_compressed_per_layer(golden):
    g = golden["ledger"]
    L = O.ledger(c=512, m=4, m_prime=128, b=2, baseline=g["gqa8_baseline_per_layer_coeff"])
    assert L["csa"] == g["csa_coeff"] == 256
    assert L["hca"] == g["hca_coeff"] == 8
    assert L["csa_ratio"] == g["csa_ratio"]
    assert L["hca_ratio"] == 8 / 2048 == 0.00390625
    assert abs(L["hca_ratio"] - g["hca_ratio_approx"]) < 5e-4  # printed to 3 decimals
    assert 30 * L["csa"] + 31 * L["hca"] == g["mix_numerator"]
    assert 61 * 2048 == g["mix_denominator"]
    assert abs(L["mix"] - 7928 / 124928) < 1e-15
    assert abs(L["mix"] - g["mix_ratio_approx"]) < 5e-4


def test_ratios_are_one_over_m():
    # the cache shrinks by exactly m (CSA) and m' (HCA) against one c-wide entry per token
    for c in (2, 128, 512):
        for m in (1, 2, 4, 128):
            assert O.compressed_bytes_per_token_layer(c, m, 2) * m == c * 2


def test_ledger_against_4096_baseline():
    # the K-and-V baseline of §1 halves every ratio
    L = O.ledger(baseline=4096)
    assert L["csa_ratio"] == 0.0625 and L["hca_ratio"] == 8 / 4096


def test_indexer_flops(golden):
    n = 10 ** 6
    assert O.indexer_flops_per_query(n, 4, 64, 128) == golden["ledger"]["indexer_flops_coeff"] * n
