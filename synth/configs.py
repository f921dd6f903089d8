"""The five workloads: shapes, dtypes and seeds.

Shapes follow the notation of "DeepSeek-V4 Hybrid Attention: CSA and HCA
from Scratch": n tokens, query position t, compressed width c, ratios m and
m', top-k budget k, n_h query heads, n_h^I indexer heads of width c^I,
hidden size d and query latent d_c.
"""

from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    kind: str            # 'chain' (from hidden states), 'csa_stage', 'hca_stage', 'hybrid'
    dtype: str           # storage dtype: 'f32' or 'bf16'
    B: int               # sequences
    t: int               # decode query position (the query sees s < t/m, s < t/m')
    c: int
    m: int
    m_prime: int
    k: int
    n_h: int
    n_hI: int
    cI: int
    d: int = 0           # hidden size (0: caches are drawn directly)
    d_c: int = 0         # query latent width
    seed: int = 0
    weight_std: float = 1.0
    n_prefill: int = 0   # chunked causal prefill queries per sequence (hybrid only)
    n_decode: int = 0    # decode steps (hybrid only)
    note: str = ""

    @property
    def n_ctx(self) -> int:
        """Context tokens whose projected streams exist before the first query."""
        return self.t

    @property
    def csa_entries(self) -> int:
        return self.t // self.m

    @property
    def hca_entries(self) -> int:
        return self.t // self.m_prime


CONFIGS = {
    # the hand-traced example: H as printed, seeded N(0,1) weights, query at the last token
    "toy6": Config("toy6", "chain", "f32", B=1, t=5, c=2, m=2, m_prime=3, k=1, n_h=1, n_hI=1,
                   cI=2, d=2, d_c=2, seed=0, weight_std=1.0,
                   note="n=6 tokens, H printed, weights N(0,1) seed 0, query t=5"),
    # one layer from hidden states: 8192 context tokens, the query is token 8192
    "decode8k": Config("decode8k", "chain", "bf16", B=1, t=8192, c=128, m=4, m_prime=128, k=64,
                       n_h=16, n_hI=4, cI=64, d=1024, d_c=128, seed=1,
                       weight_std=1024 ** -0.5, note="H ~N(0,1), weights N(0,1/d)"),
    # CSA decode at V4-Pro head shape; caches and queries drawn directly
    "csa128k": Config("csa128k", "csa_stage", "bf16", B=8, t=131072, c=512, m=4, m_prime=128,
                      k=1024, n_h=128, n_hI=64, cI=128, seed=2,
                      note="C^Comp, K^I, q, q^I ~N(0,1) bf16; w^I ~N(0,1) fp32"),
    # HCA dense decode at 1M context; cache and queries drawn directly
    "hca1m": Config("hca1m", "hca_stage", "bf16", B=16, t=1 << 20, c=512, m=4, m_prime=128, k=0,
                    n_h=128, n_hI=0, cI=0, seed=3, note="C^HCA, q ~N(0,1) bf16"),
    # full hybrid layer: compressor pass over 2^20 tokens, prefill, 256 decode steps
    "hybrid1m": Config("hybrid1m", "hybrid", "bf16", B=4, t=1 << 20, c=512, m=4, m_prime=128,
                       k=1024, n_h=128, n_hI=64, cI=128, d=7168, d_c=512, seed=4,
                       weight_std=7168 ** -0.5, n_prefill=4096, n_decode=256,
                       note="H ~N(0,1) bf16 d=7168, weights N(0,1/d)"),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


# canonical tensor ids: a tensor's seed is seed*1000 + id (see synth.gen.tensor_seed)
TENSOR_IDS = dict(
    H=0, aKV=1, bKV=2, aZ=3, bZ=4, IaKV=5, IbKV=6, IaZ=7, IbZ=8, KV=9, Z=10,
    DQ=11, IUQ=12, w=13, UQ=14, UQ_hca=15,
    Ccomp=20, KI=21, Chca=22, q=23, qI=24, wI=25, q_hca=26,
    Ba=30, Bb=31, BIa=32, BIb=33, Bh=34,
    win=16, win_hca=17,
)
