"""Seeded generators.  Random numbers only; none of the method's arithmetic.

Every tensor has a canonical id (synth.configs.TENSOR_IDS) and is drawn as
float32 ``torch.randn`` from a generator seeded with ``seed*1000 + id``,
scaled, then rounded to the storage dtype (round-to-nearest-even).  Tensors
with many rows are drawn in chunks of 2**16 rows, chunk j seeded with
``(seed*1000 + id) * 2**20 + j``, so any chunk can be drawn again alone.
Draws on a CUDA device use torch's device generator with the same seeds; a
host that needs those values copies the input back from the device.
"""

import torch

from .configs import TENSOR_IDS

CHUNK_ROWS = 1 << 16
_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}


def tensor_seed(cfg_seed: int, name_or_id, chunk=None) -> int:
    tid = TENSOR_IDS[name_or_id] if isinstance(name_or_id, str) else int(name_or_id)
    base = cfg_seed * 1000 + tid
    return base if chunk is None else base * (1 << 20) + int(chunk)


def _randn(shape, seed, device):
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type != "cuda" else dev)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=dev)


def normal(shape, seed: int, std: float = 1.0, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in float32 from one seed, then rounded to ``dtype``."""
    x = _randn(shape, seed, device)
    if std != 1.0:
        x.mul_(std)
    return x.to(_DT[dtype])


def normal_chunked_rows(rows: int, cols: int, seed_base: int, std: float = 1.0, dtype: str = "bf16",
                        device="cpu", row_begin: int = 0, row_end=None, out=None) -> torch.Tensor:
    """Rows [row_begin, row_end) of a [rows][cols] tensor drawn chunk by chunk.

    Chunk j covers rows j*2^16 ... (j+1)*2^16-1 and is seeded with
    seed_base*2^20 + j, so a sub-range is drawn without the rest.
    """
    row_end = rows if row_end is None else row_end
    assert 0 <= row_begin <= row_end <= rows
    if out is None:
        out = torch.empty((row_end - row_begin, cols), dtype=_DT[dtype], device=device)
    j0, j1 = row_begin // CHUNK_ROWS, (row_end + CHUNK_ROWS - 1) // CHUNK_ROWS
    for j in range(j0, j1):
        lo, hi = j * CHUNK_ROWS, min(rows, (j + 1) * CHUNK_ROWS)
        blk = normal((hi - lo, cols), seed_base * (1 << 20) + j, std, dtype, device)
        a, b = max(lo, row_begin), min(hi, row_end)
        out[a - row_begin:b - row_begin].copy_(blk[a - lo:b - lo])
    return out


def page_toy_hidden(dtype: str = "f32") -> torch.Tensor:
    """The six hidden states of the running example, as printed on the page
    "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch" (The Running Example)."""
    H = [[1, 0], [0, 2], [2, 1], [1, 1], [0, 1], [1, 0]]
    return torch.tensor(H, dtype=_DT[dtype])
