"""csa_attend_noalloc, the allocation-free form of csa_attend (its split
partials in the library's static scratch array), against csa_attend itself
through the C ABI: two calls in a row, the second on a smaller input, each
bit-identical to csa_attend and within the bf16 bar of the oracle."""

import ctypes as C

import numpy as np
import pytest
import torch

import dense_long_context_amd as dlc
import oracle as O
import synth
from dense_long_context_amd import binding
from devtools import DEV, assert_rows_close, need_gpu

pytestmark = pytest.mark.gpu


def _inputs(B, n_q, n_h, c, k, cap, seed):
    q = synth.normal((B, n_q, n_h, c), seed, dtype="bf16", device=DEV)
    Cc = synth.normal((B, cap, c), seed + 1, dtype="bf16", device=DEV)
    g = torch.Generator().manual_seed(seed + 2)
    idx = torch.full((B, n_q, k), -1, dtype=torch.int32)
    cnt = torch.empty((B, n_q), dtype=torch.int32)
    for b in range(B):
        for j in range(n_q):
            n = k - (b + j) % 3                      # ragged counts, one short of k and more
            idx[b, j, :n] = torch.randperm(cap, generator=g)[:n].sort().values.to(torch.int32)
            cnt[b, j] = n
    return q, Cc, idx.to(DEV), cnt.to(DEV)


def test_csa_attend_noalloc_matches_csa_attend():
    need_gpu()
    L = binding.lib()
    stream = torch.cuda.current_stream(torch.device(DEV)).cuda_stream
    # the decode shape of a 1M-context layer, then a smaller one on the same scratch
    for B, n_q, n_h, c, k, cap, seed in ((4, 1, 128, 512, 1024, 32768, 11), (2, 1, 64, 512, 300, 5000, 12)):
        print(f"noalloc B={B} n_h={n_h} c={c} k={k}", flush=True)
        q, Cc, idx, cnt = _inputs(B, n_q, n_h, c, k, cap, seed)
        ref_o, ref_l = dlc.csa_attend(q, Cc, idx, cnt)
        out = torch.full((B, n_q, n_h, c), float("nan"), device=DEV)
        lse = torch.full((B, n_q, n_h), float("nan"), device=DEV)
        p = lambda x: C.c_void_p(x.data_ptr())  # noqa: E731
        rc = L.csa_attend_noalloc(binding.DLC_BF16, B, n_q, n_h, c, k, p(q), p(Cc), cap, p(idx), p(cnt), 0.0,
                                  p(out), p(lse), C.c_void_p(stream))
        assert rc == 0, binding.last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "differs from csa_attend"
        for b in range(B):
            sel = idx[b, 0, :int(cnt[b, 0])].cpu().numpy().astype(np.int64)
            o_r, l_r = O.csa_attend(q[b, 0].cpu(), Cc[b].cpu(), sel)
            assert_rows_close(out[b, 0].cpu(), o_r, 2e-2, f"noalloc b={b}")
            assert np.abs(lse[b, 0].cpu().numpy() - l_r).max() <= 2e-2


def test_csa_attend_noalloc_refuses_oversized_shapes():
    need_gpu()
    B, k = 256, 8192                                  # far more partials than the scratch holds
    q = torch.zeros((B, 1, 128, 512), dtype=torch.bfloat16, device=DEV)
    Cc = torch.zeros((B, 16, 512), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((B, 1, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, 128, 512), device=DEV)
    lse = torch.empty((B, 1, 128), device=DEV)
    with pytest.raises(binding.DlcError, match="scratch"):
        dlc.csa_attend_noalloc(q, Cc, idx, cnt, out, lse)
