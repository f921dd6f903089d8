"""Decode throughput of one CSA layer plus one HCA layer at 1M context on one GPU.

Workload (hybrid1m): B = 4 sequences of 2^20 context tokens, d = 7168 bf16
hidden states ~N(0,1), projection weights N(0, 1/d); c = 512, m = 4, m' = 128,
k = 1024, n_h = 128, n_h^I = 64, c^I = 128.  Set-up (untimed): the hidden
states are projected to the compressor streams (dlc_project), the CSA,
indexer-key and HCA caches are built by the compressors over all 2^20 + 256
tokens, and the decode queries of the 256 decode tokens are projected.
Three copies of the caches stand for three layers' caches and rotate per
step, so a step does not re-read what the previous step left in the 256 MB
last-level cache.

One step = the whole hot path for the B decode queries at t = 2^20 + s:
  csa_compress x2 (KV and indexer keys, when token t completes a CSA block),
  hca_compress (when t completes an HCA block), csa_index_topk, csa_attend,
  hca_attend.
Every call goes through the C ABI with pre-marshalled arguments.

Prints one JSON line.  With --gpus N > 1 it exits: this build runs on one GPU.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s per CSA+HCA layer at 1M ctx; achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
SCORES_KERNEL = "scores_reg_kernel<4, 4, 3>"
SCORES_KERNEL_FP4 = "scores_fp4_reg_kernel<128, 3>"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "indexer_scores_hybrid1m_counters.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    for f in ("indexer.hip", "common.hpp"):
        with open(os.path.join(ROOT, "dense_long_context_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw hipEvent_t handles (for dlc_timing_arm) through libamdhip64."""

    def __init__(self):
        import ctypes as C

        self.C = C
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = self.C.c_void_p()
        assert self.hip.hipEventCreate(self.C.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = self.C.c_float()
        assert self.hip.hipEventElapsedTime(self.C.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


STREAMS = ["aKV", "bKV", "aZ", "bZ", "IaKV", "IbKV", "IaZ", "IbZ", "KV", "Z"]


def stream_layout(cfg):
    """Column offset and width of each projected stream in the side-by-side buffer."""
    width = {nm: (cfg.cI if nm.startswith("I") else cfg.c) for nm in STREAMS}
    off, o = {}, 0
    for nm in STREAMS:
        off[nm] = o
        o += width[nm]
    return off, width, o


def stream_weight(cfg, nm):
    """W for stream ``nm``: [d][width] bf16 on the host, N(0, 1/d)."""
    _, width, _ = stream_layout(cfg)
    import synth
    return synth.normal((cfg.d, width[nm]), synth.tensor_seed(cfg.seed, nm), cfg.weight_std, "bf16")


def query_weight(cfg, nm):
    """Query-side weights on the host: W^DQ [d][d_c], W^w [d][n_hI] (std 1/sqrt(d)), and
    W^IUQ [d_c][n_hI*cI], W^UQ and W^UQ_hca [d_c][n_h*c] (std 1/sqrt(d_c))."""
    import synth
    shape = {"DQ": (cfg.d, cfg.d_c), "w": (cfg.d, cfg.n_hI), "IUQ": (cfg.d_c, cfg.n_hI * cfg.cI),
             "UQ": (cfg.d_c, cfg.n_h * cfg.c), "UQ_hca": (cfg.d_c, cfg.n_h * cfg.c)}[nm]
    std = cfg.weight_std if nm in ("DQ", "w") else cfg.d_c ** -0.5
    return synth.normal(shape, synth.tensor_seed(cfg.seed, nm), std, "bf16")


N_WIN = 128  # sliding-window tokens per query (V4-Pro)


def window_weight(cfg, nm):
    """W^{window,KV} of the CSA layer ("win") or the HCA layer ("win_hca"): [d][c] bf16, N(0, 1/d)."""
    import synth
    return synth.normal((cfg.d, cfg.c), synth.tensor_seed(cfg.seed, nm), cfg.weight_std, "bf16")


def hidden_rows(cfg, b, n_tot, r0, r1, dev):
    """Rows [r0, r1) of sequence b's hidden states [n_tot][d] bf16, drawn on ``dev``."""
    import synth
    base = synth.tensor_seed(cfg.seed, "H") * 16 + b
    return synth.normal_chunked_rows(n_tot, cfg.d, base, 1.0, "bf16", dev, r0, r1)


def build_workload(cfg, dev, n_dec, n_sets=3):
    import torch

    import dense_long_context_amd as dlc

    B, d, c, cI, m, mp = cfg.B, cfg.d, cfg.c, cfg.cI, cfg.m, cfg.m_prime
    n_ctx = cfg.t                       # 2^20 context tokens
    n_tot = n_ctx + n_dec               # plus the decode tokens
    t0 = time.perf_counter()
    off, width, NS = stream_layout(cfg)
    Wt = torch.cat([stream_weight(cfg, nm).t() for nm in STREAMS], 0).contiguous().to(dev)  # [NS][d]
    S = torch.empty((B, n_tot, NS), dtype=torch.bfloat16, device=dev)
    H_dec = torch.empty((B, n_dec, d), dtype=torch.bfloat16, device=dev)  # hidden states of the decode tokens
    chunk = 1 << 16
    evs = []
    for b in range(B):
        for r0 in range(0, n_tot, chunk):
            r1 = min(n_tot, r0 + chunk)
            Hc = hidden_rows(cfg, b, n_tot, r0, r1, dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dlc.dlc_project(Hc, Wt, out=S[b, r0:r1])
            e1.record()
            evs.append((e0, e1))
            if r0 <= n_ctx < r1:
                H_dec[b] = Hc[n_ctx - r0:n_ctx - r0 + n_dec]
    torch.cuda.synchronize()
    t_proj = time.perf_counter() - t0
    t_proj_kernel = sum(a.elapsed_time(b) for a, b in evs) / 1e3
    col = lambda nm: S[:, :, off[nm]:off[nm] + width[nm]]  # noqa: E731

    cap_csa, cap_hca = n_tot // m, n_tot // mp
    sets = []
    cevs = []  # per set: events around the CSA KV, CSA indexer-key and HCA passes
    for _ in range(n_sets):
        Cc = torch.empty((B, cap_csa, c), dtype=torch.bfloat16, device=dev)
        KI = torch.empty((B, cap_csa, cI), dtype=torch.bfloat16, device=dev)
        Ch = torch.empty((B, cap_hca, c), dtype=torch.bfloat16, device=dev)
        ev4 = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev4[0].record()
        dlc.csa_compress(col("aZ"), col("bZ"), col("aKV"), col("bKV"), m, Cc)
        ev4[1].record()
        dlc.csa_compress(col("IaZ"), col("IbZ"), col("IaKV"), col("IbKV"), m, KI)
        ev4[2].record()
        dlc.hca_compress(col("Z"), col("KV"), mp, Ch)
        ev4[3].record()
        cevs.append(ev4)
        KIc, KIs = dlc.mxfp4_quantize(KI)  # the FP4 indexer's key cache (MXFP4 codes + scales)
        sets.append((Cc, KI, Ch, KIc, KIs))
    torch.cuda.synchronize()
    # the median set (the first is cold), each pass on its own
    per_set = sorted((tuple(e[i].elapsed_time(e[i + 1]) / 1e3 for i in range(3)) for e in cevs), key=sum)
    t_stage = per_set[len(per_set) // 2]
    t_comp = sum(t_stage)

    # decode queries of tokens n_ctx .. n_tot-1 (projected once, stored per step)
    Wq = {nm: query_weight(cfg, nm).t().contiguous().to(dev) for nm in ("DQ", "w", "IUQ", "UQ", "UQ_hca")}
    h = H_dec.reshape(B * n_dec, d)
    cQ = dlc.dlc_project(h, Wq["DQ"])
    qI = dlc.dlc_project(cQ, Wq["IUQ"])
    wI = dlc.dlc_project(h, Wq["w"], out_dtype=torch.float32)
    q = dlc.dlc_project(cQ, Wq["UQ"])
    qh = dlc.dlc_project(cQ, Wq["UQ_hca"])
    # sliding-window entries c^window_p = h_p W^{window,KV} of positions n_ctx-N_WIN .. n_tot-1, one ring per
    # layer with ring = N_WIN + n_dec rows (token p at row p % ring), so every decode step's window is in it
    ring = N_WIN + n_dec
    lo = n_ctx - N_WIN
    rings = {}
    for nm in ("win", "win_hca"):
        Ww = window_weight(cfg, nm).t().contiguous().to(dev)
        R = torch.empty((B, ring, c), dtype=torch.bfloat16, device=dev)
        for b in range(B):
            hw = hidden_rows(cfg, b, n_tot, lo, n_tot, dev)
            rows = dlc.dlc_project(hw, Ww)                        # positions lo .. n_tot-1
            pos = torch.arange(lo, n_tot, device=dev) % ring
            R[b, pos] = rows
        rings[nm] = R
    per_step = lambda x, *shape: x.reshape(B, n_dec, *shape).transpose(0, 1).contiguous()  # noqa: E731
    Q = dict(qI=per_step(qI, 1, cfg.n_hI, cI), wI=per_step(wI, 1, cfg.n_hI), q=per_step(q, 1, cfg.n_h, c),
             qh=per_step(qh, 1, cfg.n_h, c), cQ=per_step(cQ, 1, cfg.d_c))
    torch.cuda.synchronize()
    return dict(S=S, col=col, sets=sets, Q=Q, rings=rings, ring=ring, n_ctx=n_ctx, n_tot=n_tot, cap_csa=cap_csa,
                cap_hca=cap_hca, H_dec=H_dec, Wq=Wq,
                t_proj=t_proj, t_proj_kernel=t_proj_kernel, t_comp=t_comp, t_stage=t_stage, stream_bytes=S.numel() * 2,
                stage_bytes=(B * n_tot * 4 * c * 2 + B * cap_csa * c * 2, B * n_tot * 4 * cI * 2 + B * cap_csa * cI * 2,
                             B * n_tot * 2 * c * 2 + B * cap_hca * c * 2))


def fused_setup(cfg, wl, dev):
    """The three caches of the workload again, straight from the hidden rows by
    csa_project_compress (C^Comp and K^I) and hca_project_compress (C^HCA),
    chunk by chunk of rows as the two-pass build projects them; returns the
    summed kernel time (HIP events) and whether every cache equals the
    two-pass build's bit for bit."""
    import torch

    import dense_long_context_amd as dlc
    from dense_long_context_amd import binding

    L = binding.lib()
    B, d, c, cI, m, mp = cfg.B, cfg.d, cfg.c, cfg.cI, cfg.m, cfg.m_prime
    n_tot = wl["n_tot"]
    Wt = {nm: stream_weight(cfg, nm).t().contiguous().to(dev) for nm in STREAMS}
    Cc0, KI0, Ch0 = wl["sets"][0][:3]
    Cc, KI, Ch = torch.empty_like(Cc0), torch.empty_like(KI0), torch.empty_like(Ch0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    chunk = 1 << 16
    assert chunk % mp == 0 and chunk % m == 0
    evs = []
    for b in range(B):
        for r0 in range(0, n_tot, chunk):
            r1 = min(n_tot, r0 + chunk)
            h0 = max(0, r0 - m)  # CSA entries of this chunk also pool the block before it
            Hc = hidden_rows(cfg, b, n_tot, h0, r1, dev)
            rows = r1 - h0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            # rows h0 .. r1-1 as the call's sequence: its entry i is entry h0/m + i
            # of the cache; the first is skipped when it needs the rows before h0
            for out, nm, width in ((Cc, "", c), (KI, "I", cI)):
                i0 = 0 if h0 == 0 else 1
                rc = L.csa_project_compress(
                    binding.DLC_BF16, 1, rows, d, width, m, Hc.data_ptr(), d, rows * d,
                    Wt[nm + "aZ"].data_ptr(), Wt[nm + "bZ"].data_ptr(), Wt[nm + "aKV"].data_ptr(),
                    Wt[nm + "bKV"].data_ptr(), d, None, None, i0, rows // m,
                    out.data_ptr() + (b * out.shape[1] + h0 // m) * width * 2, out.shape[1] - h0 // m, stream)
                assert rc == 0, binding.last_error()
            Hh = Hc[r0 - h0:]
            rc = L.hca_project_compress(
                binding.DLC_BF16, 1, r1 - r0, d, c, mp, Hh.data_ptr(), d, (r1 - r0) * d, Wt["Z"].data_ptr(),
                Wt["KV"].data_ptr(), d, None, 0, (r1 - r0) // mp,
                Ch.data_ptr() + (b * Ch.shape[1] + r0 // mp) * c * 2, Ch.shape[1] - r0 // mp, stream)
            assert rc == 0, binding.last_error()
            e1.record()
            evs.append((e0, e1))
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in evs) / 1e3
    same = all(torch.equal(x, y) for x, y in ((Cc, Cc0), (KI, KI0), (Ch, Ch0)))
    return t, same


def make_steps(cfg, wl, dev, n_dec, window=False, fp4=False):
    """Pre-marshal the C-ABI argument tuples of every decode step.  window: each
    layer's sliding-window branch joins its attention output in place.  fp4: the
    indexer runs on the MXFP4 key cache (each new K^I entry is quantized as it
    is written) through csa_index_topk_fp4."""
    import torch

    import dense_long_context_amd as dlc
    from dense_long_context_amd import binding

    L = binding.lib()
    B, c, cI, m, mp, k, n_h, n_hI = cfg.B, cfg.c, cfg.cI, cfg.m, cfg.m_prime, cfg.k, cfg.n_h, cfg.n_hI
    BF = binding.DLC_BF16
    stream = torch.cuda.current_stream(dev).cuda_stream
    S, col = wl["S"], wl["col"]
    ld, bs = S.stride(1), S.stride(0)
    n_tot, cap_csa, cap_hca = wl["n_tot"], wl["cap_csa"], wl["cap_hca"]
    ws_i = torch.zeros(max(dlc.csa_index_topk_ws(B, 1, cap_csa, k),
                           dlc.csa_index_topk_fp4_ws(B, 1, n_hI, cI, cap_csa, k)), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, dlc.csa_attend_ws(B, 1, n_h, c, k)), dtype=torch.uint8, device=dev)
    ws_h = torch.empty(max(1, dlc.hca_attend_ws(B, 1, n_h, c, cap_hca)), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, 1), dtype=torch.int32, device=dev)
    o1 = torch.empty((B, 1, n_h, c), dtype=torch.float32, device=dev)
    l1 = torch.empty((B, 1, n_h), dtype=torch.float32, device=dev)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    ws_w = torch.empty(max(1, binding.lib().csa_attend_window_ws(B, 1, n_h, c, k, N_WIN),
                           binding.lib().hca_attend_window_ws(B, 1, n_h, c, cap_hca, N_WIN)),
                       dtype=torch.uint8, device=dev)
    tt = torch.arange(wl["n_ctx"], wl["n_ctx"] + n_dec, dtype=torch.int64, device=dev)
    tt = tt[:, None, None].expand(n_dec, B, 1).contiguous()
    p = lambda x: x.data_ptr()  # noqa: E731
    Q = wl["Q"]
    steps = []
    for s in range(n_dec):
        t = wl["n_ctx"] + s
        Cc, KI, Ch, KIc, KIs = wl["sets"][s % 3]
        calls = []
        if (t + 1) % m == 0:
            i = (t + 1) // m - 1
            calls.append((L.csa_compress, (BF, B, n_tot, c, m, p(col("aZ")), p(col("bZ")), p(col("aKV")),
                                           p(col("bKV")), ld, bs, None, None, i, i + 1, p(Cc), cap_csa, stream)))
            calls.append((L.csa_compress, (BF, B, n_tot, cI, m, p(col("IaZ")), p(col("IbZ")), p(col("IaKV")),
                                           p(col("IbKV")), ld, bs, None, None, i, i + 1, p(KI), cap_csa, stream)))
            if fp4:
                calls.append((L.mxfp4_quantize, (BF, B, 1, cI, p(KI) + i * cI * 2, cap_csa * cI,
                                                 p(KIc) + i * cI // 2, cap_csa * cI // 2, p(KIs) + i * cI // 32,
                                                 cap_csa * cI // 32, stream)))
        if (t + 1) % mp == 0:
            i = (t + 1) // mp - 1
            calls.append((L.hca_compress, (BF, B, n_tot, c, mp, p(col("Z")), p(col("KV")), ld, bs, None, i, i + 1,
                                           p(Ch), cap_hca, stream)))
        if fp4:
            calls.append((L.csa_index_topk_fp4, (BF, B, 1, n_hI, cI, m, k, p(Q["qI"][s]), p(Q["wI"][s]), p(KIc),
                                                 p(KIs), cap_csa, p(tt[s]), t, p(idx), p(cnt), None, p(ws_i),
                                                 ws_i.numel(), stream)))
        else:
            calls.append((L.csa_index_topk, (BF, B, 1, n_hI, cI, m, k, p(Q["qI"][s]), p(Q["wI"][s]), p(KI),
                                             cap_csa, p(tt[s]), t, p(idx), p(cnt), None, p(ws_i), ws_i.numel(),
                                             stream)))
        if window:  # each layer's attention with its sliding window joined in (one key list)
            calls.append((L.csa_attend_window, (BF, B, 1, n_h, c, k, p(Q["q"][s]), p(Cc), cap_csa, p(idx), p(cnt),
                                                p(wl["rings"]["win"]), wl["ring"], N_WIN, p(tt[s]), t, 0.0, p(o1),
                                                p(l1), p(ws_w), ws_w.numel(), stream)))
            calls.append((L.hca_attend_window, (BF, B, 1, n_h, c, mp, p(Q["qh"][s]), p(Ch), cap_hca, p(tt[s]), t,
                                                p(wl["rings"]["win_hca"]), wl["ring"], N_WIN, 0.0, p(o2), p(l2),
                                                p(ws_w), ws_w.numel(), stream)))
        else:
            calls.append((L.csa_attend, (BF, B, 1, n_h, c, k, p(Q["q"][s]), p(Cc), cap_csa, p(idx), p(cnt), 0.0,
                                         p(o1), p(l1), p(ws_c), ws_c.numel(), stream)))
            calls.append((L.hca_attend, (BF, B, 1, n_h, c, mp, p(Q["qh"][s]), p(Ch), cap_hca, p(tt[s]), t, 0.0,
                                         p(o2), p(l2), p(ws_h), ws_h.numel(), stream)))
        steps.append((t, calls))
    keep = dict(ws_i=ws_i, ws_c=ws_c, ws_h=ws_h, ws_w=ws_w, idx=idx, cnt=cnt, o_csa=o1, lse_csa=l1, o_hca=o2,
                lse_hca=l2, t=tt)
    return steps, keep


def prefill_pass(cfg, wl, dev, n_pref=4096, chunk=256, ev=None, fp4=False):
    """The chunked causal prefill of config 5: queries at t = 2^20-n_pref .. 2^20-1
    of every sequence, `chunk` per sequence per call, through csa_index_topk (which
    runs query-tiled at this many queries), csa_attend and hca_attend.  Returns the
    timings (ms) and the indexer's algorithmic FLOPs."""
    import torch

    import dense_long_context_amd as dlc
    from dense_long_context_amd import binding

    B, d, c, cI, m, mp, k, n_h, n_hI = cfg.B, cfg.d, cfg.c, cfg.cI, cfg.m, cfg.m_prime, cfg.k, cfg.n_h, cfg.n_hI
    n_ctx, n_tot = wl["n_ctx"], wl["n_tot"]
    Cc, KI, Ch, KIc, KIs = wl["sets"][0]
    Wq = {nm: query_weight(cfg, nm).t().contiguous().to(dev) for nm in ("DQ", "w", "IUQ", "UQ", "UQ_hca")}
    chunks = []
    for c0 in range(0, n_pref, chunk):
        h = torch.cat([hidden_rows(cfg, b, n_tot, n_ctx - n_pref + c0, n_ctx - n_pref + c0 + chunk, dev)
                       for b in range(B)])                                  # [B*chunk][d]
        cQ = dlc.dlc_project(h, Wq["DQ"])
        chunks.append(dict(
            qI=dlc.dlc_project(cQ, Wq["IUQ"]).reshape(B, chunk, n_hI, cI),
            wI=dlc.dlc_project(h, Wq["w"], out_dtype=torch.float32).reshape(B, chunk, n_hI),
            q=dlc.dlc_project(cQ, Wq["UQ"]).reshape(B, chunk, n_h, c),
            qh=dlc.dlc_project(cQ, Wq["UQ_hca"]).reshape(B, chunk, n_h, c),
            t=torch.arange(n_ctx - n_pref + c0, n_ctx - n_pref + c0 + chunk, device=dev,
                           dtype=torch.int64)[None].expand(B, chunk).contiguous()))
        del h, cQ
    ws_i = torch.zeros(max(dlc.csa_index_topk_ws(B, chunk, wl["cap_csa"], k),
                           dlc.csa_index_topk_fp4_ws(B, chunk, n_hI, cI, wl["cap_csa"], k)), dtype=torch.uint8,
                       device=dev)
    ws_c = torch.empty(max(1, dlc.csa_attend_ws(B, chunk, n_h, c, k)), dtype=torch.uint8, device=dev)
    ws_h = torch.empty(max(1, dlc.hca_attend_ws(B, chunk, n_h, c, wl["cap_hca"])), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, chunk, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, chunk), dtype=torch.int32, device=dev)
    o1 = torch.empty((B, chunk, n_h, c), dtype=torch.float32, device=dev)
    l1 = torch.empty((B, chunk, n_h), dtype=torch.float32, device=dev)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)

    def run(q, evs=None):
        t_max = int(q["t"].max())
        if evs is not None:
            binding.dlc_timing_arm(binding.STAGE_INDEX_SCORES, evs[0], evs[1])
        if fp4:
            dlc.csa_index_topk_fp4(q["qI"], q["wI"], KIc, KIs, q["t"], t_max, m, k, idx=idx, count=cnt, ws=ws_i)
        else:
            dlc.csa_index_topk(q["qI"], q["wI"], KI, q["t"], t_max, m, k, idx=idx, count=cnt, ws=ws_i)
        if evs is not None:
            binding.dlc_timing_arm(binding.STAGE_CSA_ATTEND, evs[2], evs[3])
        dlc.csa_attend(q["q"], Cc, idx, cnt, out=o1, lse=l1, ws=ws_c)
        if evs is not None:
            binding.dlc_timing_arm(binding.STAGE_HCA_ATTEND, evs[4], evs[5])
        dlc.hca_attend(q["qh"], Ch, q["t"], t_max, mp, out=o2, lse=l2, ws=ws_h)

    run(chunks[0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for q in chunks:
        run(q)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    # a second pass with the scores kernel and the two attentions bracketed by HIP events
    scores_ms, csa_ms, hca_ms = [], [], []
    for q in chunks:
        evs = [ev.create() for _ in range(6)]
        run(q, evs)
        torch.cuda.synchronize()
        scores_ms.append(ev.elapsed_ms(evs[0], evs[1]))
        csa_ms.append(ev.elapsed_ms(evs[2], evs[3]))
        hca_ms.append(ev.elapsed_ms(evs[4], evs[5]))
        for e in evs:
            ev.destroy(e)
    vis = sum((t // m) for t in range(n_ctx - n_pref, n_ctx)) * B
    idx_flop = 2.0 * vis * n_hI * cI
    hca_flop = 4.0 * sum((t // mp) for t in range(n_ctx - n_pref, n_ctx)) * B * n_h * c
    return dict(total_ms=total_ms, scores_ms=sum(scores_ms), csa_ms=sum(csa_ms), hca_ms=sum(hca_ms),
                idx_flop=idx_flop, hca_flop=hca_flop, n_pref=n_pref, chunk=chunk)


def step_bytes(cfg, t, fp4=False):
    """Algorithmic HBM bytes of one decode step (B queries at position t).  The
    second value is the indexer scores kernel's share: every visible K^I row
    (bf16, or MXFP4 codes + scales), the query and its head weights."""
    B, c, cI, m, mp, k, n_h, n_hI = cfg.B, cfg.c, cfg.cI, cfg.m, cfg.m_prime, cfg.k, cfg.n_h, cfg.n_hI
    v_csa, v_hca = t // m, t // mp
    row_i = cI // 2 + cI // 32 if fp4 else cI * 2
    idx_b = v_csa * row_i + n_hI * row_i + n_hI * 4
    csa_b = min(k, v_csa) * c * 2 + n_h * c * 2 + n_h * c * 4 + n_h * 4
    hca_b = v_hca * c * 2 + n_h * c * 2 + n_h * c * 4 + n_h * 4
    comp = 0
    if (t + 1) % m == 0:
        comp += (4 * m * c * 2 + c * 2) + (4 * m * cI * 2 + cI * 2)
        if fp4:
            comp += cI * 2 + cI // 2 + cI // 32
    if (t + 1) % mp == 0:
        comp += 2 * mp * c * 2 + c * 2
    return B * (idx_b + csa_b + hca_b + comp), B * idx_b


def percentiles(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 5), "median": round(float(np.median(a)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def timed_calls(fn, n, warmup=3):
    """fn(i) enqueues one step; returns (mean ms over n steps from one event pair,
    per-step ms from a second pass with an event pair around every step)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    mean_ms = e0.elapsed_time(e1) / n
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return mean_ms, [a.elapsed_time(b) for a, b in evs]


def stage_configs(dev, n, n_sets=3):
    """Configs csa128k (csa_index_topk + csa_attend, B = 8 queries at t = 131072
    over 32768 entries) and hca1m (hca_attend, B = 16 queries at t = 2^20 over
    8192 entries), inputs ~N(0,1) drawn as the configs state, n_sets cache sets
    rotating per step so the caches stream from HBM."""
    import torch

    import dense_long_context_amd as dlc
    import synth
    from synth import get_config

    out = {}
    # ---- csa128k
    cfg = get_config("csa128k")
    B, c, cI, m, k, t, n_h, n_hI = cfg.B, cfg.c, cfg.cI, cfg.m, cfg.k, cfg.t, cfg.n_h, cfg.n_hI
    nv = t // m
    ts = synth.tensor_seed
    sets = []
    for i in range(n_sets):
        Cc = synth.normal_chunked_rows(B * nv, c, ts(cfg.seed, "Ccomp") + 100 * i, 1.0, "bf16", dev).reshape(B, nv, c)
        KI = synth.normal_chunked_rows(B * nv, cI, ts(cfg.seed, "KI") + 100 * i, 1.0, "bf16", dev).reshape(B, nv, cI)
        sets.append((Cc, KI))
    q = synth.normal((B, 1, n_h, c), ts(cfg.seed, "q"), dtype="bf16", device=dev)
    qI = synth.normal((B, 1, n_hI, cI), ts(cfg.seed, "qI"), dtype="bf16", device=dev)
    wI = synth.normal((B, 1, n_hI), ts(cfg.seed, "wI"), dtype="f32", device=dev)
    tt = torch.full((B, 1), t, dtype=torch.int64, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, 1), dtype=torch.int32, device=dev)
    o = torch.empty((B, 1, n_h, c), device=dev)
    lse = torch.empty((B, 1, n_h), device=dev)
    ws_i = torch.zeros(dlc.csa_index_topk_ws(B, 1, nv, k), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, dlc.csa_attend_ws(B, 1, n_h, c, k)), dtype=torch.uint8, device=dev)

    def csa_step(i):
        Cc, KI = sets[i % n_sets]
        dlc.csa_index_topk(qI, wI, KI, tt, t, m, k, idx=idx, count=cnt, ws=ws_i)
        dlc.csa_attend(q, Cc, idx, cnt, out=o, lse=lse, ws=ws_c)
    mean_ms, per = timed_calls(csa_step, n)
    byts = B * (nv * cI * 2 + n_hI * cI * 2 + 4 * n_hI + min(k, nv) * c * 2 + n_h * c * 2 + 4 * n_h * c + 4 * n_h)
    out["csa128k"] = {"workload": "csa128k decode: csa_index_topk + csa_attend, B=8 queries at t=131072 "
                                  "(32768 entries), k=1024, n_h=128, c=512, n_hI=64, cI=128",
                      "query_tokens_per_s": round(B / (mean_ms * 1e-3), 1), "ms_per_step": round(mean_ms, 5),
                      "ms_per_step_events": percentiles(per),
                      "algorithmic_bytes_per_step": int(byts),
                      "hbm_gbs": round(byts / (mean_ms * 1e-3) / 1e9, 1),
                      "frac_of_8tbs": round(byts / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del sets, ws_i, ws_c
    torch.cuda.empty_cache()
    # ---- hca1m
    cfg = get_config("hca1m")
    B, c, mp, t, n_h = cfg.B, cfg.c, cfg.m_prime, cfg.t, cfg.n_h
    nv = t // mp
    caches = [synth.normal_chunked_rows(B * nv, c, ts(cfg.seed, "Chca") + 100 * i, 1.0, "bf16", dev).reshape(B, nv, c)
              for i in range(n_sets)]
    q = synth.normal((B, 1, n_h, c), ts(cfg.seed, "q"), dtype="bf16", device=dev)
    tt = torch.full((B, 1), t, dtype=torch.int64, device=dev)
    o = torch.empty((B, 1, n_h, c), device=dev)
    lse = torch.empty((B, 1, n_h), device=dev)
    ws_h = torch.empty(max(1, dlc.hca_attend_ws(B, 1, n_h, c, nv)), dtype=torch.uint8, device=dev)

    def hca_step(i):
        dlc.hca_attend(q, caches[i % n_sets], tt, t, mp, out=o, lse=lse, ws=ws_h)
    mean_ms, per = timed_calls(hca_step, n)
    byts = B * (nv * c * 2 + n_h * c * 2 + 4 * n_h * c + 4 * n_h)
    flop = B * 4.0 * nv * n_h * c
    out["hca1m"] = {"workload": "hca1m decode: hca_attend, B=16 queries at t=2^20 over 8192 entries, n_h=128, c=512",
                    "query_tokens_per_s": round(B / (mean_ms * 1e-3), 1), "ms_per_step": round(mean_ms, 5),
                    "ms_per_step_events": percentiles(per),
                    "algorithmic_bytes_per_step": int(byts), "algorithmic_flop_per_step": int(flop),
                    "hbm_gbs": round(byts / (mean_ms * 1e-3) / 1e9, 1),
                    "frac_of_8tbs": round(byts / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "tflops": round(flop / (mean_ms * 1e-3) / 1e12, 1),
                    "mfma_frac": round(flop / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "bound_note": "at 8 TB/s the 140.5 MB take 17.6 us, at 2.5 PFLOP/s the 34.4 GFLOP 13.7 us: "
                                  "even HBM-bound at peak the MFMA fraction is at most 0.78"}
    del caches, ws_h
    torch.cuda.empty_cache()
    return out


def query_projections(cfg, wl, n):
    """The decode queries' projections of one step (B tokens): c^Q = h W^DQ,
    q^I = c^Q W^IUQ, w^I = h W^w, q = c^Q W^UQ and the HCA q, all dlc_project."""
    import torch

    import dense_long_context_amd as dlc

    B, d = cfg.B, cfg.d
    H = wl["H_dec"]                      # [B][n_dec][d]
    Wq = wl["Wq"]
    n_dec = H.shape[1]
    hs = [H[:, s].contiguous() for s in range(min(n, n_dec))]
    cQ = torch.empty((B, cfg.d_c), dtype=torch.bfloat16, device=H.device)
    qI = torch.empty((B, cfg.n_hI * cfg.cI), dtype=torch.bfloat16, device=H.device)
    wI = torch.empty((B, cfg.n_hI), dtype=torch.float32, device=H.device)
    q = torch.empty((B, cfg.n_h * cfg.c), dtype=torch.bfloat16, device=H.device)
    qh = torch.empty_like(q)

    from dense_long_context_amd import binding

    # one workspace for the five calls (each leaves it zeroed): the k-split of
    # the row path where a projection has few output columns
    ws_n = max(dlc.dlc_project_ws(B, W.shape[0], W.shape[1]) for W in Wq.values())
    ws = torch.zeros(max(ws_n, 1), dtype=torch.uint8, device=H.device)
    # the C-ABI argument tuples, marshalled once (as the decode steps are)
    L = binding.lib()
    stream = torch.cuda.current_stream(H.device).cuda_stream

    def call(A, W, out):
        M, K = A.shape
        N = W.shape[0]
        dt = binding.DLC_F32 if out.dtype == torch.float32 else binding.DLC_BF16
        return (binding.DLC_BF16, M, N, K, A.data_ptr(), K, W.data_ptr(), K, out.data_ptr(), N, dt,
                ws.data_ptr(), ws.numel(), stream)
    calls = [[call(h, Wq["DQ"], cQ), call(cQ, Wq["IUQ"], qI), call(h, Wq["w"], wI), call(cQ, Wq["UQ"], q),
              call(cQ, Wq["UQ_hca"], qh)] for h in hs]

    def step(i):
        for a in calls[i % len(calls)]:
            rc = L.dlc_project(*a)
            if rc != 0:
                raise RuntimeError(binding.last_error())
    mean_ms, per = timed_calls(step, n)
    wbytes = 2 * (d * cfg.d_c + cfg.d_c * cfg.n_hI * cfg.cI + d * cfg.n_hI + 2 * cfg.d_c * cfg.n_h * cfg.c)
    flop = 2.0 * B * (d * cfg.d_c + cfg.d_c * cfg.n_hI * cfg.cI + d * cfg.n_hI + 2 * cfg.d_c * cfg.n_h * cfg.c)
    return {"ms_per_step": round(mean_ms, 5), "ms_per_step_events": percentiles(per),
            "weight_bytes_per_step": int(wbytes), "weight_gbs": round(wbytes / (mean_ms * 1e-3) / 1e9, 1),
            "tflops": round(flop / (mean_ms * 1e-3) / 1e12, 2),
            "note": "dlc_project x5 for the B decode tokens of a step (c^Q, q^I, w^I, q, HCA q) on the row-vector "
                    "path with a k-split workspace; weight-read bound at this batch; outside the compressed-attention "
                    "step and its value"}


def run_steps(steps, s0, n, n_dec):
    for j in range(s0, s0 + n):
        for fn, args in steps[j % n_dec][1]:
            rc = fn(*args)
            if rc != 0:
                from dense_long_context_amd import binding
                raise RuntimeError(f"{fn.__name__} failed: {binding.last_error()}")


def blas_info():
    """Threads and library of the BLAS numpy runs on, and the host's core counts."""
    info = {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["threads"] = int(max(i.get("num_threads", 1) for i in blas))
    except Exception:  # pragma: no cover
        pass
    info.setdefault("threads", info["affinity"])
    return info


def cpu_baseline(cfg, wl, steps, s_first, n_steps, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample of the GPU line's own
    decode steps: the same query rows (copied to the host) against the same
    caches (sequences 0 and 1; every cache set holds the same values), one
    query at a time: indexer scores over all visible entries, top-k, CSA
    attention over the rows the oracle selects, HCA attention over every
    visible entry.  Only the oracle calls are timed."""
    import numpy as np
    import torch

    import oracle as O

    m, mp, k = cfg.m, cfg.m_prime, cfg.k
    Cc, KI, Ch = wl["sets"][0][:3]
    Q = wl["Q"]
    host = {}
    for b in (0, 1):
        host[b] = (KI[b].cpu(), Cc[b].cpu(), Ch[b].cpu())
    done, spent = 0, 0.0
    n_dec = len(steps)
    j = 0
    while spent < budget_s and j < 4 * n_steps:
        s = (s_first + j // 2) % n_dec
        b = j % 2
        t = steps[s][0]
        KIh, Cch, Chh = host[b]
        qI, wI = Q["qI"][s][b, 0].cpu(), Q["wI"][s][b, 0].cpu()
        q, qh = Q["q"][s][b, 0].cpu(), Q["qh"][s][b, 0].cpu()
        t0 = time.perf_counter()
        sc = O.index_scores(qI, wI, KIh[:t // m], t, m)
        sel = O.topk_select(sc, k)
        t1 = time.perf_counter()
        rows = Cch[torch.as_tensor(sel)]                    # the selected entries (host gather, untimed)
        t2 = time.perf_counter()
        O.csa_attend(q, rows, np.arange(len(sel)))
        O.hca_attend(qh, Chh, t, mp)
        t3 = time.perf_counter()
        spent += (t1 - t0) + (t3 - t2)
        done += 1
        j += 1
    bi = blas_info()
    return {"value": done / spent, "unit": "decode query-tokens/s", "cores": int(bi["threads"]), "kind": "oracle",
            "host": bi,
            "sample": f"{done} decode queries of the timed steps (sequences 0 and 1, t = {steps[s_first][0]} ..): "
                      f"indexer over all floor(t/m) entries, top-{k}, CSA attention over the selected entries, "
                      f"HCA attention over floor(t/m') entries; fp64 numpy on the GPU line's own query rows and "
                      f"caches, {spent:.1f} s of oracle time; the per-step compressor work (one entry every m "
                      f"tokens) is left out"}


PMC_COPY_BYTES = 1 << 30


def pmc_probe():
    """The decode-shaped indexer call (B = 4, 262208-entry caches in three
    rotating sets, t = 2^20) six times, then a copy of PMC_COPY_BYTES (four
    times the 256 MB last-level cache) three times and a read of another
    PMC_COPY_BYTES in the scores kernel's load form (dlc_read, tile form) three
    times: the program the FETCH_SIZE / WRITE_SIZE counter runs profile."""
    import torch

    from dense_long_context_amd import binding
    import synth
    from synth import get_config

    cfg = get_config("hybrid1m")
    dev = torch.device("cuda:0")
    B, cI, m, k, n_hI = cfg.B, cfg.cI, cfg.m, cfg.k, cfg.n_hI
    cap = (cfg.t + cfg.n_decode) // m
    sets = [synth.normal((B, cap, cI), 7000 + i, dtype="bf16", device=dev) for i in range(3)]
    qI = synth.normal((B, 1, n_hI, cI), 7010, dtype="bf16", device=dev)
    wI = synth.normal((B, 1, n_hI), 7011, dtype="f32", device=dev)
    t = torch.full((B, 1), cfg.t, dtype=torch.int64, device=dev)
    ws = torch.empty(binding.csa_index_topk_ws(B, 1, cap, k), dtype=torch.uint8, device=dev)
    # the copy's source is written first, so that the indexer's 800 MB of key
    # streams have pushed it out of the caches before it is copied
    a = torch.ones(PMC_COPY_BYTES, dtype=torch.uint8, device=dev)
    r = torch.ones(PMC_COPY_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for i in range(6):
        binding.csa_index_topk(qI, wI, sets[i % 3], t, cfg.t, m, k, ws=ws)
    for _ in range(3):
        binding.dlc_copy(b, a)
    for _ in range(3):
        binding.dlc_read(r, binding.READ_TILES)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": "done", "scores_bytes_per_launch": step_bytes(cfg, cfg.t)[1],
                      "copy_bytes": PMC_COPY_BYTES}), flush=True)


def _counter_kib(csv_path, kernel_part, counter):
    """Per-dispatch values (KiB) of ``counter`` for kernels whose name contains
    ``kernel_part``, from a rocprofv3 counter_collection CSV."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if kernel_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(per.values())


def ingest_pmc(fetch_csv, write_csv):
    """HBM bytes per launch of the scores kernel: FETCH_SIZE scaled by what the
    counter reads for the read kernel (PMC_COPY_BYTES loaded the way the scores
    kernel loads its keys: 16-byte register loads in the MFMA operand pattern),
    and WRITE_SIZE scaled by what it reads for the copy kernel's plain stores."""
    from synth import get_config

    cfg = get_config("hybrid1m")
    f_sc = _counter_kib(fetch_csv, "scores_reg_kernel", "FETCH_SIZE")
    f_cp = _counter_kib(fetch_csv, "copy_kernel", "FETCH_SIZE")
    f_rd = _counter_kib(fetch_csv, "read_tiles_kernel", "FETCH_SIZE")
    w_sc = _counter_kib(write_csv, "scores_reg_kernel", "WRITE_SIZE")
    w_cp = _counter_kib(write_csv, "copy_kernel", "WRITE_SIZE")
    if not (f_sc and f_cp and f_rd and w_sc and w_cp):
        raise SystemExit("counter CSVs lack the scores, copy or read kernel dispatches")
    # the first launch of each cache set is cold; the profiled launches rotate 3 sets
    copy_fetch_factor = (sum(f_cp) / len(f_cp)) * 1024 / PMC_COPY_BYTES
    fetch_factor = (sum(f_rd) / len(f_rd)) * 1024 / PMC_COPY_BYTES
    write_factor = (sum(w_cp) / len(w_cp)) * 1024 / PMC_COPY_BYTES
    fetch = (sum(f_sc) / len(f_sc)) * 1024 / fetch_factor
    write = (sum(w_sc) / len(w_sc)) * 1024 / write_factor
    out = {"kernel": SCORES_KERNEL, "workload": "hybrid1m decode indexer, B=4, 262144 visible entries",
           "source_hash": source_hash(), "fetch_kib_per_dispatch": sum(f_sc) / len(f_sc),
           "write_kib_per_dispatch": sum(w_sc) / len(w_sc), "read_fetch_factor": fetch_factor,
           "copy_fetch_factor": copy_fetch_factor,
           "copy_write_factor": write_factor, "fetch_bytes_per_launch": int(fetch),
           "write_bytes_per_launch": int(write), "hbm_bytes_per_launch": int(fetch + write),
           "algorithmic_bytes_per_launch": step_bytes(cfg, cfg.t)[1], "dispatches": len(f_sc)}
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the csa128k and hca1m lines")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused projection + pooling set-up pass")
    ap.add_argument("--prefill-only", action="store_true",
                    help="build the caches, run only the chunked prefill (bf16 and FP4 indexer) and print its JSON")
    ap.add_argument("--repeat", type=int, default=1, help="time the K steps this many times, report the best")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run only the indexer on the decode shapes plus a copy kernel of known size "
                         "(the short program that rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE profile)")
    ap.add_argument("--configs-only", action="store_true",
                    help="run only the csa128k and hca1m lines (the program their rocprofv3 profiles run)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic of the scores kernel from two rocprofv3 counter CSVs")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the CSA/HCA hot path here is single-device "
              "(multi-GPU sharding is a design note, not part of this build).", file=sys.stderr)
        sys.exit(2)

    if args.pmc_probe:
        pmc_probe()
        return
    if args.configs_only:
        import torch
        print(json.dumps({"configs": stage_configs(torch.device("cuda:0"), max(args.steps, 20))}), flush=True)
        return

    import torch

    import dense_long_context_amd as dlc
    from dense_long_context_amd import binding
    from synth import get_config

    cfg = get_config("hybrid1m")
    dev = torch.device("cuda:0")
    n_dec = cfg.n_decode
    log("building the 2^20-token caches (projection + compressors)")
    wl = build_workload(cfg, dev, n_dec)
    log(f"set-up: projection {wl['t_proj']:.2f} s, compressors {wl['t_comp']*1e3:.1f} ms per cache set")
    ev = HipEvents()
    if args.prefill_only:
        out = {}
        for name, fp4 in (("bf16_indexer", False), ("fp4_indexer", True)):
            pf = prefill_pass(cfg, wl, dev, ev=ev, fp4=fp4)
            out[name] = {"ms": round(pf["total_ms"], 3), "indexer_ms": round(pf["scores_ms"], 3),
                         "csa_attend_ms": round(pf["csa_ms"], 3), "hca_attend_ms": round(pf["hca_ms"], 3),
                         "queries": cfg.B * pf["n_pref"]}
        print(json.dumps({"prefill": out}), flush=True)
        return
    steps, keep = make_steps(cfg, wl, dev, n_dec)

    run_steps(steps, 0, args.warmup, n_dec)
    torch.cuda.synchronize()
    K = args.steps

    def timed(armed, steps=steps):
        """K steps between a barrier-free pair of stream events.  armed: also
        time every launch of the scores kernel with its own HIP events."""
        evs = [(ev.create(), ev.create()) for _ in range(K)] if armed else []
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for j in range(K):
            s = args.warmup + j
            if armed:
                binding.dlc_timing_arm(binding.STAGE_INDEX_SCORES, evs[j][0], evs[j][1])
            for fn, a in steps[s % n_dec][1]:
                rc = fn(*a)
                if rc != 0:
                    raise RuntimeError(binding.last_error())
        stop.record()
        torch.cuda.synchronize()
        k_ms = [ev.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            ev.destroy(a)
            ev.destroy(b)
        return start.elapsed_time(stop), k_ms

    # the step rate is taken without the per-kernel events (their records add
    # gaps to the stream); the same K steps then run again with the scores
    # kernel timed launch by launch
    best = None
    for rep in range(args.repeat):
        ms, _ = timed(False)
        ms_armed, k_ms = timed(True)
        if best is None or ms < best[0]:
            best = (ms, k_ms, ms_armed)
    ms, k_ms, ms_armed = best
    # per-step spread: the same steps once more with an event pair around each
    _, step_ms = timed_calls(lambda j: run_steps(steps, args.warmup + j, 1, n_dec), K, warmup=0)
    # the same steps with each layer's sliding-window branch joined in (reported beside the main line)
    steps_w, keep_w = make_steps(cfg, wl, dev, n_dec, window=True)
    run_steps(steps_w, 0, args.warmup, n_dec)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(steps_w, args.warmup, K, n_dec)
    e1.record()
    torch.cuda.synchronize()
    ms_win = e0.elapsed_time(e1)
    del keep_w
    # the same steps with the FP4 (MXFP4) indexer (reported beside the main line)
    steps_f, keep_f = make_steps(cfg, wl, dev, n_dec, fp4=True)
    run_steps(steps_f, 0, args.warmup, n_dec)
    torch.cuda.synchronize()
    ms_f, _ = timed(False, steps_f)
    _, kf_ms = timed(True, steps_f)
    del keep_f
    ts = [steps[(args.warmup + j) % n_dec][0] for j in range(K)]
    total_bytes = sum(step_bytes(cfg, t)[0] for t in ts)
    idx_bytes = sum(step_bytes(cfg, t)[1] for t in ts) / K
    k_avg_ms = sum(k_ms) / len(k_ms)
    achieved = idx_bytes / (k_avg_ms * 1e-3) / 1e9
    ms_step = ms / K
    value = cfg.B * K / (ms * 1e-3)
    idx_bytes_f = sum(step_bytes(cfg, t, fp4=True)[1] for t in ts) / K
    kf_avg_ms = sum(kf_ms) / len(kf_ms)
    achieved_f = idx_bytes_f / (kf_avg_ms * 1e-3) / 1e9
    hbm_gbs = total_bytes / (ms * 1e-3) / 1e9

    # copy-kernel reference for achievable bandwidth
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        binding.dlc_copy(b, a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        binding.dlc_copy(b, a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b

    # read-only reference: dlc_read in the scores kernel's own load form over
    # the same number of bytes, three rotating buffers (past the last-level
    # cache), one HIP event pair per launch bound to the kernel's dispatch, as
    # for the scores kernel
    nb = (int(idx_bytes) + 4095) // 4096 * 4096
    rbufs = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(3)]
    for i in range(3):
        binding.dlc_read(rbufs[i], binding.READ_TILES)
    torch.cuda.synchronize()
    read_ms = []
    for i in range(30):
        e0, e1 = ev.create(), ev.create()
        binding.dlc_timing_arm(binding.STAGE_READ, e0, e1)
        binding.dlc_read(rbufs[i % 3], binding.READ_TILES)
        torch.cuda.synchronize()
        read_ms.append(ev.elapsed_ms(e0, e1))
        ev.destroy(e0)
        ev.destroy(e1)
    read_avg_ms = sum(read_ms) / len(read_ms)
    read_gbs = nb / (read_avg_ms * 1e-3) / 1e9
    del rbufs

    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        if cnt.get("source_hash") == source_hash():
            traffic = cnt.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "decode query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hybrid1m decode: one CSA + one HCA layer, B=4 sequences at 2^20 context "
                               "(t = 2^20 .. 2^20+255), c=512 m=4 m'=128 k=1024 n_h=128 n_hI=64 cI=128, "
                               "caches built from d=7168 hidden states",
                   "global_batch": cfg.B, "seq_len": wl["n_ctx"], "parallelism": "single GPU"},
        "roofline": {"kernel": SCORES_KERNEL, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(k_avg_ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(idx_bytes),
                     "read_reference": {"kernel": "dlc_read (tile form)", "bytes": nb,
                                        "avg_launch_us": round(read_avg_ms * 1e3, 3), "gbs": round(read_gbs, 1),
                                        "kernel_frac_of_it": round(achieved / read_gbs, 4),
                                        "note": "a read of the same bytes in the scores kernel's load form, "
                                                "nothing else, timed the same way"}},
        "ms_per_step_events": percentiles(step_ms),
        "ms_per_step_with_kernel_events": round(ms_armed / K, 5),
        "with_sliding_window": {"value": round(cfg.B * K / (ms_win * 1e-3), 1), "ms_per_step": round(ms_win / K, 5),
                                "n_win": N_WIN, "note": "csa_attend_window / hca_attend_window: each layer's "
                                                        "128-token window joined to its compressed keys"},
        "with_fp4_indexer": {"value": round(cfg.B * K / (ms_f * 1e-3), 1), "ms_per_step": round(ms_f / K, 5),
                             "scores_kernel": SCORES_KERNEL_FP4, "scores_avg_launch_us": round(kf_avg_ms * 1e3, 3),
                             "scores_achieved_gbs": round(achieved_f, 1),
                             "scores_frac": round(achieved_f / PEAK_HBM_GBS, 4),
                             "scores_algorithmic_bytes_per_launch": int(idx_bytes_f),
                             "note": "csa_index_topk_fp4 on the MXFP4 K^I cache (68 B per entry: 64 code bytes + "
                                     "4 E8M0 scales); new entries quantized as they are written; the top-k set "
                                     "differs from the bf16 indexer's by the FP4 rounding of the scores"},
        "step_hbm_gbs": round(hbm_gbs, 1),
        "step_frac_of_peak": round(hbm_gbs / PEAK_HBM_GBS, 4),
        "copy_kernel_gbs": round(copy_gbs, 1),
        "setup": {"projection_s": round(wl["t_proj"], 3), "compress_ms_per_cache_set": round(wl["t_comp"] * 1e3, 2),
                  "compress_stream_gbs": round(wl["stream_bytes"] / wl["t_comp"] / 1e9, 1),
                  "compress_passes": {nm: {"ms": round(t * 1e3, 3), "gbs": round(nb / t / 1e9, 1),
                                           "frac_of_8tbs": round(nb / t / 1e9 / PEAK_HBM_GBS, 4)}
                                      for nm, t, nb in zip(("csa_kv", "csa_index_keys", "hca"), wl["t_stage"],
                                                           wl["stage_bytes"])},
                  "compress_note": "full passes over the side-by-side stream buffer, HIP events around each call, "
                                   "the median of the cache sets; bytes are the streams read plus the entries "
                                   "written"},
    }
    if not args.no_fused:
        log("fused projection + pooling pass")
        t_fused, same = fused_setup(cfg, wl, dev)
        flops = 2.0 * cfg.B * wl["n_tot"] * cfg.d * stream_layout(cfg)[2]
        result["setup"].update({
            "projection_kernel_s": round(wl["t_proj_kernel"], 3),
            "projection_tflops": round(flops / wl["t_proj_kernel"] / 1e12, 1),
            "two_pass_kernel_s": round(wl["t_proj_kernel"] + wl["t_comp"], 3),
            "fused_kernel_s": round(t_fused, 3),
            "fused_equals_two_pass": bool(same),
        })
    log("decode query projections")
    result["query_projection"] = query_projections(cfg, wl, K)
    if not args.no_configs:
        log("configs csa128k and hca1m")
        result["configs"] = stage_configs(dev, max(K, 20))
    if not args.no_prefill:
        log("chunked causal prefill of 4096 queries per sequence")
        pf = prefill_pass(cfg, wl, dev, ev=ev)
        result["prefill"] = {
            "queries": cfg.B * pf["n_pref"], "chunk_per_sequence": pf["chunk"], "ms": round(pf["total_ms"], 3),
            "query_tokens_per_s": round(cfg.B * pf["n_pref"] / (pf["total_ms"] * 1e-3), 1),
            "indexer_ms": round(pf["scores_ms"], 3),
            "indexer_tflops": round(pf["idx_flop"] / (pf["scores_ms"] * 1e-3) / 1e12, 1),
            "indexer_mfma_frac": round(pf["idx_flop"] / (pf["scores_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "csa_attend_ms": round(pf["csa_ms"], 3), "hca_attend_ms": round(pf["hca_ms"], 3),
            "hca_attend_tflops": round(pf["hca_flop"] / (pf["hca_ms"] * 1e-3) / 1e12, 1),
            "note": "t = 2^20-4096 .. 2^20-1, causal against the full caches; the indexer runs query-tiled "
                    "(scores_prefill_kernel, v_mfma_f32_32x32x16_bf16) at 256 queries per sequence per call, the "
                    "cache in ranges of 32768 entries; indexer_ms is the whole indexer (every range's scores, "
                    "selection and merge), indexer_tflops the score FLOPs over that time"}
        pf4 = prefill_pass(cfg, wl, dev, ev=ev, fp4=True)
        result["prefill"]["with_fp4_indexer"] = {
            "ms": round(pf4["total_ms"], 3),
            "query_tokens_per_s": round(cfg.B * pf4["n_pref"] / (pf4["total_ms"] * 1e-3), 1),
            "indexer_ms": round(pf4["scores_ms"], 3),
            "indexer_tflops": round(pf4["idx_flop"] / (pf4["scores_ms"] * 1e-3) / 1e12, 1),
            "note": "csa_index_topk_fp4 (scores_prefill_fp4_kernel, v_mfma_scale_f32_32x32x64_f8f6f4) on the "
                    "MXFP4 key cache"}
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(cfg, wl, steps, args.warmup, K)
    else:
        result["cpu_baseline"] = None
    del keep
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
