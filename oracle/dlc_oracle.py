"""fp64 CPU oracle: what the CSA/HCA hot path computes, written out plainly.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Sources, cited by page title and section:

* [Scratch] "DeepSeek-V4 Hybrid Attention: CSA and HCA from Scratch"
  (prathamp.com).  The authority on what the method computes.
* [Stack] "DeepSeek's attention stack: how DSA, CSA, HCA and mHC fit
  together" (dev.to).  Hyper-parameters and context only.
* [Evolution] "From MHA, GQA to MLA, DSA, HCA/CSA" (bhhxx.wiki, Chinese).
  A second formula source; where it differs from [Scratch], [Scratch] wins.

Everything is numpy float64.  Inputs stored in bf16 or fp32 are upcast
exactly.  Where the method stores an intermediate (projected streams,
compressed caches, queries), ``store`` mirrors that rounding so an
end-to-end chain sees the same values a device that stores them would.

Readings of points the pages leave open (each listed in the design notes):

* joint softmax over all 2m rows of a CSA window ([Scratch] §4), not two
  separate block softmaxes as [Evolution] §6.2.2 writes;
* the i = 0 window's missing b-rows are excluded from the softmax (their
  logit is -inf and weight exactly 0, [Scratch] §4 "Block i = 0");
* visibility s < floor(t/m) for CSA and s < floor(t/m') for HCA
  ([Scratch] §7 and §10);
* k larger than the visible count keeps everything (k_eff = min(k, vis));
* top-k ties: larger score first, then smaller index; -0.0 equals +0.0;
* nothing visible: output 0 and log-sum-exp -inf;
* both attentions scale logits by 1/sqrt(c) ([Scratch] §8, applied to HCA
  through the unified operator of §11); the indexer is unscaled (§6.4);
* the sliding-window branch ([Evolution] §6.1-6.2, n_win = 128 per [Stack]
  §4) covers the n_win most recent tokens including the query token itself,
  uses the same scale, and is joined to the compressed branch as one
  attention over both key sets (no entry is removed from either set);
* the FP4 indexer ([Scratch] §6.4 and §12 say the indexer's products run in
  FP4 without naming a format) uses the OCP microscaling MXFP4 format: E2M1
  elements, one power-of-two (E8M0) scale per 32 consecutive elements of a
  row, shared exponent floor(log2(block max |x|)) - 2, elements rounded to
  the nearest E2M1 value with ties to the even code and saturated at 6; a
  zero element is stored as +0.  Both q^I and K^I are quantized this way and
  the score is the exact fp64 value of the formula on the dequantized
  operands (w^I stays fp32);
* [Evolution] §6.2 derives the indexer key from the compressed KV entry,
  k^I_u = c^comp_u W^I_k, and the indexer query from the hidden state,
  q^I_{t,j} = h_t W^I_{q,j}; [Scratch] §6.2-6.4 instead compresses separate
  indexer streams and up-projects c^Q.  Both derivations feed the same
  scoring formula;
* sink logits ([Scratch] §12 names them without a formula) are read as one
  logit z_h per head that joins the softmax as an extra key whose value is
  the zero vector: it takes probability mass and contributes nothing.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "f64",
    "round_bf16",
    "store_as",
    "project",
    "column_softmax",
    "csa_window_weights",
    "csa_compress",
    "hca_window_weights",
    "hca_compress",
    "csa_visible",
    "hca_visible",
    "index_scores",
    "topk_select",
    "mqa_attend",
    "csa_attend",
    "hca_attend",
    "window_positions",
    "window_attend",
    "merge_lse",
    "split_heads",
    "queries_from_hidden",
    "decode_chain",
    "gqa_kv_bytes_per_token_layer",
    "compressed_bytes_per_token_layer",
    "ledger",
    "indexer_flops_per_query",
    "MXFP4_BLOCK",
    "E2M1_MAGNITUDES",
    "mxfp4_quantize",
    "mxfp4_dequantize",
    "index_scores_fp4",
    "evolution_indexer_keys",
    "evolution_indexer_queries",
    "mqa_attend_with_sink",
    "apply_sink",
]


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16 and fp32 values are all representable)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, which is exact for bf16
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 keeps 8 significant bits.  frexp gives x = f * 2**e with
    0.5 <= |f| < 1, so f * 2**8 lies in [128, 256) and rounding it to an
    integer with ties-to-even (np.rint) keeps exactly 8 significant bits.
    Values here stay far from the bf16 subnormal and overflow ranges.
    """
    x = f64(x)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(f * 256.0), e - 8)


def store_as(x, dtype: str) -> np.ndarray:
    """Mirror the rounding of storing ``x`` in ``dtype`` ('bf16' | 'f32' | 'f64')."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return f64(np.asarray(f64(x), dtype=np.float32))
    if dtype == "f64":
        return f64(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# projections ([Scratch] §3 and §6.1-6.3, §8, §10)
# --------------------------------------------------------------------------

def project(H, W) -> np.ndarray:
    """Dense projection of hidden states, e.g. C^a = H W^{aKV} ([Scratch] §3)."""
    return f64(H) @ f64(W)


def split_heads(v, n_heads: int, width: int) -> np.ndarray:
    """[q_1; ...; q_nh] = v: head h takes columns h*width ... (h+1)*width-1
    ([Scratch] §6.2 and §8 write the heads side by side)."""
    v = f64(v)
    assert v.shape[-1] == n_heads * width
    return v.reshape(v.shape[:-1] + (n_heads, width))


# --------------------------------------------------------------------------
# compressor ([Scratch] §2, §4, §5, §10)
# --------------------------------------------------------------------------

def column_softmax(logits) -> np.ndarray:
    """Softmax down the rows, independently for every column ([Scratch] §4,
    "Softmax_row").  Computed max-subtracted, which is the same value."""
    L = f64(logits)
    e = np.exp(L - L.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def csa_window_weights(Za, Zb, m: int, i: int, Ba=None, Bb=None):
    """Softmax weights of CSA entry i ([Scratch] §4).

    The window stacks the a-rows m*i ... m*(i+1)-1 (current block) over the
    b-rows m*(i-1) ... m*i-1 (previous block); one softmax per column runs
    jointly over all 2m stacked logits Z + B.  For i = 0 the b-rows do not
    exist: their logit is -inf, so they are left out and get weight 0.

    Returns (S_a [m][c], S_b [m][c]); S_b is all zeros for i = 0.
    """
    Za, Zb = f64(Za), f64(Zb)
    c = Za.shape[1]
    Ba = np.zeros((m, c)) if Ba is None else f64(Ba)
    Bb = np.zeros((m, c)) if Bb is None else f64(Bb)
    la = Za[m * i:m * (i + 1)] + Ba
    if i == 0:
        return column_softmax(la), np.zeros((m, c))
    lb = Zb[m * (i - 1):m * i] + Bb
    S = column_softmax(np.vstack([la, lb]))
    return S[:m], S[m:]


def csa_compress(Za, Zb, Ca, Cb, m: int, Ba=None, Bb=None, i_begin: int = 0, i_end=None):
    """CSA compressed entries i_begin ... i_end-1 ([Scratch] §5, boxed formula):

        C^Comp_i = sum_{j in block i} S^a_j (.) C^a_j + sum_{j in block i-1} S^b_j (.) C^b_j
    """
    Za, Zb, Ca, Cb = f64(Za), f64(Zb), f64(Ca), f64(Cb)
    n, c = Za.shape
    if i_end is None:
        i_end = n // m
    assert 0 <= i_begin <= i_end <= n // m
    out = np.zeros((i_end - i_begin, c))
    for i in range(i_begin, i_end):
        Sa, Sb = csa_window_weights(Za, Zb, m, i, Ba, Bb)
        acc = (Sa * Ca[m * i:m * (i + 1)]).sum(axis=0)
        if i > 0:
            acc = acc + (Sb * Cb[m * (i - 1):m * i]).sum(axis=0)
        out[i - i_begin] = acc
    return out


def hca_window_weights(Z, m_prime: int, i: int, B=None):
    """HCA weights of entry i: one softmax per column over the m' rows of the
    non-overlapping block i ([Scratch] §10)."""
    Z = f64(Z)
    c = Z.shape[1]
    B = np.zeros((m_prime, c)) if B is None else f64(B)
    return column_softmax(Z[m_prime * i:m_prime * (i + 1)] + B)


def hca_compress(Z, C, m_prime: int, B=None, i_begin: int = 0, i_end=None):
    """HCA compressed entries ([Scratch] §10, boxed formula):
    C_i = sum_{j in block i} S_j (.) C_j, blocks of m' rows, no overlap."""
    Z, C = f64(Z), f64(C)
    n, c = Z.shape
    if i_end is None:
        i_end = n // m_prime
    assert 0 <= i_begin <= i_end <= n // m_prime
    out = np.zeros((i_end - i_begin, c))
    for i in range(i_begin, i_end):
        S = hca_window_weights(Z, m_prime, i, B)
        out[i - i_begin] = (S * C[m_prime * i:m_prime * (i + 1)]).sum(axis=0)
    return out


# --------------------------------------------------------------------------
# visibility, indexer, selection ([Scratch] §6, §7, §10)
# --------------------------------------------------------------------------

def csa_visible(t: int, m: int) -> int:
    """Number of CSA entries query t may see: s < floor(t/m) ([Scratch] §7)."""
    return t // m


def hca_visible(t: int, m_prime: int) -> int:
    """Number of HCA entries query t may see: s < floor(t/m') ([Scratch] §10)."""
    return t // m_prime


def index_scores(qI, wI, KI, t: int, m: int) -> np.ndarray:
    """Lightning-indexer scores over the visible CSA entries ([Scratch] §6.4):

        I_{t,s} = sum_h w^I_{t,h} * ReLU(q^I_{t,h} . K^IComp_s),   s < floor(t/m)

    No softmax and no scale.  -0.0 is returned as +0.0.
    """
    qI, wI, KI = f64(qI), f64(wI), f64(KI)
    nvis = csa_visible(t, m)
    dots = KI[:nvis] @ qI.T                 # [nvis][n_hI]
    scores = np.maximum(dots, 0.0) @ wI     # [nvis]
    return scores + 0.0


def topk_select(scores, k: int) -> np.ndarray:
    """Indices of the k largest scores, returned in ascending index order
    ([Scratch] §7).  k larger than the candidate count keeps them all.
    Ties: the larger score ranks first, then the smaller index."""
    s = f64(scores)
    n = s.shape[0]
    k_eff = min(int(k), n)
    order = np.lexsort((np.arange(n), -s))  # last key is primary
    return np.sort(order[:k_eff]).astype(np.int64)


# --------------------------------------------------------------------------
# FP4 indexer ([Scratch] §6.4: the indexer's attention runs in FP4, which the
# ReLU makes safe; §12: FP4 indexer FLOPs).  The format is the OCP MXFP4
# reading stated in the module header.
# --------------------------------------------------------------------------

MXFP4_BLOCK = 32
# magnitude of E2M1 codes 0..7 (sign in bit 3): 0, the subnormal 0.5, then
# 1.x * 2^(e-1) for e = 1..3 with one mantissa bit
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_quantize(x):
    """MXFP4 quantization of the last axis in blocks of 32.

    Returns (codes, shared): codes are integers 0..15 with the layout of x
    (bit 3 the sign, bits 0..2 the E2M1 magnitude code), shared the block
    exponents (x.shape[:-1] + (width/32,)), so that an element's value is
    sign * E2M1_MAGNITUDES[code & 7] * 2**shared.

    Per block: shared = floor(log2(max |x|)) - 2, the exponent that puts the
    block maximum in [4, 8), E2M1's top binade; an all-zero block takes the
    smallest E8M0 exponent, -127.  Each element x / 2**shared (exact: a power
    of two) is rounded to the nearest E2M1 magnitude, a tie going to the even
    code (even mantissa), and magnitudes above 6 become 6.
    """
    x = f64(x)
    width = x.shape[-1]
    if width % MXFP4_BLOCK:
        raise ValueError("width must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (width // MXFP4_BLOCK, MXFP4_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)            # amax = f * 2**e with 0.5 <= f < 1
    shared = np.where(amax > 0, (e - 1) - 2, -127)
    shared = np.clip(shared, -127, 127).astype(np.int64)
    y = blocks / np.ldexp(1.0, shared)[..., None]
    # nearest magnitude: scan the grid upwards, keeping the closest so far; an
    # equal distance (a midpoint, between codes c-1 and c) goes to c if c is even
    mag_code = np.zeros(y.shape, dtype=np.int64)
    best = np.full(y.shape, np.inf)
    for c, g in enumerate(E2M1_MAGNITUDES):
        d = np.abs(np.abs(y) - g)
        take = (d < best) | ((d == best) & (c % 2 == 0))
        mag_code = np.where(take, c, mag_code)
        best = np.where(take, d, best)
    negative = (y < 0) & (mag_code > 0)
    codes = (mag_code + 8 * negative).reshape(x.shape)
    return codes.astype(np.int64), shared


def mxfp4_dequantize(codes, shared) -> np.ndarray:
    """Values of MXFP4 codes with their block exponents (inverse of the grid map)."""
    codes = np.asarray(codes, dtype=np.int64)
    shared = np.asarray(shared, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDES)[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    scale = np.repeat(np.ldexp(1.0, shared), MXFP4_BLOCK, axis=-1)
    return val * scale


def index_scores_fp4(qI, wI, KI, t: int, m: int) -> np.ndarray:
    """Indexer scores with q^I and K^I in MXFP4: the formula of index_scores
    evaluated exactly on the dequantized operands ([Scratch] §6.4)."""
    qd = mxfp4_dequantize(*mxfp4_quantize(qI))
    kd = mxfp4_dequantize(*mxfp4_quantize(KI))
    return index_scores(qd, wI, kd, t, m)


# --------------------------------------------------------------------------
# the [Evolution] derivation of the indexer's inputs (§6.2)
# --------------------------------------------------------------------------

def evolution_indexer_keys(Ccomp, W_kI) -> np.ndarray:
    """k^I_u = c^comp_u W^I_k: the indexer key of every compressed entry, a
    projection of the entry itself ([Evolution] §6.2)."""
    return project(Ccomp, W_kI)


def evolution_indexer_queries(h_t, W_qI, n_hI: int, cI: int) -> np.ndarray:
    """q^I_{t,j} = h_t W^I_{q,j} for the n_hI heads, side by side in W
    ([Evolution] §6.2): rows [n_hI][cI]."""
    return split_heads(project(h_t, W_qI), n_hI, cI)


# --------------------------------------------------------------------------
# shared-KV multi-query attention ([Scratch] §8, §10, §11)
# --------------------------------------------------------------------------

def mqa_attend(q, KV, scale=None):
    """Shared-KV MQA ([Scratch] §8): for every head h,

        o_h = sum_s softmax_s(q_h . KV_s * scale) KV_s,   lse_h = log sum_s exp(q_h . KV_s * scale)

    with key = value = KV_s and scale = 1/sqrt(c).  An empty KV set gives
    o = 0 and lse = -inf.
    """
    q, KV = f64(q), f64(KV)
    nh, c = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(c)
    if KV.shape[0] == 0:
        return np.zeros((nh, c)), np.full(nh, -np.inf)
    logits = (q @ KV.T) * scale                       # [nh][N]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    ssum = e.sum(axis=1)
    o = (e @ KV) / ssum[:, None]
    lse = mx[:, 0] + np.log(ssum)
    return o, lse


def csa_attend(q, Ccomp, idx, scale=None):
    """Core CSA attention over the selected entries C^SprsComp ([Scratch] §8)."""
    Ccomp = f64(Ccomp)
    idx = np.asarray(idx, dtype=np.int64)
    return mqa_attend(q, Ccomp[idx], scale)


def hca_attend(q, Chca, t: int, m_prime: int, scale=None):
    """Dense HCA attention over every visible HCA entry ([Scratch] §10)."""
    Chca = f64(Chca)
    return mqa_attend(q, Chca[:hca_visible(t, m_prime)], scale)


# --------------------------------------------------------------------------
# sliding-window branch ([Evolution] §6.1 and §6.2, "sliding window path";
# [Stack] §4 gives n_win = 128 for V4-Pro)
# --------------------------------------------------------------------------

def window_positions(t: int, n_win: int) -> np.ndarray:
    """Token positions of query t's sliding window: the n_win most recent
    tokens up to and including t, i.e. max(0, t - n_win + 1) ... t.
    ([Evolution] writes the same set 1-based as max(1, t-n_win+1) ... t.)"""
    return np.arange(max(0, t - n_win + 1), t + 1, dtype=np.int64)


def window_attend(q, Cwin, t: int, n_win: int, scale=None):
    """Shared-KV MQA over the raw window entries c^window_p = h_p W^{window,KV}
    for p in the window of t ([Evolution] §6.1).  Cwin is indexed by token
    position: row p holds c^window_p."""
    Cwin = f64(Cwin)
    return mqa_attend(q, Cwin[window_positions(t, n_win)], scale)


def mqa_attend_with_sink(q, KV, z, scale=None):
    """Shared-KV MQA with one sink logit per head: the softmax of head h runs
    over the logits of the keys and z_h, and the sink's value is zero, so
    o_h = sum_s p_s KV_s with p = softmax([q_h . KV_s * scale ..., z_h]) over
    the keys only, and lse_h = log(sum_s exp(q_h . KV_s * scale) + exp(z_h)).
    Written out directly from the definition (one extra logit, zero value)."""
    q, KV, z = f64(q), f64(KV), f64(z)
    nh, c = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(c)
    logits = np.concatenate([(q @ KV.T) * scale, z[:, None]], axis=1)   # [nh][N+1]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    tot = e.sum(axis=1, keepdims=True)
    p = e / tot
    values = np.concatenate([KV, np.zeros((1, c))], axis=0)             # the sink's value is 0
    return p @ values, (mx + np.log(tot))[:, 0]


def apply_sink(o, lse, z):
    """The sink applied to a finished attention (o, lse) of one head set:
    o' = o * e^lse / (e^lse + e^z), lse' = log(e^lse + e^z); an empty key set
    (lse = -inf) gives o' = 0 and lse' = z."""
    o, lse, z = f64(o), f64(lse), f64(z)
    m = np.maximum(lse, z)
    a = np.where(np.isfinite(lse), np.exp(lse - m), 0.0)
    bz = np.exp(z - m)
    return o * (a / (a + bz))[..., None], m + np.log(a + bz)


def merge_lse(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint key sets, from each part's
    normalised output and log-sum-exp: the pages join the window entries to the
    compressed ones by concatenation before one shared-KV MQA ([Evolution]
    §6.1, §6.2); since softmax sums over keys, that MQA equals
        lse = log(e^lse1 + e^lse2),  o = e^(lse1 - lse) o1 + e^(lse2 - lse) o2.
    An empty part has lse = -inf and contributes nothing."""
    o1, o2 = f64(o1), f64(o2)
    l1, l2 = f64(lse1), f64(lse2)
    m = np.maximum(l1, l2)
    both_empty = ~np.isfinite(m)
    ms = np.where(both_empty, 0.0, m)
    w1 = np.where(np.isfinite(l1), np.exp(l1 - ms), 0.0)
    w2 = np.where(np.isfinite(l2), np.exp(l2 - ms), 0.0)
    tot = w1 + w2
    safe = np.where(tot > 0, tot, 1.0)
    o = (w1[..., None] * o1 + w2[..., None] * o2) / safe[..., None]
    lse = np.where(both_empty, -np.inf, ms + np.log(safe))
    return np.where(both_empty[..., None], 0.0, o), lse


# --------------------------------------------------------------------------
# a whole decode query, from hidden states ([Scratch] §3-§10)
# --------------------------------------------------------------------------

def queries_from_hidden(h_t, W_DQ, W_IUQ, W_w, W_UQ, W_UQ_hca, n_h, c, n_hI, cI, dtype="f64"):
    """Query side of one token ([Scratch] §6.1-6.3 and §8).

    c^Q = h_t W^{DQ};  [q^I_1; ...] = c^Q W^{IUQ};  w^I = h_t W^w;
    [q_1; ...] = c^Q W^{UQ}.  HCA gets its own up-projection W^{UQ,HCA} of
    the same latent (the pages name no HCA query projection of their own).
    Stored intermediates are rounded as ``dtype`` storage would; w^I is kept
    in fp32.
    """
    cQ = store_as(project(h_t, W_DQ), dtype)
    qI = store_as(split_heads(project(cQ, W_IUQ), n_hI, cI), dtype)
    wI = store_as(project(h_t, W_w), "f32")
    q = store_as(split_heads(project(cQ, W_UQ), n_h, c), dtype)
    q_hca = store_as(split_heads(project(cQ, W_UQ_hca), n_h, c), dtype)
    return dict(cQ=cQ, qI=qI, wI=wI, q=q, q_hca=q_hca)


def decode_chain(H, W, t, m, m_prime, k, n_h, c, n_hI, cI, dtype="f64", KI_override=None,
                 Ba=None, Bb=None, BIa=None, BIb=None, Bh=None):
    """One CSA layer and one HCA layer for the query at position t, from H.

    ``W`` maps names to weight matrices: aKV bKV aZ bZ (CSA, [Scratch] §3),
    IaKV IbKV IaZ IbZ (the indexer's own compressor weights, [Scratch] §6.4),
    KV Z (HCA, [Scratch] §10), DQ IUQ w UQ UQ_hca (queries).  ``dtype`` is the
    storage format the chain mirrors.  ``KI_override`` injects indexer keys
    directly, as the worked example of [Scratch] §6.4 does.
    """
    H = f64(H)
    st = lambda x: store_as(x, dtype)  # noqa: E731
    Ca, Cb = st(project(H, W["aKV"])), st(project(H, W["bKV"]))
    Za, Zb = st(project(H, W["aZ"])), st(project(H, W["bZ"]))
    Ccomp = st(csa_compress(Za, Zb, Ca, Cb, m, Ba, Bb))
    if KI_override is not None:
        KI = f64(KI_override)
    else:
        ICa, ICb = st(project(H, W["IaKV"])), st(project(H, W["IbKV"]))
        IZa, IZb = st(project(H, W["IaZ"])), st(project(H, W["IbZ"]))
        KI = st(csa_compress(IZa, IZb, ICa, ICb, m, BIa, BIb))
    Ch, Zh = st(project(H, W["KV"])), st(project(H, W["Z"]))
    Chca = st(hca_compress(Zh, Ch, m_prime, Bh))
    Q = queries_from_hidden(H[t], W["DQ"], W["IUQ"], W["w"], W["UQ"], W["UQ_hca"],
                            n_h, c, n_hI, cI, dtype)
    scores = index_scores(Q["qI"], Q["wI"], KI, t, m)
    idx = topk_select(scores, k)
    o_csa, lse_csa = csa_attend(Q["q"], Ccomp, idx)
    o_hca, lse_hca = hca_attend(Q["q_hca"], Chca, t, m_prime)
    return dict(Ca=Ca, Cb=Cb, Za=Za, Zb=Zb, Ccomp=Ccomp, KI=KI, Chca=Chca, scores=scores,
                idx=idx, o_csa=o_csa, lse_csa=lse_csa, o_hca=o_hca, lse_hca=lse_hca, **Q)


# --------------------------------------------------------------------------
# the efficiency ledger ([Scratch] §1, §12)
# --------------------------------------------------------------------------

def gqa_kv_bytes_per_token_layer(n_kv_heads: int = 8, d_h: int = 128, b: int = 2) -> int:
    """Raw GQA KV cache: one key and one value per KV head ([Scratch] §1)."""
    return 2 * n_kv_heads * d_h * b


def compressed_bytes_per_token_layer(c: int, ratio: int, b: int = 2) -> float:
    """One c-wide entry per ``ratio`` tokens ([Scratch] §12.1): c*b/m or c*b/m'."""
    return c * b / ratio


def ledger(c=512, m=4, m_prime=128, b=2, baseline=2048, n_csa=30, n_hca=31):
    """KV-cache ledger of [Scratch] §12.1: per-layer bytes per token and the
    ratios against a raw baseline of ``baseline`` bytes per token per layer."""
    csa = compressed_bytes_per_token_layer(c, m, b)
    hca = compressed_bytes_per_token_layer(c, m_prime, b)
    mix = (n_csa * csa + n_hca * hca) / ((n_csa + n_hca) * baseline)
    return dict(csa=csa, hca=hca, csa_ratio=csa / baseline, hca_ratio=hca / baseline, mix=mix)


def indexer_flops_per_query(n: int, m: int, n_hI: int, cI: int) -> float:
    """Indexer cost per query, counted as in [Scratch] §12.2: (n/m) * n_h^I * c^I."""
    return n / m * n_hI * cI
