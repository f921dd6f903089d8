"""Thin ctypes binding of libdlc.so (include/dlc.h).

Argument marshalling only: tensors become device pointers, sizes and
strides; every step of the computation runs in the HIP kernels behind the
C ABI.  The functions carry the C names.  Outputs and workspaces that the
caller does not pass are allocated here with torch on the tensors' device
(PyTorch serves as the device allocator and stream provider).  There is no
fallback: if the library is missing or a call fails, an exception says so.
"""

from __future__ import annotations

import ctypes as C
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdlc.so")

DLC_F32, DLC_BF16 = 0, 1
_DTYPES = {torch.float32: DLC_F32, torch.bfloat16: DLC_BF16}

_i64, _vp, _f32, _sz, _i32 = C.c_int64, C.c_void_p, C.c_float, C.c_size_t, C.c_int

# name -> (restype, argtypes), mirroring include/dlc.h
SIGNATURES = {
    "dlc_abi_version": (_i32, []),
    "dlc_status_str": (C.c_char_p, [_i32]),
    "dlc_last_error": (C.c_char_p, []),
    "csa_compress": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                            _i64, _i64, _vp, _i64, _vp]),
    "hca_compress": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _i64,
                            _vp, _i64, _vp]),
    "csa_project_compress": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                    _i64, _vp, _vp, _i64, _i64, _vp, _i64, _vp]),
    "hca_project_compress": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp,
                                    _i64, _i64, _vp, _i64, _vp]),
    "csa_index_topk_ws": (_sz, [_i64, _i64, _i64, _i64]),
    "csa_index_topk": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp,
                              _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mxfp4_quantize": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "csa_index_topk_fp4_ws": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "csa_index_topk_fp4": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp,
                                  _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "csa_attend_ws": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "csa_attend": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _f32, _vp,
                          _vp, _vp, _sz, _vp]),
    "csa_attend_noalloc": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _f32, _vp,
                                  _vp, _vp]),
    "hca_attend_ws": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "hca_attend": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _f32, _vp,
                          _vp, _vp, _sz, _vp]),
    "window_attend_ws": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "window_attend": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _f32, _vp, _vp,
                             _vp, _vp, _vp, _sz, _vp]),
    "csa_attend_window_ws": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "csa_attend_window": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64,
                                 _vp, _i64, _f32, _vp, _vp, _vp, _sz, _vp]),
    "hca_attend_window_ws": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "hca_attend_window": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _i64,
                                 _f32, _vp, _vp, _vp, _sz, _vp]),
    "attend_sink": (_i32, [_i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "dlc_project_ws": (_sz, [_i32, _i64, _i64, _i64]),
    "dlc_project": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _vp, _sz, _vp]),
    "dlc_timing_arm": (_i32, [_i32, _vp, _vp]),
    "dlc_copy": (_i32, [_vp, _vp, _sz, _vp]),
    "dlc_read": (_i32, [_vp, _sz, _i32, _vp]),
}

STAGE_INDEX_SCORES, STAGE_TOPK_SELECT, STAGE_CSA_ATTEND, STAGE_HCA_ATTEND, STAGE_COMPRESS = 1, 2, 3, 4, 5
STAGE_WINDOW_ATTEND = 6
STAGE_READ = 7


class DlcError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} ({status}): {detail}")


_lib = None


def lib():
    """The loaded library (loads it on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dense_long_context_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().dlc_status_str(status).decode()


def last_error() -> str:
    return lib().dlc_last_error().decode()


def _check(fn, status):
    if status != 0:
        raise DlcError(fn, status, last_error())


def _dt(x: torch.Tensor) -> int:
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    return _DTYPES[x.dtype]


def _p(x):
    return None if x is None else x.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _stride(x, dim, minimum):
    """x.stride(dim), or ``minimum`` when that dimension has one element (torch
    leaves the stride of a size-1 dimension arbitrary)."""
    return x.stride(dim) if x.shape[dim] > 1 else minimum


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_device(dev, **named):
    """Every named tensor (None is skipped) is a tensor on the CUDA device
    ``dev``: the kernels dereference these pointers, so a host tensor or one
    on another device must never reach them."""
    _need(isinstance(dev, torch.device) and dev.type == "cuda", f"inputs must be on a CUDA device, not {dev}")
    for nm, x in named.items():
        if x is None:
            continue
        _need(isinstance(x, torch.Tensor), f"{nm} must be a torch tensor")
        _need(x.device == dev, f"{nm} is on {x.device}; every tensor of the call must be on {dev}")


def _exact(x, nm, dtype, shape):
    """An output or side input the C ABI reads as a dense array of ``shape``."""
    if x is None:
        return
    _need(x.dtype == dtype, f"{nm} must be {dtype}, got {x.dtype}")
    _need(tuple(x.shape) == tuple(shape), f"{nm} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    _need(x.is_contiguous(), f"{nm} must be contiguous")


def _ws(nbytes, dev, ws):
    if ws is not None:
        _need(ws.is_contiguous(), "ws must be contiguous")
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


# ------------------------------------------------------------------ compress

def csa_compress(Za, Zb, Ca, Cb, m, out, i_begin=0, i_end=None, Ba=None, Bb=None, n=None):
    """Compress CSA entries [i_begin, i_end) of every sequence into ``out`` [B][cap][c].

    Streams are [B][rows][c] tensors (views with a row stride are fine) that
    share one stride pattern; ``n`` is the number of valid rows (default: all).
    """
    _on_device(Za.device, Za=Za, Zb=Zb, Ca=Ca, Cb=Cb, out=out, Ba=Ba, Bb=Bb)
    B, rows, c = Za.shape
    for x in (Zb, Ca, Cb):
        _need(x.shape == Za.shape and x.stride() == Za.stride() and x.dtype == Za.dtype,
              "the four streams must share shape, strides and dtype")
    _need(Za.stride(2) == 1, "stream rows must be contiguous")
    _need(out.dtype == Za.dtype and out.dim() == 3 and out.shape[0] == B and out.shape[2] == c and out.is_contiguous(),
          "out must be a contiguous [B][cap][c] tensor in the streams' dtype")
    _exact(Ba, "Ba", torch.float32, (m, c))
    _exact(Bb, "Bb", torch.float32, (m, c))
    n = rows if n is None else n
    i_end = n // m if i_end is None else i_end
    _check("csa_compress", lib().csa_compress(
        _dt(Za), B, n, c, m, _p(Za), _p(Zb), _p(Ca), _p(Cb), _stride(Za, 1, c), _stride(Za, 0, rows * c),
        _p(Ba), _p(Bb), i_begin, i_end, _p(out), out.shape[1], _stream(Za.device)))
    return out


def hca_compress(Z, Cs, m_prime, out, i_begin=0, i_end=None, bias=None, n=None):
    """Compress HCA entries [i_begin, i_end) into ``out`` [B][cap][c]."""
    _on_device(Z.device, Z=Z, C=Cs, out=out, bias=bias)
    B, rows, c = Z.shape
    _need(Cs.shape == Z.shape and Cs.stride() == Z.stride() and Cs.dtype == Z.dtype,
          "Z and C must share shape, strides and dtype")
    _need(Z.stride(2) == 1, "stream rows must be contiguous")
    _need(out.dtype == Z.dtype and out.dim() == 3 and out.shape[0] == B and out.shape[2] == c and out.is_contiguous(),
          "out must be a contiguous [B][cap][c] tensor in the streams' dtype")
    _exact(bias, "bias", torch.float32, (m_prime, c))
    n = rows if n is None else n
    i_end = n // m_prime if i_end is None else i_end
    _check("hca_compress", lib().hca_compress(
        _dt(Z), B, n, c, m_prime, _p(Z), _p(Cs), _stride(Z, 1, c), _stride(Z, 0, rows * c), _p(bias), i_begin, i_end,
        _p(out), out.shape[1], _stream(Z.device)))
    return out


def _fused_inputs(H, Wts, out, c):
    """Shape and layout checks shared by the fused projection + pooling calls:
    H [B][rows][d] bf16 with contiguous rows, each Wt [c][d] (rows contiguous,
    one leading dimension for all), out [B][cap][c] bf16 contiguous."""
    _need(H.dim() == 3 and H.dtype == torch.bfloat16 and H.stride(2) == 1,
          "H must be a bf16 [B][rows][d] tensor with contiguous rows")
    B, rows, d = H.shape
    for W in Wts:
        _need(W.dim() == 2 and tuple(W.shape) == (c, d) and W.dtype == torch.bfloat16 and W.stride(1) == 1
              and W.stride(0) == Wts[0].stride(0), "weights must be bf16 [c][d] with one row stride")
    _need(out.dtype == torch.bfloat16 and out.dim() == 3 and out.shape[0] == B and out.shape[2] == c
          and out.is_contiguous(), "out must be a contiguous bf16 [B][cap][c] tensor")
    return B, rows, d


def csa_project_compress(H, WtZa, WtZb, WtCa, WtCb, m, out, i_begin=0, i_end=None, Ba=None, Bb=None, n=None):
    """CSA entries [i_begin, i_end) straight from hidden rows H [B][rows][d]:
    the four stream projections (weights transposed, [c][d]) and the pooling in
    one pass, equal to dlc_project of each stream followed by csa_compress."""
    Wts = (WtZa, WtZb, WtCa, WtCb)
    _on_device(H.device, H=H, WtZa=WtZa, WtZb=WtZb, WtCa=WtCa, WtCb=WtCb, out=out, Ba=Ba, Bb=Bb)
    c = out.shape[-1]
    B, rows, d = _fused_inputs(H, Wts, out, c)
    _exact(Ba, "Ba", torch.float32, (m, c))
    _exact(Bb, "Bb", torch.float32, (m, c))
    n = rows if n is None else n
    i_end = n // m if i_end is None else i_end
    _check("csa_project_compress", lib().csa_project_compress(
        DLC_BF16, B, n, d, c, m, _p(H), _stride(H, 1, d), _stride(H, 0, rows * d), _p(WtZa), _p(WtZb), _p(WtCa),
        _p(WtCb), _stride(WtZa, 0, d), _p(Ba), _p(Bb), i_begin, i_end, _p(out), out.shape[1], _stream(H.device)))
    return out


def hca_project_compress(H, WtZ, WtC, m_prime, out, i_begin=0, i_end=None, bias=None, n=None):
    """HCA entries [i_begin, i_end) straight from hidden rows H [B][rows][d]
    (weights transposed, [c][d]), equal to dlc_project then hca_compress."""
    _on_device(H.device, H=H, WtZ=WtZ, WtC=WtC, out=out, bias=bias)
    c = out.shape[-1]
    B, rows, d = _fused_inputs(H, (WtZ, WtC), out, c)
    _exact(bias, "bias", torch.float32, (m_prime, c))
    n = rows if n is None else n
    i_end = n // m_prime if i_end is None else i_end
    _check("hca_project_compress", lib().hca_project_compress(
        DLC_BF16, B, n, d, c, m_prime, _p(H), _stride(H, 1, d), _stride(H, 0, rows * d), _p(WtZ), _p(WtC),
        _stride(WtZ, 0, d), _p(bias), i_begin, i_end, _p(out), out.shape[1], _stream(H.device)))
    return out


# ------------------------------------------------------------ indexer, top-k

def csa_index_topk_ws(B, n_q, cap, k):
    return lib().csa_index_topk_ws(B, n_q, cap, k)


def csa_index_topk(qI, wI, KI, t, t_max, m, k, idx=None, count=None, scores=None, ws=None):
    """Indexer scores and top-k.  qI [B][n_q][n_hI][cI], wI fp32 [B][n_q][n_hI],
    KI [B][cap][cI], t int64 [B][n_q] on the device.  Returns (idx, count)."""
    dev = qI.device
    _on_device(dev, qI=qI, wI=wI, KI=KI, t=t, idx=idx, count=count, scores=scores, ws=ws)
    B, n_q, n_hI, cI = qI.shape
    cap = KI.shape[1]
    for x, nm in ((qI, "qI"), (wI, "wI"), (KI, "KI"), (t, "t")):
        _need(x.is_contiguous(), f"{nm} must be contiguous")
    _need(wI.dtype == torch.float32 and t.dtype == torch.int64, "wI must be fp32 and t int64")
    _need(tuple(wI.shape) == (B, n_q, n_hI) and tuple(t.shape) == (B, n_q), "wI/t shape mismatch")
    _need(KI.dim() == 3 and KI.shape[0] == B and KI.shape[2] == cI and KI.dtype == qI.dtype,
          "KI shape/dtype mismatch")
    _exact(idx, "idx", torch.int32, (B, n_q, k))
    _exact(count, "count", torch.int32, (B, n_q))
    _exact(scores, "scores", torch.float32, (B, n_q, cap))
    if idx is None:
        idx = torch.empty((B, n_q, k), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    nb = csa_index_topk_ws(B, n_q, cap, k)
    ws = _ws(nb, dev, ws)
    _check("csa_index_topk", lib().csa_index_topk(
        _dt(qI), B, n_q, n_hI, cI, m, k, _p(qI), _p(wI), _p(KI), cap, _p(t), int(t_max), _p(idx),
        _p(count), _p(scores), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return idx, count


def mxfp4_quantize(x, codes=None, scales=None):
    """MXFP4 codes and E8M0 scales of the rows of x ([..., width], width % 32 == 0,
    fp32 or bf16, contiguous).  Returns (codes uint8 [..., width/2],
    scales uint8 [..., width/32]); see include/dlc.h for the format."""
    _on_device(x.device, x=x, codes=codes, scales=scales)
    _need(x.is_contiguous(), "x must be contiguous")
    width = x.shape[-1]
    rows = x.numel() // width if width else 0
    dev = x.device
    if codes is None:
        codes = torch.empty(tuple(x.shape[:-1]) + (width // 2,), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(tuple(x.shape[:-1]) + (width // 32,), dtype=torch.uint8, device=dev)
    _need(codes.is_contiguous() and scales.is_contiguous(), "codes/scales must be contiguous")
    _need(codes.dtype == torch.uint8 and scales.dtype == torch.uint8, "codes/scales must be uint8")
    _need(codes.numel() == rows * (width // 2) and scales.numel() == rows * (width // 32), "codes/scales size")
    _check("mxfp4_quantize", lib().mxfp4_quantize(
        _dt(x), 1, rows, width, _p(x), rows * width, _p(codes), rows * (width // 2), _p(scales),
        rows * (width // 32), _stream(dev)))
    return codes, scales


def csa_index_topk_fp4_ws(B, n_q, n_hI, cI, cap, k):
    return lib().csa_index_topk_fp4_ws(B, n_q, n_hI, cI, cap, k)


def csa_index_topk_fp4(qI, wI, KIc, KIs, t, t_max, m, k, idx=None, count=None, scores=None, ws=None):
    """FP4 (MXFP4) indexer scores and top-k.  qI [B][n_q][n_hI][cI] fp32/bf16 (quantized
    inside), wI fp32 [B][n_q][n_hI], KIc uint8 [B][cap][cI/2] and KIs uint8 [B][cap][cI/32]
    (mxfp4_quantize of the K^I cache), t int64 [B][n_q].  Returns (idx, count)."""
    dev = qI.device
    _on_device(dev, qI=qI, wI=wI, KIc=KIc, KIs=KIs, t=t, idx=idx, count=count, scores=scores, ws=ws)
    B, n_q, n_hI, cI = qI.shape
    cap = KIc.shape[1]
    _exact(idx, "idx", torch.int32, (B, n_q, k))
    _exact(count, "count", torch.int32, (B, n_q))
    _exact(scores, "scores", torch.float32, (B, n_q, cap))
    for x, nm in ((qI, "qI"), (wI, "wI"), (KIc, "KIc"), (KIs, "KIs"), (t, "t")):
        _need(x.is_contiguous(), f"{nm} must be contiguous")
    _need(wI.dtype == torch.float32 and t.dtype == torch.int64, "wI must be fp32 and t int64")
    _need(tuple(wI.shape) == (B, n_q, n_hI) and tuple(t.shape) == (B, n_q), "wI/t shape mismatch")
    _need(KIc.dtype == torch.uint8 and KIs.dtype == torch.uint8, "KIc/KIs must be uint8")
    _need(tuple(KIc.shape) == (B, cap, cI // 2) and tuple(KIs.shape) == (B, cap, cI // 32), "KIc/KIs shape")
    if idx is None:
        idx = torch.empty((B, n_q, k), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    nb = csa_index_topk_fp4_ws(B, n_q, n_hI, cI, cap, k)
    ws = _ws(nb, dev, ws)
    _check("csa_index_topk_fp4", lib().csa_index_topk_fp4(
        _dt(qI), B, n_q, n_hI, cI, m, k, _p(qI), _p(wI), _p(KIc), _p(KIs), cap, _p(t), int(t_max), _p(idx),
        _p(count), _p(scores), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return idx, count


# ---------------------------------------------------------------- attention

def csa_attend_ws(B, n_q, n_h, c, k):
    return lib().csa_attend_ws(B, n_q, n_h, c, k)


def hca_attend_ws(B, n_q, n_h, c, cap):
    return lib().hca_attend_ws(B, n_q, n_h, c, cap)


def csa_attend(q, Ccomp, idx, count, scale=0.0, out=None, lse=None, ws=None):
    """Shared-KV MQA over the selected CSA entries.  q [B][n_q][n_h][c];
    Ccomp [B][cap][c]; idx int32 [B][n_q][k]; count int32 [B][n_q].
    Returns (out fp32 [B][n_q][n_h][c], lse fp32 [B][n_q][n_h])."""
    dev = q.device
    _on_device(dev, q=q, Ccomp=Ccomp, idx=idx, count=count, out=out, lse=lse, ws=ws)
    B, n_q, n_h, c = q.shape
    k = idx.shape[2]
    _need(q.is_contiguous() and Ccomp.is_contiguous() and idx.is_contiguous() and count.is_contiguous(),
          "inputs must be contiguous")
    _need(Ccomp.dim() == 3 and Ccomp.shape[0] == B and Ccomp.shape[2] == c and Ccomp.dtype == q.dtype,
          "Ccomp shape/dtype mismatch")
    _exact(idx, "idx", torch.int32, (B, n_q, k))
    _exact(count, "count", torch.int32, (B, n_q))
    _exact(out, "out", torch.float32, (B, n_q, n_h, c))
    _exact(lse, "lse", torch.float32, (B, n_q, n_h))
    if out is None:
        out = torch.empty((B, n_q, n_h, c), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, n_h), dtype=torch.float32, device=dev)
    ws = _ws(csa_attend_ws(B, n_q, n_h, c, k), dev, ws)
    _check("csa_attend", lib().csa_attend(
        _dt(q), B, n_q, n_h, c, k, _p(q), _p(Ccomp), Ccomp.shape[1], _p(idx), _p(count), float(scale),
        _p(out), _p(lse), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out, lse


def csa_attend_noalloc(q, Ccomp, idx, count, out, lse, scale=0.0):
    """csa_attend without a workspace: the library's static scratch array holds
    the split partials (see include/dlc.h for its size limit).  ``out`` fp32
    [B][n_q][n_h][c] and ``lse`` fp32 [B][n_q][n_h] are the caller's; nothing
    is allocated on this path."""
    dev = q.device
    _on_device(dev, q=q, Ccomp=Ccomp, idx=idx, count=count, out=out, lse=lse)
    B, n_q, n_h, c = q.shape
    k = idx.shape[2]
    _need(q.is_contiguous() and Ccomp.is_contiguous(), "inputs must be contiguous")
    _need(Ccomp.dim() == 3 and Ccomp.shape[0] == B and Ccomp.shape[2] == c and Ccomp.dtype == q.dtype,
          "Ccomp shape/dtype mismatch")
    _exact(idx, "idx", torch.int32, (B, n_q, k))
    _exact(count, "count", torch.int32, (B, n_q))
    _need(out is not None and lse is not None, "out and lse are required")
    _exact(out, "out", torch.float32, (B, n_q, n_h, c))
    _exact(lse, "lse", torch.float32, (B, n_q, n_h))
    _check("csa_attend_noalloc", lib().csa_attend_noalloc(
        _dt(q), B, n_q, n_h, c, k, _p(q), _p(Ccomp), Ccomp.shape[1], _p(idx), _p(count), float(scale),
        _p(out), _p(lse), _stream(dev)))
    return out, lse


def hca_attend(q, Chca, t, t_max, m_prime, scale=0.0, out=None, lse=None, ws=None):
    """Dense shared-KV MQA over the visible HCA entries.  Returns (out, lse)."""
    dev = q.device
    _on_device(dev, q=q, Chca=Chca, t=t, out=out, lse=lse, ws=ws)
    B, n_q, n_h, c = q.shape
    cap = Chca.shape[1]
    _need(q.is_contiguous() and Chca.is_contiguous() and t.is_contiguous(), "inputs must be contiguous")
    _need(Chca.dim() == 3 and Chca.shape[0] == B and Chca.shape[2] == c and Chca.dtype == q.dtype,
          "Chca shape/dtype mismatch")
    _need(t.dtype == torch.int64 and tuple(t.shape) == (B, n_q), "t must be int64 [B][n_q]")
    _exact(out, "out", torch.float32, (B, n_q, n_h, c))
    _exact(lse, "lse", torch.float32, (B, n_q, n_h))
    if out is None:
        out = torch.empty((B, n_q, n_h, c), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, n_h), dtype=torch.float32, device=dev)
    ws = _ws(hca_attend_ws(B, n_q, n_h, c, cap), dev, ws)
    _check("hca_attend", lib().hca_attend(
        _dt(q), B, n_q, n_h, c, m_prime, _p(q), _p(Chca), cap, _p(t), int(t_max), float(scale),
        _p(out), _p(lse), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out, lse


def window_attend_ws(B, n_q, n_h, c, n_win):
    return lib().window_attend_ws(B, n_q, n_h, c, n_win)


def window_attend(q, Cwin, t, t_max, n_win, o_in=None, lse_in=None, scale=0.0, out=None, lse=None, ws=None):
    """Sliding-window branch over the ring Cwin [B][ring][c] (token p at row
    p % ring, ring >= n_win), optionally joined to a compressed branch's
    (o_in, lse_in) by their log-sum-exp.  Returns (out, lse); out may be o_in."""
    dev = q.device
    _on_device(dev, q=q, Cwin=Cwin, t=t, o_in=o_in, lse_in=lse_in, out=out, lse=lse, ws=ws)
    B, n_q, n_h, c = q.shape
    ring = Cwin.shape[1]
    _exact(out, "out", torch.float32, (B, n_q, n_h, c))
    _exact(lse, "lse", torch.float32, (B, n_q, n_h))
    _need(q.is_contiguous() and Cwin.is_contiguous() and t.is_contiguous(), "inputs must be contiguous")
    _need(Cwin.shape[0] == B and Cwin.shape[2] == c and Cwin.dtype == q.dtype, "Cwin shape/dtype mismatch")
    _need(t.dtype == torch.int64 and tuple(t.shape) == (B, n_q), "t must be int64 [B][n_q]")
    _need((o_in is None) == (lse_in is None), "o_in and lse_in come together")
    if o_in is not None:
        _need(o_in.dtype == torch.float32 and tuple(o_in.shape) == (B, n_q, n_h, c) and o_in.is_contiguous(),
              "o_in must be fp32 [B][n_q][n_h][c]")
        _need(lse_in.dtype == torch.float32 and tuple(lse_in.shape) == (B, n_q, n_h) and lse_in.is_contiguous(),
              "lse_in must be fp32 [B][n_q][n_h]")
    if out is None:
        out = torch.empty((B, n_q, n_h, c), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, n_h), dtype=torch.float32, device=dev)
    ws = _ws(window_attend_ws(B, n_q, n_h, c, n_win), dev, ws)
    _check("window_attend", lib().window_attend(
        _dt(q), B, n_q, n_h, c, n_win, _p(q), _p(Cwin), ring, _p(t), int(t_max), float(scale), _p(o_in), _p(lse_in),
        _p(out), _p(lse), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out, lse


def csa_attend_window(q, Ccomp, idx, count, Cwin, t, t_max, n_win, scale=0.0, out=None, lse=None, ws=None):
    """csa_attend joined with the sliding window of the ring Cwin [B][ring][c]."""
    dev = q.device
    _on_device(dev, q=q, Ccomp=Ccomp, idx=idx, count=count, Cwin=Cwin, t=t, out=out, lse=lse, ws=ws)
    B, n_q, n_h, c = q.shape
    k, ring = idx.shape[2], Cwin.shape[1]
    _exact(idx, "idx", torch.int32, (B, n_q, k))
    _exact(count, "count", torch.int32, (B, n_q))
    _exact(out, "out", torch.float32, (B, n_q, n_h, c))
    _exact(lse, "lse", torch.float32, (B, n_q, n_h))
    _need(all(x.is_contiguous() for x in (q, Ccomp, idx, count, Cwin, t)), "inputs must be contiguous")
    _need(Ccomp.shape[0] == B and Ccomp.shape[2] == c and Ccomp.dtype == q.dtype, "Ccomp shape/dtype mismatch")
    _need(Cwin.shape[0] == B and Cwin.shape[2] == c and Cwin.dtype == q.dtype, "Cwin shape/dtype mismatch")
    _need(idx.dtype == torch.int32 and count.dtype == torch.int32, "idx/count must be int32")
    _need(t.dtype == torch.int64 and tuple(t.shape) == (B, n_q), "t must be int64 [B][n_q]")
    if out is None:
        out = torch.empty((B, n_q, n_h, c), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, n_h), dtype=torch.float32, device=dev)
    ws = _ws(lib().csa_attend_window_ws(B, n_q, n_h, c, k, n_win), dev, ws)
    _check("csa_attend_window", lib().csa_attend_window(
        _dt(q), B, n_q, n_h, c, k, _p(q), _p(Ccomp), Ccomp.shape[1], _p(idx), _p(count), _p(Cwin), ring, n_win,
        _p(t), int(t_max), float(scale), _p(out), _p(lse), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out, lse


def hca_attend_window(q, Chca, t, t_max, m_prime, Cwin, n_win, scale=0.0, out=None, lse=None, ws=None):
    """hca_attend joined with the sliding window of the ring Cwin [B][ring][c]."""
    dev = q.device
    _on_device(dev, q=q, Chca=Chca, t=t, Cwin=Cwin, out=out, lse=lse, ws=ws)
    B, n_q, n_h, c = q.shape
    cap, ring = Chca.shape[1], Cwin.shape[1]
    _exact(out, "out", torch.float32, (B, n_q, n_h, c))
    _exact(lse, "lse", torch.float32, (B, n_q, n_h))
    _need(all(x.is_contiguous() for x in (q, Chca, Cwin, t)), "inputs must be contiguous")
    _need(Chca.shape[0] == B and Chca.shape[2] == c and Chca.dtype == q.dtype, "Chca shape/dtype mismatch")
    _need(Cwin.shape[0] == B and Cwin.shape[2] == c and Cwin.dtype == q.dtype, "Cwin shape/dtype mismatch")
    _need(t.dtype == torch.int64 and tuple(t.shape) == (B, n_q), "t must be int64 [B][n_q]")
    if out is None:
        out = torch.empty((B, n_q, n_h, c), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, n_h), dtype=torch.float32, device=dev)
    ws = _ws(lib().hca_attend_window_ws(B, n_q, n_h, c, cap, n_win), dev, ws)
    _check("hca_attend_window", lib().hca_attend_window(
        _dt(q), B, n_q, n_h, c, m_prime, _p(q), _p(Chca), cap, _p(t), int(t_max), _p(Cwin), ring, n_win,
        float(scale), _p(out), _p(lse), _p(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out, lse


# --------------------------------------------------------------- projection

def dlc_project_ws(M, N, K, dtype=torch.bfloat16):
    """Bytes of the optional dlc_project workspace for an [M][K] x [K][N] call (0: none used)."""
    return lib().dlc_project_ws(DLC_BF16 if dtype == torch.bfloat16 else DLC_F32, M, N, K)


def project_workspace(M, N, K, device, dtype=torch.bfloat16):
    """A zeroed workspace for dlc_project calls of this shape (None if the call uses none); every
    call leaves it zeroed, so calls of any shape it is large enough for can reuse it."""
    n = dlc_project_ws(M, N, K, dtype)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def dlc_project(A, Wt, out=None, out_dtype=None, ws=None):
    """out[M][N] = A[M][K] . W with W given transposed as Wt [N][K]; fp32 accumulation.
    ws: optional zeroed workspace (project_workspace) that lets a call with few rows spread
    its k-range over more workgroups."""
    _on_device(A.device, A=A, Wt=Wt, out=out, ws=ws)
    M, K = A.shape
    N = Wt.shape[0]
    _need(Wt.dim() == 2 and Wt.shape[1] == K and Wt.dtype == A.dtype, "Wt must be [N][K] in A's dtype")
    _need(A.stride(1) == 1 and Wt.stride(1) == 1, "rows must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or A.dtype, device=A.device)
    _need(out.stride(1) == 1 and tuple(out.shape) == (M, N), "out must be [M][N] with contiguous rows")
    _need(out.dtype in (torch.float32, A.dtype), "out must be fp32 or A's dtype")
    _need(ws is None or ws.is_contiguous(), "ws must be contiguous")
    _check("dlc_project", lib().dlc_project(
        _dt(A), M, N, K, _p(A), _stride(A, 0, K), _p(Wt), _stride(Wt, 0, K), _p(out), _stride(out, 0, N), _dt(out),
        None if ws is None else _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(A.device)))
    return out


def attend_sink(out, lse, z):
    """Per-head sink logits z (fp32 [n_h]) applied in place to an attention's
    fp32 output [..., n_h, c] and log-sum-exp [..., n_h]; returns (out, lse)."""
    _on_device(out.device, out=out, lse=lse, z=z)
    n_h, c = out.shape[-2], out.shape[-1]
    rows = out.numel() // (n_h * c) if n_h * c else 0
    _need(out.dtype == torch.float32 and lse.dtype == torch.float32 and z.dtype == torch.float32, "fp32 only")
    _need(out.is_contiguous() and lse.is_contiguous() and z.is_contiguous(), "contiguous tensors only")
    _need(lse.numel() == rows * n_h and z.numel() == n_h, "lse / z shape")
    _check("attend_sink", lib().attend_sink(rows, n_h, c, _p(out), _p(lse), _p(z), _stream(out.device)))
    return out, lse


def dlc_timing_arm(stage, ev_begin, ev_end):
    """Arm raw hipEvent_t handles (ints) around the next launch of ``stage``."""
    _check("dlc_timing_arm", lib().dlc_timing_arm(stage, ev_begin, ev_end))


def dlc_copy(dst, src):
    """Copy kernel (bandwidth reference): dst[:] = src[:] for equal-size device tensors."""
    _on_device(src.device, dst=dst, src=src)
    _need(dst.is_contiguous() and src.is_contiguous(), "dst and src must be contiguous")
    nb = src.numel() * src.element_size()
    _need(dst.numel() * dst.element_size() == nb, "size mismatch")
    _check("dlc_copy", lib().dlc_copy(_p(dst), _p(src), nb, _stream(src.device)))
    return dst


READ_LDS, READ_TILES = 0, 1  # load forms of dlc_read


def dlc_read(src, form=READ_TILES):
    """Read-only kernel over a contiguous device tensor in one load form (the
    calibration reference for read counters): READ_TILES (size a multiple of
    4 KB, the bf16 indexer's form) or READ_LDS (a multiple of 1 KB, the FP4
    indexer's form); returns nothing."""
    _on_device(src.device, src=src)
    _need(src.is_contiguous(), "src must be contiguous")
    _check("dlc_read", lib().dlc_read(_p(src), src.numel() * src.element_size(), int(form), _stream(src.device)))


def default_scale(c: int) -> float:
    return 1.0 / math.sqrt(c)
