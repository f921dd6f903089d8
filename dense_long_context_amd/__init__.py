"""CSA/HCA compressed-attention hot path for AMD MI355X (gfx950).

The computation lives in libdlc.so (HIP kernels behind the C ABI declared in
include/dlc.h); this package is its Python binding plus the in-tree build.
"""

from .binding import (  # noqa: F401
    DlcError,
    attend_sink,
    csa_attend,
    csa_attend_noalloc,
    csa_attend_window,
    csa_attend_ws,
    csa_compress,
    csa_project_compress,
    csa_index_topk,
    csa_index_topk_fp4,
    csa_index_topk_fp4_ws,
    csa_index_topk_ws,
    default_scale,
    dlc_project,
    dlc_project_ws,
    hca_attend,
    hca_attend_window,
    hca_attend_ws,
    hca_compress,
    hca_project_compress,
    last_error,
    lib,
    mxfp4_quantize,
    project_workspace,
    status_str,
    window_attend,
    window_attend_ws,
)
