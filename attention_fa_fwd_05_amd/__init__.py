"""Exact attention for MI355X (gfx950): tiled online-softmax forward that keeps
O and the natural-log row logsumexp L, and a backward that rebuilds the score
and probability tiles from Q, K, V, O and L.  The computation lives in
libfa05.so (C ABI in include/fa.h); this package only marshals arguments.
"""

from ._binding import (EXPORTS, FA_DTYPE_BF16, FA_DTYPE_F32, LIB_PATH, STAGE_ALL,  # noqa: F401
                       STAGE_DKDV, STAGE_DQ, STAGE_PRE, STATUS, FaError, attention, backward, forward,
                       backward_masked, backward_noalloc, backward_paged, backward_varlen, forward_masked,
                       forward_paged, pack_mask, forward_splitk, forward_varlen, forward_varlen_masked,
                       forward_varlen_splitk, backward_varlen_masked, load_library,
                       splitk_workspace_bytes, status_string, workspace_bytes)
