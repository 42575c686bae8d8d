"""MI355X (gfx950) hybrid linear temporal attention forward.

A thin Python binding over the C ABI of ``include/kairos.h`` (``libkairos.so``,
built in-tree by ``python -m video_world_model_chunkwise_amd.build``).  The
functions below carry the C entry points' names and only marshal arguments:
they check tensor dtypes, shapes and devices, allocate outputs and workspace
with torch (device memory plumbing), pass raw pointers and the current HIP
stream, and raise on a non-zero status.  Every step of the computation runs
in the library's kernels; there is no fallback.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    KairosError, Context, lib, lib_path, symbols, status_string, version,
    GdnDesc, HltaDesc, F32, BF16, FP8_E4M3, FP4_E2M1, PROLOGUE_NORMALIZE_Q, PROLOGUE_LITERAL_EQ6,
    QK_BLOCKS_TOKENS, QK_BLOCKS_FRAMES, kairos_hlta_ring_size, alloc_rings,
    WINDOW_CAUSAL, WINDOW_CENTERED,
    kairos_gdn_prologue, kairos_rope, kairos_gdn_fwd, kairos_gdn_fwd_noalloc, kairos_hlta_fwd, kairos_hlta_window_fwd, kairos_window_fwd, kairos_fp8_quantize, kairos_fp4_quantize,
    kairos_gdn_workspace_size, kairos_hlta_workspace_size, kairos_hlta_ring_frames_required,
    gdn_desc, hlta_desc, ring_key_shape, kairos_gdn_check_gates, KAIROS_ERR_RANGE,
)
