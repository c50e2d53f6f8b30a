"""TTQ (activation-aware test-time quantization) linear projection on MI355X.

The projection runs in hand-written gfx950 kernels behind the C ABI of
``include/ttq.h`` (``libttq.so``, built in-tree by
``python -m online_activation_aware_ttq_amd.build``); this package is the
thin Python binding over it.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    QFORMATS,
    LIB_PATH,
    TTQ_EALIGN,
    TTQ_EHIP,
    TTQ_EINVAL,
    TTQ_ENULL,
    TTQ_EUNSUPPORTED,
    TTQ_EWORKSPACE,
    TTQ_FLAG_FORCE_FUSED,
    TTQ_FLAG_FORCE_TWO_PHASE,
    TTQ_OK,
    TTQError,
    container_bits,
    load_library,
    make_params,
    qformat_code,
    stream_read,
    timing_enable,
    timing_query,
    timing_reset,
    ttq_linear,
    ttq_linear_batched,
    ttq_linear_noalloc,
    TTQ_NOALLOC_SCRATCH_BYTES,
    ttq_linear_segmented,
    ttq_lowrank_pca,
    ttq_lowrank_pca_workspace_bytes,
    ttq_segmented_workspace_bytes,
    ttq_params,
    ttq_packed_row_bytes,
    ttq_path,
    ttq_qmatmul,
    ttq_qmatmul_workspace_bytes,
    ttq_quantize,
    ttq_quantize_workspace_bytes,
    ttq_status_string,
    ttq_version,
    ttq_workspace_bytes,
)
