"""MI355X-native batched speculative-decoding verify step.

The work is done by hand-written HIP kernels for gfx950 behind the C ABI of
``include/spec_verify.h`` (``librsv_hip.so``, built in-tree by
``rejection_sampling_verify_amd.build``). This package is a thin ctypes
binding with the same entry-point names; PyTorch only supplies device memory
and the current stream. There is no fallback: if the library is missing the
calls raise.
"""
from .binding import (  # noqa: F401
    LIB_PATH,
    SV_DTYPE_BF16,
    SV_DTYPE_F32,
    SV_ERR_SCRATCH_LIMIT,
    SV_NOALLOC_SCRATCH_BYTES,
    SV_SEQ_BAD_LOGITS,
    SV_SEQ_BAD_TEMPERATURE,
    SV_SEQ_BAD_TOKEN,
    SV_SEQ_BAD_TREE,
    SV_SEQ_INTERNAL,
    SVError,
    Workspace,
    exported_symbols,
    lib,
    spec_verify_greedy,
    spec_verify_sample,
    spec_verify_sample_noalloc,
    spec_verify_tree,
    spec_verify_tree_sample,
    sv_kv_rollback,
    sv_kv_rollback_layers,
    sv_ngram_draft,
    sv_tree_mask,
    sv_debug_noise,
    sv_debug_read_stream,
    sv_debug_wave_max,
    sv_debug_philox,
    sv_status_string,
    sv_workspace_bytes,
    sv_workspace_init,
)
