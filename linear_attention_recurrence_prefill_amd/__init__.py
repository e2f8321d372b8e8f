"""MI355X (gfx950) Gated DeltaNet chunked prefill.

``gdn`` holds the Python binding of the HIP library (``libgdn_mi355x.so``, built by
``python -m linear_attention_recurrence_prefill_amd.build``); the C ABI is ``include/gdn.h`` (and
``include/gdn_calib.h`` for the measurement kernels).
"""
from .gdn import (GdnError, calib_copy, calib_mfma_bf16, chunk_bwd, chunk_fwd, chunk_fwd_noalloc,
                  gdn_chunk_fwd_noalloc,
                  chunk_fwd_intermediates, chunk_fwd_plan, decode_step, device_faults,
                  gdn_calib_copy, gdn_calib_mfma_bf16, gdn_chunk_bwd, gdn_chunk_fwd,
                  gdn_chunk_fwd_intermediates, gdn_chunk_fwd_plan, gdn_decode_step,
                  gdn_device_faults, gdn_get_debug, gdn_set_debug, gdn_validate_cu_seqlens,
                  get_debug, load_library, set_debug, validate_cu_seqlens)

__all__ = ["GdnError", "chunk_fwd", "chunk_fwd_noalloc", "gdn_chunk_fwd_noalloc", "chunk_bwd", "chunk_fwd_plan", "chunk_fwd_intermediates",
           "decode_step", "validate_cu_seqlens", "set_debug", "get_debug", "device_faults",
           "calib_copy", "calib_mfma_bf16", "load_library", "gdn_chunk_fwd",
           "gdn_chunk_fwd_plan", "gdn_chunk_fwd_intermediates", "gdn_chunk_bwd", "gdn_decode_step",
           "gdn_validate_cu_seqlens", "gdn_set_debug", "gdn_get_debug", "gdn_device_faults",
           "gdn_calib_copy", "gdn_calib_mfma_bf16"]
