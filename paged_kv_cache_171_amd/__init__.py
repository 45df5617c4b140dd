"""Paged KV-cache decode attention for MI355X (gfx950).

The compute lives in ``libpkv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pkv.h``); this package is its ctypes binding.  Build the
library with ``python -m paged_kv_cache_171_amd.build``.
"""
from .binding import (  # noqa: F401
    BlockAllocator, Scheduler, Batch, PkvError, LIB_PATH, EXPORTED,
    pkv_version, pkv_append, pkv_copy_blocks, pkv_swap_blocks, pkv_attention_workspace_bytes,
    pkv_attention_decode_shared, pkv_attention_decode_shared_workspace_bytes, pkv_attention_decode_append,
    pkv_attention_decode, pkv_attention_prefill_chunk, pkv_decode_plan_bytes, pkv_decode_plan, plan_for,
    workspace_for, pkv_attention_decode_noalloc, PKV_NOALLOC_SCRATCH_BYTES,
    pkv_decode_shared_plan_bytes, pkv_decode_shared_plan, shared_plan_for, pkv_attention_decode_shared_planned,
    PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP,
    PKV_ERR_UNKNOWN_SEQ, PKV_F32, PKV_BF16, PKV_SCHED_CONTINUOUS, PKV_SCHED_STATIC,
    PKV_REQ_WAITING, PKV_REQ_RUNNING, PKV_REQ_SWAPPED, PKV_REQ_FINISHED,
)
