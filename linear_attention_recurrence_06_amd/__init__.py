"""MI355X (gfx950) Kimi Delta Attention: chunked prefill and decode step.

The computation lives in libkda.so (hand-written HIP, C ABI in include/kda.h);
this package holds its sources (csrc/), the in-tree build script and a thin
ctypes binding whose functions carry the C ABI's names.
"""

from .kda import (KDA_NOALLOC_SCRATCH_BYTES, KDAError, kda_checkpoint_count, kda_chunk_prefill,
                  kda_chunk_prefill_checkpoints, kda_chunk_prefill_ex,
                  kda_chunk_prefill_noalloc, kda_decode_step,
                  kda_decode_step_ex, kda_dims, kda_prefill_path, kda_prefill_path_workspace_bytes,
                  kda_prefill_pipeline_segments, kda_prefill_workspace_bytes, load_library,
                  make_dims, status_string)

__all__ = ["KDA_NOALLOC_SCRATCH_BYTES", "KDAError", "kda_checkpoint_count", "kda_chunk_prefill",
           "kda_chunk_prefill_checkpoints", "kda_chunk_prefill_ex", "kda_chunk_prefill_noalloc",
           "kda_decode_step",
           "kda_decode_step_ex", "kda_dims", "kda_prefill_path", "kda_prefill_path_workspace_bytes",
           "kda_prefill_pipeline_segments",
           "kda_prefill_workspace_bytes", "load_library", "make_dims", "status_string"]
