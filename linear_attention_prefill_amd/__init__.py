"""MI355X-native KDA (Kimi Delta Attention): chunked prefill and decode.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
of ``libkda.so`` (``include/kda.h``); ``kda`` is its thin binding.
"""
from .kda import (KdaError, check_prefill_inputs, chunk_prefill,  # noqa: F401
                  chunk_prefill_no_alloc, conv_extent, decode_step, decode_tokens, line_extent,
                  load_library, prefill_fuse_chunks, prefill_windows,
                  prefill_workspace_size)
