"""VAR-Q packed KV cache for MI355X (gfx950).

The hot path -- (block, channel) min/max quantization of each decoded block,
2-, 3-, 4- or 8-bit packing (dense rows, or block-aligned 3-bit words), and
block-causal attention over the packed cache -- runs
in the HIP kernels of libkvq.so behind the C ABI of include/kvq.h.  The
functions below are its thin Python binding (torch supplies device memory and
streams only).
"""
from .kvq import (  # noqa: F401
    BF16, F32, KvqError, Layout, S_NONFINITE, S_RANGE, STATIC_SCRATCH_BYTES, alloc_cache, cache_shapes,
    header_symbols, kvq_attend_packed, kvq_attend_packed_split, kvq_attend_packed_split_noalloc,
    kvq_attend_split_workspace,
    kvq_bytes, kvq_dequantize, kvq_pack, kvq_quantize_attend, kvq_quantize_block,
    kvq_stream_copy, kvq_stream_read, kvq_unpack, kvq_version, lib, make_layout,
)
