"""Paged KV cache + PagedAttention decode for AMD MI355X (gfx950).

The compute path is libpa.so (hand-written HIP kernels behind a C ABI,
``include/pa.h``); this package only loads it and marshals torch tensors to
it (``binding``). ``inputs`` holds the seeded synthetic workloads.
"""

from .binding import (BlockAllocator, PAError, decode_scratch, pa_copy_blocks,  # noqa: F401
                      pa_decode, pa_decode_balanced, pa_decode_fp8,
                      pa_decode_balanced_static, pa_decode_partitioned_balanced,
                      pa_decode_scratch_bytes, pa_decode_partitioned, pa_decode_partitioned_fp8,
                      pa_decode_step, pa_decode_plan_bytes,
                      pa_decode_partitioned_planned, decode_plan_buffer,
                      pa_partition_workspace_bytes, pa_prefill_chunk, pa_reduce,
                      pa_read_probe, pa_reshape_and_cache, pa_reshape_and_cache_fp8,
                      pa_swap_blocks)

__version__ = "0.1.0"
