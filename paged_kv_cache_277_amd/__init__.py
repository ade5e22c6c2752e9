"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (hand-written HIP kernels behind the C
ABI of ``include/pagedkv.h``); ``binding`` is its ctypes binding, with the
same function names as the C entry points.  ``workloads`` draws seeded
synthetic inputs and ``device`` uploads them and runs one step of the hot path.
"""
from .binding import (PagedCache, PageAllocator, PkvError, Scheduler, decode_workspace, lib, version,  # noqa: F401
                      pkv_decode_split_tokens, pkv_decode_workspace_bytes, pkv_fp8_e4m3fn_to_f32,
                      pkv_kv_cache_append, pkv_lse_merge, pkv_paged_attn_chunked_prefill,
                      pkv_paged_attn_decode, pkv_paged_attn_decode_partial, pkv_decode_work_list,
                      pkv_decode_step, DecodeStepCall,
                      pkv_prefill_split_tokens, pkv_prefill_workspace_bytes, prefill_workspace,
                      pkv_validate_block_tables, pkv_mixed_step, append_batch,
                      decode_batch, prefill_batch, pkv_context_fmha, context_workspace)
