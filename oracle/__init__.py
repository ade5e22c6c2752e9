"""CPU oracle for paged KV-cache attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product path (the HIP
library and its Python binding) never imports, calls or falls back to it.

What it computes, in float64 on the CPU, with plain loops and library
primitives (matmul, exp, searchsorted) and no blocking or fusion:

* ``formats``   — storage codecs: bf16 and OCP fp8 e4m3fn decode, and the
                  round-to-nearest-even, saturating fp8 encode used when new
                  keys/values enter an fp8 cache.
* ``attention`` — the page gather through the block table, scaled
                  dot-product softmax attention per query head (textbook form,
                  max-shifted), the causal chunked-prefill variant, the cache
                  append (scatter) and the split/log-sum-exp merge identity.

Sources (pages of the reference material, by title and section):
  "TensorRT-LLM框架解析与高性能推理优化实践" §4.2 (paged KV cache, block table),
  §6.1 (flash attention: running max / running sum), §6.2 (paged attention
  walks the block table), §7.2 (KV-cache quantization with one scale per
  head, dequantised inside the kernel); "TensorRT-LLM性能调优：提升LLM推理效率",
  layer-fusion discussion (fused MHA: scaled dot-product attention with a
  causal mask); §5.3 of the first page (chunked context).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
independent facts: a library SDPA on logical (unpaged) K/V, pure-Python brute
force, closed forms, page-permutation invariance, torch's own fp8 cast, and
the OCP fp8 table values under ``tests/golden``.  One reading is not pinned
against the pages because they do not state it: the grouped-query head map
(query head h reads KV head h // G) — "parity unpinned" for G > 1 with respect
to the pages; the G = 1 reduction to multi-head attention is pinned.
"""
from . import formats, attention  # noqa: F401

__all__ = ["formats", "attention"]
