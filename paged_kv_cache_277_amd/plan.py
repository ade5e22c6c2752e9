"""A scheduler step plan -> the kernels' batch arguments (host int32 arrays).

The step scheduler (``binding.Scheduler``) plans, per running request, a
prefill chunk or one decode token starting at its cached length; the kernels
take packed rows.  ``step_arrays`` lays one plan out: every item appends its
tokens (``pkv_kv_cache_append`` rows), decode items are the rows of
``pkv_paged_attn_decode`` (context = start + 1: the token itself), prefill
items the requests of ``pkv_paged_attn_chunked_prefill`` (ctx_before =
start).  Block tables are the scheduler's, padded with -1 to ``bt_stride``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .binding import PKV_WORK_DECODE


@dataclass
class StepArrays:
    items: list                 # (req_id, slot, kind, start_pos, num_tokens)
    block_tables: np.ndarray    # [items][bt_stride] int32
    app_cu: np.ndarray          # [items+1]: packed new-token offsets
    app_start: np.ndarray       # [items]
    dec_idx: np.ndarray         # item indices of decode rows
    dec_lens: np.ndarray        # [decode rows]: start + 1
    pf_idx: np.ndarray          # item indices of prefill requests
    pf_cu: np.ndarray           # [prefill + 1]
    pf_ctx: np.ndarray          # [prefill]: start
    max_chunk: int
    max_total: int


def step_arrays(sched, items, bt_stride: int) -> StepArrays:
    n = len(items)
    bt = np.full((n, bt_stride), -1, dtype=np.int32)
    for i, (rid, *_rest) in enumerate(items):
        t = sched.block_table(rid)
        if len(t) > bt_stride:
            raise ValueError(f"request {rid} holds {len(t)} pages > bt_stride {bt_stride}")
        bt[i, : len(t)] = t
    tokens = np.array([it[4] for it in items], dtype=np.int32)
    start = np.array([it[3] for it in items], dtype=np.int32)
    kind = np.array([it[2] for it in items], dtype=np.int32)
    dec = np.nonzero(kind == PKV_WORK_DECODE)[0]
    pf = np.nonzero(kind != PKV_WORK_DECODE)[0]
    return StepArrays(
        items=list(items), block_tables=bt,
        app_cu=np.concatenate([[0], np.cumsum(tokens)]).astype(np.int32),
        app_start=start,
        dec_idx=dec, dec_lens=(start[dec] + 1).astype(np.int32),
        pf_idx=pf, pf_cu=np.concatenate([[0], np.cumsum(tokens[pf])]).astype(np.int32),
        pf_ctx=start[pf],
        max_chunk=int(tokens[pf].max()) if len(pf) else 0,
        max_total=int((start[pf] + tokens[pf]).max()) if len(pf) else 0)
