"""Device-side plumbing for a generated workload: upload arrays with PyTorch,
build the paged cache, and run the hot path through the C ABI.

``DeviceWorkload.setup()`` fills the cache before the step (prompt tokens
already cached); ``DeviceWorkload.step()`` is one pass of the hot path:
append the step's new tokens, decode attention for every decode sequence
(partial pass, then the log-sum-exp merge) and, for a mixed step, chunked
prefill.  All of it runs in the library's kernels on one stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import POISON, Workload, decode_step_tokens

_TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8,
                  "int8": torch.int8}


def _dev(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """numpy array (float32 / uint16 bf16 bits / uint8 / int8 / int32) -> device tensor."""
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(x.astype(np.float32, copy=False)).to(device)
    if dtype == "fp8":
        return torch.from_numpy(x.astype(np.uint8, copy=False)).to(device)
    if dtype == "int8":
        return torch.from_numpy(x.astype(np.int8, copy=False)).to(device)
    if dtype == "i32":
        return torch.from_numpy(x.astype(np.int32, copy=False)).to(device)
    raise ValueError(dtype)


def poisoned_pool(num_pages: int, Hkv: int, P: int, D: int, kv_dtype: str, device) -> torch.Tensor:
    shape = (num_pages, Hkv, P, D)
    if kv_dtype == "f32":
        return torch.full(shape, int(POISON["f32"].view(np.int32)), dtype=torch.int32,
                          device=device).view(torch.float32)
    if kv_dtype == "bf16":
        return torch.full(shape, int(POISON["bf16"].view(np.int16)), dtype=torch.int16,
                          device=device).view(torch.bfloat16)
    if kv_dtype == "int8":
        return torch.full(shape, int(POISON["int8"]), dtype=torch.int8, device=device)
    return torch.full(shape, int(POISON["fp8"]), dtype=torch.uint8, device=device)


@dataclass
class DeviceBatch:
    k: torch.Tensor
    v: torch.Tensor
    cu: torch.Tensor
    start: torch.Tensor
    bt: torch.Tensor
    rows: int
    tokens: int


@dataclass
class DeviceWorkload:
    wl: Workload
    cache: B.PagedCache
    setup_batch: DeviceBatch
    step_batch: DeviceBatch
    q: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    bt: torch.Tensor
    lens: torch.Tensor
    max_len: int
    split_tokens: int
    workspace: Optional[torch.Tensor]
    pf: dict = field(default_factory=dict)
    _batches: Optional[tuple] = None
    _step_call: Optional[B.DecodeStepCall] = None

    def setup(self, stream=None) -> None:
        self._append(self.setup_batch, stream)

    def _append(self, b: DeviceBatch, stream=None) -> None:
        if b.rows == 0:
            return
        B.pkv_kv_cache_append(self.cache, b.k, b.v, b.cu, b.start, b.bt, stream=stream)

    def append_step(self, stream=None) -> None:
        self._append(self.step_batch, stream)

    def decode(self, stream=None) -> None:
        if self.wl.num_seqs == 0:
            return
        B.pkv_paged_attn_decode(self.cache, self.q, self.out, self.bt, self.lens, self.max_len,
                                float(self.wl.sm_scale), lse=self.lse,
                                split_tokens=self.split_tokens, workspace=self.workspace,
                                stream=stream)

    def decode_step(self, stream=None) -> None:
        """Append every sequence's step token and decode in one attention
        launch (pkv_decode_step).  Decode-only workloads whose sequences each
        append a token of their own."""
        if self.wl.num_seqs == 0:
            return
        if self._step_call is None:
            if self.pf:
                raise ValueError("decode_step: the workload has a prefill part")
            kn, vn = decode_step_tokens(self.wl)
            d, dt = self.q.device, self.wl.spec.kv_in_dtype
            self._step_call = B.DecodeStepCall(
                self.cache, _dev(kn, dt, d), _dev(vn, dt, d), self.q, self.out, self.bt,
                self.lens, self.max_len, float(self.wl.sm_scale), lse=self.lse,
                split_tokens=self.split_tokens, workspace=self.workspace)
        self._step_call(stream)

    def decode_partial(self, stream=None, listed: bool = False) -> None:
        """The partial pass; listed=True takes its items from the work list
        (build_work_list), the order pkv_mixed_step's decode uses."""
        B.pkv_paged_attn_decode_partial(self.cache, self.q, self.out, self.bt, self.lens,
                                        self.max_len, float(self.wl.sm_scale), lse=self.lse,
                                        split_tokens=self.split_tokens, workspace=self.workspace,
                                        stream=stream, listed=listed)

    def build_work_list(self, stream=None) -> None:
        B.pkv_decode_work_list(self.cache, self.lens, self.wl.spec.num_q_heads, self.max_len,
                               split_tokens=self.split_tokens, workspace=self.workspace,
                               stream=stream)

    def merge(self, stream=None) -> None:
        B.pkv_lse_merge(self.cache, self.out, self.lens, self.max_len, lse=self.lse,
                        split_tokens=self.split_tokens, workspace=self.workspace, stream=stream)

    def prefill(self, stream=None) -> None:
        if not self.pf:
            return
        p = self.pf
        B.pkv_paged_attn_chunked_prefill(self.cache, p["q"], p["out"], p["cu"], p["ctx"], p["bt"],
                                         p["max_chunk"], p["max_total"], float(self.wl.sm_scale),
                                         lse=p["lse"], split_tokens=p["split"],
                                         workspace=p["ws"], stream=stream)

    def step(self, stream=None) -> None:
        """One pass of the hot path: append -> decode (partial + merge) -> prefill."""
        self.append_step(stream)
        self.decode(stream)
        self.prefill(stream)

    def mixed_step(self, stream=None, side_stream=None) -> None:
        """The same step in one library call; with side_stream the prefill
        runs concurrently with the decode."""
        if self._batches is None:
            p = self.pf
            a = self.step_batch
            self._batches = (
                B.append_batch(a.k, a.v, a.cu, a.start, a.bt) if a.rows else None,
                B.decode_batch(self.q, self.out, self.bt, self.lens, self.max_len, lse=self.lse,
                               split_tokens=self.split_tokens, workspace=self.workspace)
                if self.wl.num_seqs else None,
                B.prefill_batch(p["q"], p["out"], p["cu"], p["ctx"], p["bt"], p["max_chunk"],
                                p["max_total"], lse=p["lse"], split_tokens=p["split"],
                                workspace=p["ws"]) if p else None)
        B.pkv_mixed_step(self.cache, *self._batches, float(self.wl.sm_scale), stream=stream,
                         side_stream=side_stream)

    def capture_step(self, side_stream=None) -> "torch.cuda.CUDAGraph":
        """Record one step as a HIP graph.

        The library launches only kernels on the caller's streams and
        allocates nothing, so stream capture records the whole step; replaying
        the graph re-runs the same kernels on the same buffers with one launch.
        With side_stream the step is the one-call mixed step whose prefill
        branch forks onto side_stream (the fork and join are captured too).
        (A CUDA graph captured per batch shape is the pages' own remedy for
        launch overhead in small decode steps:
        "TensorRT-LLM框架解析与高性能推理优化实践" §8.1.)"""
        def run():
            if side_stream is None:
                self.step()
            else:
                self.mixed_step(side_stream=side_stream)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):          # warm the capture stream once
            run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
        return g


def upload(wl: Workload, device="cuda", split_tokens: int = 0,
           prefill_split: int = 0) -> DeviceWorkload:
    s = wl.spec
    kp = poisoned_pool(wl.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.kv_dtype, device)
    vp = poisoned_pool(wl.num_pages, s.num_kv_heads, s.page_size, s.head_dim, s.kv_dtype, device)
    ks = vs = None
    if s.kv_dtype in ("fp8", "int8"):
        ks = torch.from_numpy(wl.k_scale).to(device)
        vs = torch.from_numpy(wl.v_scale).to(device)
    cache = B.PagedCache(kp, vp, ks, vs)

    def batch(b) -> DeviceBatch:
        return DeviceBatch(k=_dev(b.k, s.kv_in_dtype, device), v=_dev(b.v, s.kv_in_dtype, device),
                           cu=_dev(b.cu, "i32", device), start=_dev(b.start_pos, "i32", device),
                           bt=_dev(b.block_tables, "i32", device), rows=b.num_rows,
                           tokens=b.num_tokens)

    q = _dev(wl.q, s.q_dtype, device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=device)
    max_len = int(wl.context_lens.max()) if wl.num_seqs else 0
    split = split_tokens or (B.pkv_decode_split_tokens(cache, wl.num_seqs, s.num_q_heads, max_len)
                             if wl.num_seqs else 0)
    ws = (B.decode_workspace(cache, wl.num_seqs, s.num_q_heads, max_len, split)
          if wl.num_seqs else None)
    dw = DeviceWorkload(wl=wl, cache=cache, setup_batch=batch(wl.setup), step_batch=batch(wl.step),
                        q=q, out=out, lse=lse, bt=_dev(wl.block_tables, "i32", device),
                        lens=_dev(wl.context_lens, "i32", device), max_len=max_len,
                        split_tokens=split, workspace=ws)
    if wl.num_prefill:
        pq = _dev(wl.pf_q, s.q_dtype, device)
        chunk = np.diff(wl.pf_cu)
        max_chunk = int(chunk.max())
        max_total = int((wl.pf_ctx_before + chunk).max())
        R, T = wl.num_prefill, pq.shape[0]
        psplit = prefill_split or B.pkv_prefill_split_tokens(cache, R, s.num_q_heads, max_chunk,
                                                             max_total)
        dw.pf = dict(q=pq, out=torch.empty_like(pq),
                     lse=torch.empty(pq.shape[:2], dtype=torch.float32, device=device),
                     cu=_dev(wl.pf_cu, "i32", device), ctx=_dev(wl.pf_ctx_before, "i32", device),
                     bt=_dev(wl.pf_block_tables, "i32", device),
                     max_chunk=max_chunk, max_total=max_total, split=psplit,
                     ws=B.prefill_workspace(cache, R, T, s.num_q_heads, max_chunk, max_total,
                                            psplit))
    return dw


def storage_to_numpy(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the storage representation the oracle uses."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
