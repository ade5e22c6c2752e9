"""Python binding of the C ABI in ``include/pagedkv.h`` (ctypes).

Argument marshalling only: every function here checks that tensors have the
layout the C call documents, passes raw device pointers, sizes and the current
HIP stream to ``libpagedkv.so``, and raises ``PkvError`` on a non-OK status.
Every step of the computation runs in the library's HIP kernels.  PyTorch
supplies device memory and streams.

The library is loaded from the package directory (built in-tree by
``python -m paged_kv_cache_277_amd.build``); if it is missing the import
fails with an error that says so — there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_OUT_OF_PAGES, \
    PKV_ERR_BAD_BLOCK_TABLE, PKV_ERR_HIP = range(6)
PKV_F32, PKV_BF16, PKV_FP8_E4M3FN, PKV_INT8 = 0, 1, 2, 3
_STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_UNSUPPORTED",
                 3: "PKV_ERR_OUT_OF_PAGES", 4: "PKV_ERR_BAD_BLOCK_TABLE", 5: "PKV_ERR_HIP"}
DTYPE_CODES = {"f32": PKV_F32, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3FN, "int8": PKV_INT8}


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class CacheDescStruct(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p),
                ("num_pages", C.c_int32), ("num_kv_heads", C.c_int32),
                ("page_size", C.c_int32), ("head_dim", C.c_int32), ("kv_dtype", C.c_int32)]


class AppendBatchStruct(C.Structure):
    _fields_ = [("k_new", C.c_void_p), ("v_new", C.c_void_p), ("in_dtype", C.c_int32),
                ("cu_new_tokens", C.c_void_p), ("start_pos", C.c_void_p),
                ("block_tables", C.c_void_p), ("bt_stride", C.c_int32), ("num_rows", C.c_int32),
                ("num_new_tokens", C.c_int32)]


class DecodeBatchStruct(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_dtype", C.c_int32), ("out", C.c_void_p),
                ("out_dtype", C.c_int32), ("lse", C.c_void_p), ("block_tables", C.c_void_p),
                ("bt_stride", C.c_int32), ("context_lens", C.c_void_p), ("num_seqs", C.c_int32),
                ("num_q_heads", C.c_int32), ("max_context_len", C.c_int32),
                ("split_tokens", C.c_int32), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t)]


class PrefillBatchStruct(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_dtype", C.c_int32), ("out", C.c_void_p),
                ("out_dtype", C.c_int32), ("lse", C.c_void_p), ("cu_q_lens", C.c_void_p),
                ("ctx_before", C.c_void_p), ("block_tables", C.c_void_p),
                ("bt_stride", C.c_int32), ("num_reqs", C.c_int32), ("num_q_tokens", C.c_int32),
                ("num_q_heads", C.c_int32), ("max_chunk_len", C.c_int32),
                ("max_total_len", C.c_int32), ("split_tokens", C.c_int32),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t)]


class SchedConfigStruct(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("max_batch_size", C.c_int32), ("max_num_tokens", C.c_int32),
                ("chunk_size", C.c_int32), ("policy", C.c_int32)]


class SchedItemStruct(C.Structure):
    _fields_ = [("req_id", C.c_int64), ("slot", C.c_int32), ("kind", C.c_int32),
                ("start_pos", C.c_int32), ("num_tokens", C.c_int32)]


class SchedRequestStateStruct(C.Structure):
    _fields_ = [("num_tokens", C.c_int32), ("num_computed", C.c_int32),
                ("generated", C.c_int32), ("num_pages", C.c_int32), ("slot", C.c_int32),
                ("running", C.c_int32)]


class SchedCountsStruct(C.Structure):
    _fields_ = [("waiting", C.c_int32), ("running", C.c_int32), ("free_pages", C.c_int32),
                ("preemptions", C.c_int64)]


_P = C.c_void_p
_I = C.c_int32
_F = C.c_float
_SZ = C.c_size_t
_SIGS = {
    "pkv_version": (C.c_char_p, []),
    "pkv_last_error": (C.c_char_p, []),
    "pkv_allocator_create": (_I, [_I, C.POINTER(C.c_void_p)]),
    "pkv_allocator_destroy": (None, [_P]),
    "pkv_alloc_pages": (_I, [_P, _I, _P]),
    "pkv_share_pages": (_I, [_P, _I, _P]),
    "pkv_free_pages": (_I, [_P, _I, _P]),
    "pkv_num_free_pages": (_I, [_P]),
    "pkv_page_refcount": (_I, [_P, _I]),
    "pkv_kv_cache_append": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _P]),
    "pkv_decode_split_tokens": (_I, [_P, _I, _I, _I]),
    "pkv_decode_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I]),
    "pkv_paged_attn_decode": (_I, [_P, _P, _I, _P, _I, _P, _P, _I, _P, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "pkv_decode_step": (_I, [_P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _I, _I, _I, _F, _I,
                             _P, _SZ, _P]),
    "pkv_paged_attn_decode_noalloc": (_I, [_P, _P, _I, _P, _I, _P, _P, _I, _P, _I, _I, _I, _F, _I, _P]),
    "pkv_paged_attn_decode_partial": (_I, [_P, _P, _I, _P, _I, _P, _P, _I, _P, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "pkv_paged_attn_decode_partial_listed": (_I, [_P, _P, _I, _P, _I, _P, _P, _I, _P, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "pkv_decode_work_list": (_I, [_P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "pkv_lse_merge": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "pkv_paged_attn_chunked_prefill": (_I, [_P, _P, _I, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I,
                                            _I, _I, _F, _I, _P, _SZ, _P]),
    "pkv_prefill_split_tokens": (_I, [_P, _I, _I, _I, _I]),
    "pkv_prefill_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I, _I, _I]),
    "pkv_mixed_step": (_I, [_P, _P, _P, _P, _F, _P, _P]),
    "pkv_context_fmha": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                              _SZ, _P]),
    "pkv_context_fmha_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "pkv_validate_block_tables": (_I, [_P, _P, _I, _P, _I, _P]),
    "pkv_sched_create": (_I, [_P, C.POINTER(C.c_void_p)]),
    "pkv_sched_destroy": (None, [_P]),
    "pkv_sched_add_prefix": (_I, [_P, C.c_int64, _I, _P]),
    "pkv_sched_remove_prefix": (_I, [_P, C.c_int64]),
    "pkv_sched_add_request": (_I, [_P, C.c_int64, _I, _I, C.c_int64]),
    "pkv_sched_schedule": (_I, [_P, _P, _I, _P, _P, _I, _P]),
    "pkv_sched_block_table": (_I, [_P, C.c_int64, _P, _I]),
    "pkv_sched_commit": (_I, [_P, _P, _I, _P]),
    "pkv_sched_finish": (_I, [_P, C.c_int64]),
    "pkv_sched_query": (_I, [_P, C.c_int64, _P]),
    "pkv_sched_stats": (_I, [_P, _P]),
    "pkv_fp8_e4m3fn_to_f32": (_I, [_P, _P, C.c_int64, _P]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def lib() -> C.CDLL:
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m paged_kv_cache_277_amd.build` (no fallback exists)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, lib().pkv_last_error().decode(errors="replace"))


def version() -> str:
    return lib().pkv_version().decode()


# ------------------------------------------------------------ helpers -------
_gpu_present: Optional[bool] = None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of a tensor the library reads or writes.  Where a GPU
    is present, a tensor in host memory is refused here: its address would
    reach a kernel, which cannot read it.  (Empty tensors are never read.)"""
    global _gpu_present
    if t is None:
        return None
    if t.device.type != "cuda" and t.numel() > 0:
        if _gpu_present is None:
            _gpu_present = torch.cuda.is_available()
        if _gpu_present:
            raise ValueError(f"a tensor on {t.device} was passed where the library takes GPU "
                             "memory")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _code_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3FN
    if t.dtype == torch.int8:
        return PKV_INT8
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def _i32(t: torch.Tensor, name: str) -> None:
    _need(t.dtype == torch.int32 and t.is_contiguous(), f"{name} must be contiguous int32")


@dataclass
class PagedCache:
    """One layer's paged cache: K/V pools [num_pages][Hkv][page][D] on the device.

    fp8 pools are uint8 (or float8_e4m3fn) tensors with float32 per-head scales."""
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    def __post_init__(self):
        _need(self.k_pool.shape == self.v_pool.shape and self.k_pool.dim() == 4,
              "k_pool/v_pool must both be [num_pages][Hkv][page][D]")
        _need(self.k_pool.dtype == self.v_pool.dtype, "k_pool/v_pool dtypes differ")
        _need(self.k_pool.is_contiguous() and self.v_pool.is_contiguous(), "pools must be contiguous")
        for s in (self.k_scale, self.v_scale):
            if s is not None:
                _need(s.dtype == torch.float32 and s.is_contiguous(), "scales must be float32")
        n, h, p, d = self.k_pool.shape
        self._s = CacheDescStruct(_ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.k_scale),
                                  _ptr(self.v_scale), n, h, p, d, _code_of(self.k_pool))

    @property
    def num_pages(self) -> int: return self.k_pool.shape[0]
    @property
    def num_kv_heads(self) -> int: return self.k_pool.shape[1]
    @property
    def page_size(self) -> int: return self.k_pool.shape[2]
    @property
    def head_dim(self) -> int: return self.k_pool.shape[3]
    @property
    def kv_dtype(self) -> int: return self._s.kv_dtype

    @property
    def desc(self):
        return C.byref(self._s)


# ---------------------------------------------------------- allocator -------
PKV_SCHED_CONSERVATIVE, PKV_SCHED_AGGRESSIVE = 0, 1
PKV_WORK_PREFILL, PKV_WORK_DECODE = 0, 1


class Scheduler:
    """Host step scheduler with its KV-cache page manager (pkv_sched_*).

    schedule() returns ([(req_id, slot, kind, start_pos, num_tokens)], [evicted
    req_ids]); commit() records the step as executed and returns the finished
    req_ids."""

    def __init__(self, num_pages: int, page_size: int, max_batch_size: int,
                 max_num_tokens: int, chunk_size: int, policy: int = PKV_SCHED_AGGRESSIVE):
        cfg = SchedConfigStruct(num_pages, page_size, max_batch_size, max_num_tokens, chunk_size,
                                policy)
        h = C.c_void_p()
        _check(lib().pkv_sched_create(C.byref(cfg), C.byref(h)))
        self._h = h
        self.page_size = page_size
        self.max_batch_size = max_batch_size
        self._items = (SchedItemStruct * max_batch_size)()
        self._ids = (C.c_int64 * max_batch_size)()
        self._n = C.c_int32()
        self._m = C.c_int32()

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pkv_sched_destroy(h)
            self._h = None

    def add_prefix(self, prefix_id: int, num_tokens: int) -> list:
        out = (C.c_int32 * max(1, num_tokens // self.page_size))()
        _check(lib().pkv_sched_add_prefix(self._h, prefix_id, num_tokens, out))
        return list(out)[: num_tokens // self.page_size]

    def remove_prefix(self, prefix_id: int) -> None:
        _check(lib().pkv_sched_remove_prefix(self._h, prefix_id))

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int,
                    prefix_id: int = -1) -> None:
        _check(lib().pkv_sched_add_request(self._h, req_id, prompt_len, max_new_tokens,
                                           prefix_id))

    def schedule(self):
        _check(lib().pkv_sched_schedule(self._h, self._items, self.max_batch_size,
                                        C.byref(self._n), self._ids, self.max_batch_size,
                                        C.byref(self._m)))
        items = [(it.req_id, it.slot, it.kind, it.start_pos, it.num_tokens)
                 for it in self._items[: self._n.value]]
        return items, list(self._ids[: self._m.value])

    def block_table(self, req_id: int) -> list:
        n = lib().pkv_sched_block_table(self._h, req_id, None, 0)
        _need(n >= 0, f"unknown request {req_id}")
        out = (C.c_int32 * max(1, n))()
        lib().pkv_sched_block_table(self._h, req_id, out, n)
        return list(out)[:n]

    def commit(self) -> list:
        _check(lib().pkv_sched_commit(self._h, self._ids, self.max_batch_size,
                                      C.byref(self._n)))
        return list(self._ids[: self._n.value])

    def finish(self, req_id: int) -> None:
        _check(lib().pkv_sched_finish(self._h, req_id))

    def query(self, req_id: int) -> dict:
        st = SchedRequestStateStruct()
        _check(lib().pkv_sched_query(self._h, req_id, C.byref(st)))
        return {k: getattr(st, k) for k, _ in st._fields_}

    def stats(self) -> dict:
        st = SchedCountsStruct()
        _check(lib().pkv_sched_stats(self._h, C.byref(st)))
        return {k: getattr(st, k) for k, _ in st._fields_}


class PageAllocator:
    """Host page allocator (refcounted; all-or-nothing allocation)."""

    def __init__(self, num_pages: int):
        h = C.c_void_p()
        _check(lib().pkv_allocator_create(num_pages, C.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int) -> list:
        out = (C.c_int32 * max(1, n))()
        _check(lib().pkv_alloc_pages(self._h, n, out))
        return list(out[:n])

    def share(self, ids) -> None:
        arr = (C.c_int32 * max(1, len(ids)))(*ids)
        _check(lib().pkv_share_pages(self._h, len(ids), arr))

    def free(self, ids) -> None:
        arr = (C.c_int32 * max(1, len(ids)))(*ids)
        _check(lib().pkv_free_pages(self._h, len(ids), arr))

    @property
    def num_free(self) -> int:
        return lib().pkv_num_free_pages(self._h)

    def refcount(self, page: int) -> int:
        return lib().pkv_page_refcount(self._h, page)


# ------------------------------------------------------------- kernels ------
def pkv_kv_cache_append(cache: PagedCache, k_new: torch.Tensor, v_new: torch.Tensor,
                        cu_new_tokens: torch.Tensor, start_pos: torch.Tensor,
                        block_tables: torch.Tensor, stream=None) -> None:
    """Scatter packed new tokens [T][Hkv][D] into their page slots."""
    _need(k_new.shape == v_new.shape and k_new.dim() == 3, "k_new/v_new must be [T][Hkv][D]")
    _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new/v_new must be contiguous")
    _need(k_new.shape[1:] == (cache.num_kv_heads, cache.head_dim), "k_new shape mismatch")
    for t, n in ((cu_new_tokens, "cu_new_tokens"), (start_pos, "start_pos"),
                 (block_tables, "block_tables")):
        _i32(t, n)
    rows = start_pos.shape[0]
    _need(cu_new_tokens.shape[0] == rows + 1 and block_tables.shape[0] == rows, "row counts differ")
    _check(lib().pkv_kv_cache_append(cache.desc, _ptr(k_new), _ptr(v_new), _code_of(k_new),
                                     _ptr(cu_new_tokens), _ptr(start_pos), _ptr(block_tables),
                                     block_tables.shape[1] if block_tables.dim() == 2 else 0,
                                     rows, k_new.shape[0], _stream(stream)))


def pkv_decode_split_tokens(cache: PagedCache, num_seqs: int, num_q_heads: int,
                            max_context_len: int) -> int:
    return lib().pkv_decode_split_tokens(cache.desc, num_seqs, num_q_heads, max_context_len)


def pkv_decode_workspace_bytes(cache: PagedCache, num_seqs: int, num_q_heads: int,
                               max_context_len: int, split_tokens: int = 0) -> int:
    return lib().pkv_decode_workspace_bytes(cache.desc, num_seqs, num_q_heads, max_context_len,
                                            split_tokens)


def decode_workspace(cache: PagedCache, num_seqs: int, num_q_heads: int, max_context_len: int,
                     split_tokens: int = 0) -> Optional[torch.Tensor]:
    """A device buffer of the size the decode call needs (None if it needs none)."""
    n = pkv_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_context_len, split_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=cache.k_pool.device)


def _decode_args(cache, q, out, lse, block_tables, context_lens):
    _need(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B][Hq][D]")
    _need(out.shape == q.shape and out.is_contiguous(), "out must be contiguous like q")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == q.shape[0], "block_tables rows")
    _need(context_lens.shape[0] == q.shape[0], "context_lens length")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.shape == q.shape[:2] and lse.is_contiguous(),
              "lse must be float32 [B][Hq]")


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def pkv_paged_attn_decode(cache: PagedCache, q: torch.Tensor, out: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          max_context_len: int, sm_scale: float, lse: Optional[torch.Tensor] = None,
                          split_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> None:
    """Decode attention (partial pass + log-sum-exp merge)."""
    _decode_args(cache, q, out, lse, block_tables, context_lens)
    wp, wb = _ws(workspace)
    _check(lib().pkv_paged_attn_decode(cache.desc, _ptr(q), _code_of(q), _ptr(out), _code_of(out),
                                       _ptr(lse), _ptr(block_tables), block_tables.shape[1],
                                       _ptr(context_lens), q.shape[0], q.shape[1], max_context_len,
                                       float(sm_scale), split_tokens, wp, wb, _stream(stream)))


class DecodeStepCall:
    """pkv_decode_step with its arguments checked and marshalled once; each
    call issues the C call alone (for launch-bound step loops).  It holds the
    tensors, so their memory stays allocated while it lives."""

    def __init__(self, cache: PagedCache, k_new: torch.Tensor, v_new: torch.Tensor,
                 q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, max_context_len: int, sm_scale: float,
                 lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                 workspace: Optional[torch.Tensor] = None):
        _decode_args(cache, q, out, lse, block_tables, context_lens)
        _need(k_new.shape == v_new.shape and k_new.dim() == 3, "k_new/v_new must be [B][Hkv][D]")
        _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new/v_new must be contiguous")
        _need(k_new.shape == (q.shape[0], cache.num_kv_heads, cache.head_dim),
              "k_new shape mismatch")
        wp, wb = _ws(workspace)
        self._fn = lib().pkv_decode_step
        self._args = (cache.desc, _ptr(k_new), _ptr(v_new), _code_of(k_new), _ptr(q),
                      _code_of(q), _ptr(out), _code_of(out), _ptr(lse), _ptr(block_tables),
                      block_tables.shape[1], _ptr(context_lens), q.shape[0], q.shape[1],
                      max_context_len, float(sm_scale), split_tokens, wp, wb)
        self._tensors = (cache, k_new, v_new, q, out, lse, block_tables, context_lens, workspace)

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def pkv_decode_step(cache: PagedCache, k_new: torch.Tensor, v_new: torch.Tensor,
                    q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_context_len: int, sm_scale: float,
                    lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """One decode step in one attention launch: sequence s's new token
    (k_new[s], v_new[s], [B][Hkv][D]) is written at position
    context_lens[s] - 1, then the sequence's query attends its context."""
    DecodeStepCall(cache, k_new, v_new, q, out, block_tables, context_lens, max_context_len,
                   sm_scale, lse, split_tokens, workspace)(stream)


NOALLOC_SCRATCH_BYTES = 32 << 20      # PKV_NOALLOC_SCRATCH_BYTES of include/pagedkv.h


def pkv_paged_attn_decode_noalloc(cache: PagedCache, q: torch.Tensor, out: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  max_context_len: int, sm_scale: float,
                                  lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                                  stream=None) -> None:
    """Decode attention with the partials in the library's fixed per-GPU
    array: no workspace, no device allocation."""
    _decode_args(cache, q, out, lse, block_tables, context_lens)
    _check(lib().pkv_paged_attn_decode_noalloc(cache.desc, _ptr(q), _code_of(q), _ptr(out),
                                               _code_of(out), _ptr(lse), _ptr(block_tables),
                                               block_tables.shape[1], _ptr(context_lens),
                                               q.shape[0], q.shape[1], max_context_len,
                                               float(sm_scale), split_tokens, _stream(stream)))


def pkv_paged_attn_decode_partial(cache: PagedCache, q: torch.Tensor, out: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  max_context_len: int, sm_scale: float,
                                  lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                                  workspace: Optional[torch.Tensor] = None, stream=None,
                                  listed: bool = False) -> None:
    """The partial pass; with listed=True, pkv_paged_attn_decode_partial_listed
    (items in the order of the work list pkv_decode_work_list wrote)."""
    _decode_args(cache, q, out, lse, block_tables, context_lens)
    wp, wb = _ws(workspace)
    f = lib().pkv_paged_attn_decode_partial_listed if listed else lib().pkv_paged_attn_decode_partial
    _check(f(cache.desc, _ptr(q), _code_of(q), _ptr(out), _code_of(out), _ptr(lse),
             _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0], q.shape[1],
             max_context_len, float(sm_scale), split_tokens, wp, wb, _stream(stream)))


def pkv_decode_work_list(cache: PagedCache, context_lens: torch.Tensor, num_q_heads: int,
                         max_context_len: int, split_tokens: int = 0,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Order a decode call's work items longest first into its workspace."""
    _i32(context_lens, "context_lens")
    wp, wb = _ws(workspace)
    _check(lib().pkv_decode_work_list(cache.desc, _ptr(context_lens), context_lens.shape[0],
                                      num_q_heads, max_context_len, split_tokens, wp, wb,
                                      _stream(stream)))


def pkv_lse_merge(cache: PagedCache, out: torch.Tensor, context_lens: torch.Tensor,
                  max_context_len: int, lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _i32(context_lens, "context_lens")
    wp, wb = _ws(workspace)
    _check(lib().pkv_lse_merge(cache.desc, _ptr(out), _code_of(out), _ptr(lse), _ptr(context_lens),
                               out.shape[0], out.shape[1], max_context_len, split_tokens, wp, wb,
                               _stream(stream)))


def pkv_prefill_split_tokens(cache: PagedCache, num_reqs: int, num_q_heads: int,
                             max_chunk_len: int, max_total_len: int) -> int:
    return lib().pkv_prefill_split_tokens(cache.desc, num_reqs, num_q_heads, max_chunk_len,
                                          max_total_len)


def pkv_prefill_workspace_bytes(cache: PagedCache, num_reqs: int, num_q_tokens: int,
                                num_q_heads: int, max_chunk_len: int, max_total_len: int,
                                split_tokens: int = 0) -> int:
    return lib().pkv_prefill_workspace_bytes(cache.desc, num_reqs, num_q_tokens, num_q_heads,
                                             max_chunk_len, max_total_len, split_tokens)


def prefill_workspace(cache: PagedCache, num_reqs: int, num_q_tokens: int, num_q_heads: int,
                      max_chunk_len: int, max_total_len: int,
                      split_tokens: int = 0) -> Optional[torch.Tensor]:
    """A device buffer of the size the prefill call needs (None if it needs none)."""
    n = pkv_prefill_workspace_bytes(cache, num_reqs, num_q_tokens, num_q_heads, max_chunk_len,
                                    max_total_len, split_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=cache.k_pool.device)


def pkv_paged_attn_chunked_prefill(cache: PagedCache, q: torch.Tensor, out: torch.Tensor,
                                   cu_q_lens: torch.Tensor, ctx_before: torch.Tensor,
                                   block_tables: torch.Tensor, max_chunk_len: int,
                                   max_total_len: int, sm_scale: float,
                                   lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                                   workspace: Optional[torch.Tensor] = None,
                                   stream=None) -> None:
    """Causal chunked prefill over packed query rows [T][Hq][D] (key ranges
    plus the log-sum-exp merge when the workspace holds several ranges)."""
    _need(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [T][Hq][D]")
    _need(out.shape == q.shape and out.is_contiguous(), "out must be contiguous like q")
    for t, n in ((cu_q_lens, "cu_q_lens"), (ctx_before, "ctx_before"),
                 (block_tables, "block_tables")):
        _i32(t, n)
    R = ctx_before.shape[0]
    _need(cu_q_lens.shape[0] == R + 1 and block_tables.shape[0] == R, "request counts differ")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.shape == q.shape[:2] and lse.is_contiguous(),
              "lse must be float32 [T][Hq]")
    wp, wb = _ws(workspace)
    _check(lib().pkv_paged_attn_chunked_prefill(
        cache.desc, _ptr(q), _code_of(q), _ptr(out), _code_of(out), _ptr(lse), _ptr(cu_q_lens),
        _ptr(ctx_before), _ptr(block_tables), block_tables.shape[1], R, q.shape[0], q.shape[1],
        max_chunk_len, max_total_len, float(sm_scale), split_tokens, wp, wb, _stream(stream)))


def context_workspace(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int,
                      head_dim: int, max_seqlen: int, split_tokens: int = 0,
                      device="cuda") -> Optional[torch.Tensor]:
    n = lib().pkv_context_fmha_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads,
                                               head_dim, max_seqlen, split_tokens)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def pkv_context_fmha(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                     cu_seqlens: torch.Tensor, max_seqlen: int, sm_scale: float,
                     lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Causal attention of whole prompts over contiguous K/V (no pages)."""
    _need(q.dim() == 3 and q.is_contiguous() and out.shape == q.shape and out.is_contiguous(),
          "q / out must be contiguous [T][Hq][D]")
    _need(k.dim() == 3 and k.shape == v.shape and k.is_contiguous() and v.is_contiguous()
          and k.shape[0] == q.shape[0] and k.shape[2] == q.shape[2],
          "k / v must be contiguous [T][Hkv][D] like q")
    _need(q.dtype == k.dtype == v.dtype == out.dtype, "q, k, v and out share one dtype")
    _i32(cu_seqlens, "cu_seqlens")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.shape == q.shape[:2] and lse.is_contiguous(),
              "lse must be float32 [T][Hq]")
    wp, wb = _ws(workspace)
    _check(lib().pkv_context_fmha(_ptr(q), _ptr(k), _ptr(v), _code_of(q), _ptr(out), _ptr(lse),
                                  _ptr(cu_seqlens), cu_seqlens.shape[0] - 1, q.shape[0],
                                  q.shape[1], k.shape[1], q.shape[2], max_seqlen,
                                  float(sm_scale), split_tokens, wp, wb, _stream(stream)))


def append_batch(k_new: torch.Tensor, v_new: torch.Tensor, cu_new_tokens: torch.Tensor,
                 start_pos: torch.Tensor, block_tables: torch.Tensor) -> AppendBatchStruct:
    """The append part of pkv_mixed_step (tensors as for pkv_kv_cache_append).

    The struct carries raw device pointers; it also holds references to the
    tensors so their memory stays allocated for as long as the struct lives
    (the batch helpers below do the same)."""
    for t, n in ((cu_new_tokens, "cu_new_tokens"), (start_pos, "start_pos"),
                 (block_tables, "block_tables")):
        _i32(t, n)
    _need(k_new.shape == v_new.shape and k_new.is_contiguous() and v_new.is_contiguous(),
          "k_new / v_new must be contiguous [T][Hkv][D]")
    b = AppendBatchStruct(_ptr(k_new), _ptr(v_new), _code_of(k_new), _ptr(cu_new_tokens),
                          _ptr(start_pos), _ptr(block_tables),
                          block_tables.shape[1] if block_tables.dim() == 2 else 0,
                          start_pos.shape[0], k_new.shape[0])
    b._tensors = (k_new, v_new, cu_new_tokens, start_pos, block_tables)
    return b


def decode_batch(q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, max_context_len: int,
                 lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                 workspace: Optional[torch.Tensor] = None) -> DecodeBatchStruct:
    """The decode part of pkv_mixed_step (arguments as for pkv_paged_attn_decode)."""
    _decode_args(None, q, out, lse, block_tables, context_lens)
    wp, wb = _ws(workspace)
    b = DecodeBatchStruct(_ptr(q), _code_of(q), _ptr(out), _code_of(out), _ptr(lse),
                          _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                          q.shape[0], q.shape[1], max_context_len, split_tokens, wp, wb)
    b._tensors = (q, out, lse, block_tables, context_lens, workspace)
    return b


def prefill_batch(q: torch.Tensor, out: torch.Tensor, cu_q_lens: torch.Tensor,
                  ctx_before: torch.Tensor, block_tables: torch.Tensor, max_chunk_len: int,
                  max_total_len: int, lse: Optional[torch.Tensor] = None, split_tokens: int = 0,
                  workspace: Optional[torch.Tensor] = None) -> PrefillBatchStruct:
    """The prefill part of pkv_mixed_step (arguments as for
    pkv_paged_attn_chunked_prefill)."""
    _need(q.dim() == 3 and q.is_contiguous() and out.shape == q.shape and out.is_contiguous(),
          "q / out must be contiguous [T][Hq][D]")
    for t, n in ((cu_q_lens, "cu_q_lens"), (ctx_before, "ctx_before"),
                 (block_tables, "block_tables")):
        _i32(t, n)
    R = ctx_before.shape[0]
    _need(cu_q_lens.shape[0] == R + 1 and block_tables.shape[0] == R, "request counts differ")
    wp, wb = _ws(workspace)
    b = PrefillBatchStruct(_ptr(q), _code_of(q), _ptr(out), _code_of(out), _ptr(lse),
                           _ptr(cu_q_lens), _ptr(ctx_before), _ptr(block_tables),
                           block_tables.shape[1], R, q.shape[0], q.shape[1], max_chunk_len,
                           max_total_len, split_tokens, wp, wb)
    b._tensors = (q, out, lse, cu_q_lens, ctx_before, block_tables, workspace)
    return b


def pkv_mixed_step(cache: PagedCache, append: Optional[AppendBatchStruct],
                   decode: Optional[DecodeBatchStruct], prefill: Optional[PrefillBatchStruct],
                   sm_scale: float, stream=None, side_stream=None) -> None:
    """Append, then decode and prefill (concurrently when side_stream is given)."""
    side = None if side_stream is None else _stream(side_stream)
    _check(lib().pkv_mixed_step(cache.desc, None if append is None else C.byref(append),
                                None if decode is None else C.byref(decode),
                                None if prefill is None else C.byref(prefill), float(sm_scale),
                                _stream(stream), side))


def pkv_validate_block_tables(cache: PagedCache, block_tables: torch.Tensor, lens: torch.Tensor,
                              stream=None) -> None:
    _i32(block_tables, "block_tables")
    _i32(lens, "lens")
    _check(lib().pkv_validate_block_tables(cache.desc, _ptr(block_tables), block_tables.shape[1],
                                           _ptr(lens), lens.shape[0], _stream(stream)))


def pkv_fp8_e4m3fn_to_f32(codes: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _need(codes.dtype in (torch.uint8, torch.float8_e4m3fn) and codes.is_contiguous(), "codes")
    _need(out.dtype == torch.float32 and out.numel() == codes.numel(), "out")
    _check(lib().pkv_fp8_e4m3fn_to_f32(_ptr(codes), _ptr(out), codes.numel(), _stream(stream)))
