"""Paged KV-cache attention, textbook form, float64 on the CPU (oracle; test infrastructure).

What the method computes (pages by title and section):

* Paged cache.  Keys and values live in fixed-size pages of one shared pool;
  each sequence owns a block table that maps its logical page i to a physical
  page, so storage need not be contiguous ("TensorRT-LLM框架解析与高性能推理优化实践"
  §4.2 KV缓存管理细节; §6.2 Paged Attention优化: the kernel reaches K/V through
  the block table; repeated prompts reuse cached pages).  Token t of a
  sequence sits in page ``block_table[t // page_size]`` at slot
  ``t % page_size``.  Pool layout here: ``[num_pages][num_kv_heads][page_size][head_dim]``.

* Attention.  Scaled dot-product attention ("TensorRT-LLM性能调优：提升LLM推理效率",
  layer-fusion discussion, fused multi-head attention row): the score of key t
  for query head h is ``sm_scale * <q_h, k_t>``, softmax over the attended
  keys, output = probability-weighted sum of the values.  The paged-attention
  sketch of §6.2 leaves out the scale and the normalisation; §6.1 (running max
  and running sum) fixes that a normalised, max-shifted softmax is meant.
  That running form and any split of the keys with a log-sum-exp merge are
  exact rewritings of the same softmax, so the oracle uses the direct form.

* Grouped heads (reading; the pages do not describe GQA): query head h reads
  KV head ``h // G`` with ``G = Hq / Hkv``.  G = 1 is multi-head attention.

* Decode: one query per sequence attends its ``L`` cached tokens (its own
  token included).  ``L = 0`` gives output 0 and log-sum-exp -inf.

* Chunked prefill (§5.3 分块上下文处理 of the first page; causal mask from the
  fused-MHA pseudocode of "TensorRT-LLM性能调优"): request r has P_r cached
  tokens and a chunk of C_r new tokens, already in its pages; chunk query i
  (absolute position P_r + i) attends keys 0 .. P_r + i inclusive.

* Append: each new token's K/V row for every KV head is written to
  ``pool[bt[start + i // P]][j][(start + i) % P]``.  fp32/bf16 caches copy;
  an fp8 cache stores ``e4m3fn(float32(x) / float32(scale[j]))`` with
  round-to-nearest-even and saturation (§7.2: one scale per head); an int8
  cache stores the symmetric code of the same quotient (formats.py).

Storage: "f32" float32 arrays, "bf16" uint16 bit patterns, "fp8" uint8 codes,
"int8" int8 codes.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .formats import bf16_to_f64, e4m3fn_to_f64, f32_to_e4m3fn, f32_to_int8_sym, int8_to_f64


# ----------------------------------------------------------- storage -------
def storage_to_f64(raw: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None,
                   head_axis: int = -2) -> np.ndarray:
    """Decode stored elements to float64; fp8 and int8 codes are multiplied by
    their head's scale.

    ``head_axis`` names the KV-head axis of ``raw`` (used only for codes)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(raw)
    if dtype in ("fp8", "int8"):
        x = e4m3fn_to_f64(raw) if dtype == "fp8" else int8_to_f64(raw)
        assert scale is not None
        shape = [1] * x.ndim
        shape[head_axis] = -1
        return x * np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(shape)
    raise ValueError(dtype)


# ------------------------------------------------------------- gather ------
def gather_tokens(pool: np.ndarray, block_table: np.ndarray, length: int,
                  page_size: int) -> np.ndarray:
    """Raw rows of tokens 0..length-1 of one sequence: [length][Hkv][D].

    Token t comes from physical page ``block_table[t // page_size]``, slot
    ``t % page_size`` — the block-table address map of §4.2/§6.2."""
    t = np.arange(length)
    pages = np.asarray(block_table)[t // page_size].astype(np.int64)
    bad = (pages < 0) | (pages >= pool.shape[0])
    if bad.any():
        first = int(np.argmax(bad))
        raise IndexError(f"token {first}: block-table entry {int(pages[first])} outside the pool")
    return pool[pages, :, t % page_size, :]


# ---------------------------------------------------------- attention ------
def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query position over L logically contiguous keys.

    q: [Hq][D] float64; k, v: [L][Hkv][D] float64.  Returns (out [Hq][D],
    lse [Hq]) with lse the natural-log log-sum-exp of the scaled scores."""
    Hq, D = q.shape
    L, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    lse = np.full(Hq, -np.inf, dtype=np.float64)
    if L == 0:
        return out, lse
    sigma = float(np.float64(sm_scale))
    for h in range(Hq):
        j = h // G
        s = sigma * (k[:, j, :] @ q[h])          # [L] scaled scores
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        out[h] = (p @ v[:, j, :]) / l
        lse[h] = m + np.log(l)
    return out, lse


def paged_attn_decode(q: np.ndarray, q_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray,
                      kv_dtype: str, block_tables: np.ndarray, context_lens: np.ndarray,
                      sm_scale: float, k_scale: Optional[np.ndarray] = None,
                      v_scale: Optional[np.ndarray] = None,
                      seqs: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention: sequence b's query over its first ``context_lens[b]`` tokens.

    Returns float64 (out [n][Hq][D], lse [n][Hq]) for the sequences ``seqs``
    (all by default, in order)."""
    P = k_pool.shape[2]
    if seqs is None:
        seqs = np.arange(q.shape[0])
    Hq, D = q.shape[1], q.shape[2]
    out = np.zeros((len(seqs), Hq, D))
    lse = np.zeros((len(seqs), Hq))
    for i, b in enumerate(seqs):
        L = int(context_lens[b])
        k = storage_to_f64(gather_tokens(k_pool, block_tables[b], L, P), kv_dtype, k_scale)
        v = storage_to_f64(gather_tokens(v_pool, block_tables[b], L, P), kv_dtype, v_scale)
        qb = storage_to_f64(q[b], q_dtype)
        out[i], lse[i] = attend(qb, k, v, sm_scale)
    return out, lse


def paged_attn_chunked_prefill(q: np.ndarray, q_dtype: str, k_pool: np.ndarray,
                               v_pool: np.ndarray, kv_dtype: str, cu_q_lens: np.ndarray,
                               ctx_before: np.ndarray, block_tables: np.ndarray,
                               sm_scale: float, k_scale: Optional[np.ndarray] = None,
                               v_scale: Optional[np.ndarray] = None,
                               rows: Optional[np.ndarray] = None
                               ) -> Tuple[np.ndarray, np.ndarray]:
    """Causal chunked prefill over paged K/V.

    Packed queries ``q [T][Hq][D]``; request r owns rows cu_q_lens[r]..cu_q_lens[r+1]-1.
    Chunk row i of request r attends keys 0 .. ctx_before[r] + i.  Returns
    float64 (out, lse) for the packed rows ``rows`` (all by default)."""
    P = k_pool.shape[2]
    T, Hq, D = q.shape
    if rows is None:
        rows = np.arange(T)
    req_of = np.searchsorted(cu_q_lens, np.arange(T), side="right") - 1
    out = np.zeros((len(rows), Hq, D))
    lse = np.zeros((len(rows), Hq))
    cache = {}
    for n, t in enumerate(rows):
        r = int(req_of[t])
        i = int(t - cu_q_lens[r])
        last = int(ctx_before[r]) + i          # inclusive causal boundary
        if r not in cache:
            total = int(ctx_before[r]) + int(cu_q_lens[r + 1] - cu_q_lens[r])
            cache = {r: (storage_to_f64(gather_tokens(k_pool, block_tables[r], total, P),
                                        kv_dtype, k_scale),
                         storage_to_f64(gather_tokens(v_pool, block_tables[r], total, P),
                                        kv_dtype, v_scale))}
        k, v = cache[r]
        out[n], lse[n] = attend(storage_to_f64(q[t], q_dtype), k[:last + 1], v[:last + 1],
                                sm_scale)
    return out, lse


# ------------------------------------------------- context attention -------
def context_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: str,
                      cu_seqlens: np.ndarray, sm_scale: float,
                      rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Causal attention of whole prompts over their own contiguous K/V
    (fused MHA with a causal mask, "TensorRT-LLM性能调优：提升LLM推理效率"; the
    context_fmha path of "如何用TensorRT-LLM和Triton Server实现LLM的高效推理？…" §2).

    Packed q [T][Hq][D], k/v [T][Hkv][D]; sequence s owns rows
    cu_seqlens[s] .. cu_seqlens[s+1]-1, and its token i attends its tokens
    0..i.  Returns float64 (out, lse) for the packed rows ``rows`` (all by
    default)."""
    T, Hq, D = q.shape
    if rows is None:
        rows = np.arange(T)
    seq_of = np.searchsorted(cu_seqlens, np.arange(T), side="right") - 1
    out = np.zeros((len(rows), Hq, D))
    lse = np.zeros((len(rows), Hq))
    for n, t in enumerate(rows):
        c0 = int(cu_seqlens[int(seq_of[t])])
        kk = storage_to_f64(k[c0:t + 1], dtype)
        vv = storage_to_f64(v[c0:t + 1], dtype)
        out[n], lse[n] = attend(storage_to_f64(q[t], dtype), kk, vv, sm_scale)
    return out, lse


# ----------------------------------------------------- split + merge -------
def split_partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                   split: int):
    """Per key-range partial states (m, l, acc) of the softmax for one query position.

    Range s covers keys [s*split, (s+1)*split).  m = max score of the range,
    l = sum exp(score - m), acc = sum exp(score - m) * v (unnormalised)."""
    Hq, D = q.shape
    L = k.shape[0]
    G = Hq // k.shape[1]
    parts = []
    for s0 in range(0, L, split):
        ks, vs = k[s0:s0 + split], v[s0:s0 + split]
        m = np.empty(Hq)
        l = np.empty(Hq)
        acc = np.empty((Hq, D))
        for h in range(Hq):
            sc = float(sm_scale) * (ks[:, h // G, :] @ q[h])
            m[h] = sc.max()
            p = np.exp(sc - m[h])
            l[h] = p.sum()
            acc[h] = p @ vs[:, h // G, :]
        parts.append((m, l, acc))
    return parts


def lse_merge(parts) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial states: M = max m_s, w_s = exp(m_s - M),
    out = sum w_s acc_s / sum w_s l_s, lse = M + ln(sum w_s l_s)."""
    ms = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    accs = np.stack([p[2] for p in parts])
    M = ms.max(axis=0)
    w = np.exp(ms - M)
    denom = (w * ls).sum(axis=0)
    out = (w[:, :, None] * accs).sum(axis=0) / denom[:, None]
    return out, M + np.log(denom)


# -------------------------------------------------------------- append -----
def kv_cache_append(k_pool: np.ndarray, v_pool: np.ndarray, kv_dtype: str,
                    k_new: np.ndarray, v_new: np.ndarray, in_dtype: str,
                    cu_new: np.ndarray, start_pos: np.ndarray, block_tables: np.ndarray,
                    k_scale: Optional[np.ndarray] = None,
                    v_scale: Optional[np.ndarray] = None,
                    rows: Optional[np.ndarray] = None) -> None:
    """Scatter new tokens into their page slots, in place.

    Row r's new token i lands at position start_pos[r] + i of that row:
    page ``block_tables[r][pos // P]``, slot ``pos % P``, for every KV head.
    Copies for fp32/bf16 caches (input dtype must equal the cache dtype); an
    fp8 cache takes float32 input and stores e4m3fn(x / scale[head]), an int8
    cache the symmetric code of x / scale[head], the division done in float32.
    ``rows`` restricts the work to some rows."""
    P = k_pool.shape[2]
    if rows is None:
        rows = range(start_pos.shape[0])
    for r in rows:
        t0, t1 = int(cu_new[r]), int(cu_new[r + 1])
        if kv_dtype in ("fp8", "int8"):
            assert in_dtype == "f32"
            enc = f32_to_e4m3fn if kv_dtype == "fp8" else f32_to_int8_sym
            ks = np.asarray(k_scale, dtype=np.float32)[None, :, None]
            vs = np.asarray(v_scale, dtype=np.float32)[None, :, None]
            kq = enc(np.asarray(k_new[t0:t1], dtype=np.float32) / ks)
            vq = enc(np.asarray(v_new[t0:t1], dtype=np.float32) / vs)
        else:
            assert in_dtype == kv_dtype
            kq, vq = k_new[t0:t1], v_new[t0:t1]
        for i in range(t1 - t0):
            pos = int(start_pos[r]) + i
            page = int(block_tables[r][pos // P])
            if page < 0 or page >= k_pool.shape[0]:
                raise IndexError(f"row {r} position {pos}: no page")
            k_pool[page, :, pos % P, :] = kq[i]
            v_pool[page, :, pos % P, :] = vq[i]
