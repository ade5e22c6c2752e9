"""Seeded synthetic workloads for paged KV-cache attention.

This module only draws random numbers and lays out indices: context lengths,
page-id assignments (block tables), i.i.d. N(0,1) queries and keys/values, and
the per-head fp8 scales that the workload recipe fixes.  It holds none of the
attention arithmetic, no page gather/scatter and no fp8 encoding: both the HIP
path and the CPU oracle receive the same arrays from here and do that work
themselves.

Workload shapes follow the paged KV cache of "TensorRT-LLM框架解析与高性能推理优化实践"
(§4.2 KV缓存管理细节: fixed-size pages, non-contiguous physical storage, block
table per sequence; §6.2: shared-prefix reuse) and the in-flight batch of
"TensorRT-LLM内核融合与动态批处理" (In-flight Batching section: requests of mixed
lengths joining every step), with chunked context from §5.3 of the first page.

Recipe (every decision that the shapes leave open is written here):
  * streams: numpy SeedSequence(20261202 + workload id), spawned into children
    in a fixed order; each bulk draw uses its own child so that draws can run on
    a thread pool and stay deterministic;
  * lengths: fixed lists, uniform integers inclusive of both ends, or a
    lognormal ``rint(exp(ln(median) + sigma*z))`` clipped to [lo, hi];
  * page ids: one seeded permutation of the pool consumed in sequence order
    (decode sequences, then prefill requests); the pool holds
    ceil(1.25 * pages needed) pages unless the workload fixes the count;
    shared prefix pages are taken once, first;
  * values: standard normal float32; bf16 inputs are the RNE cast of those
    draws (carried as uint16 bit patterns), fp8 and int8 caches take float32
    inputs;
  * scale per KV head: float32(amax / 448) for fp8, float32(amax / 127) for
    int8, over every drawn token of that head (the workload's calibration
    recipe, an input of the method);
  * every pool byte that no token occupies is a NaN (poison) — for int8,
    which has none, the code -128 that the symmetric encoding never writes —
    so a read of an unused slot shows up in the result.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

SEED_BASE = 20261202

# Element sizes of the storage dtypes, in bytes.
DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}
# Bit patterns used to poison unused pool bytes (NaN; int8: the unused code -128).
POISON = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F),
          "int8": np.int8(-128)}
STORAGE_NP = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "int8": np.int8}
# Largest code magnitude of the 8-bit KV formats (scale = amax / this).
CODE_MAX = {"fp8": 448.0, "int8": 127.0}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------- #
# Workload specifications
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class LenDist:
    """How context lengths are drawn."""
    kind: str                      # "fixed" | "uniform" | "lognormal"
    values: Tuple[int, ...] = ()   # fixed
    lo: int = 0
    hi: int = 0
    median: float = 0.0
    sigma: float = 1.0


@dataclass(frozen=True)
class Spec:
    """One synthetic workload.  Decode sequences, optional prefill chunks."""
    wid: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: str                   # "f32" | "bf16"
    kv_dtype: str                  # "f32" | "bf16" | "fp8" | "int8"
    out_dtype: str                 # "f32" | "bf16"
    lens: LenDist
    num_pages: Optional[int] = None
    shared_prefix_pages: int = 0
    # Mixed in-flight step: decode lengths are the cache sizes before the step
    # (the step appends one token per decode sequence), and every prefill
    # request appends one chunk after ``prefill_ctx[r]`` cached tokens.
    decode_lens_are_pre_step: bool = False
    prefill_ctx: Tuple[int, ...] = ()
    prefill_chunk: int = 0
    max_len: Optional[int] = None  # block-table stride = ceil(max_len/page)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def kv_in_dtype(self) -> str:
        """Dtype of the new K/V handed to the append (8-bit caches quantize f32)."""
        return "f32" if self.kv_dtype in CODE_MAX else self.kv_dtype


# The five workloads: tiny fp32; 13B-shaped MHA bf16; 8B-shaped GQA bf16 with a
# shared prefix; 70B-shaped GQA with fp8 KV; mixed in-flight step.
C1 = Spec(1, "tiny_f32_decode", 4, 4, 4, 64, 16, "f32", "f32", "f32",
          LenDist("fixed", values=(7, 33, 64, 100)), num_pages=64, max_len=100)
C2 = Spec(2, "llama2_13b_mha_bf16_decode", 64, 40, 40, 128, 64, "bf16", "bf16", "bf16",
          LenDist("uniform", lo=128, hi=4096), max_len=4096)
C3 = Spec(3, "llama3_8b_gqa_bf16_prefix_decode", 256, 32, 8, 128, 32, "bf16", "bf16", "bf16",
          LenDist("lognormal", lo=16, hi=8192, median=512.0, sigma=1.0),
          shared_prefix_pages=4, max_len=8192)
C4 = Spec(4, "llama3_70b_gqa_fp8kv_decode", 128, 64, 8, 128, 64, "bf16", "fp8", "bf16",
          LenDist("uniform", lo=1024, hi=16384), max_len=16384)
C5 = Spec(5, "llama3_8b_gqa_bf16_mixed_step", 48, 32, 8, 128, 32, "bf16", "bf16", "bf16",
          LenDist("uniform", lo=256, hi=4096), decode_lens_are_pre_step=True,
          prefill_ctx=(0, 512, 1024, 2048), prefill_chunk=512, max_len=4097)

CONFIGS = {1: C1, 2: C2, 3: C3, 4: C4, 5: C5}


# --------------------------------------------------------------------------- #
# Generated arrays
# --------------------------------------------------------------------------- #
@dataclass
class AppendBatch:
    """New tokens to place in the cache: packed [T][Hkv][D] plus per-row metadata."""
    block_tables: np.ndarray       # int32 [n][stride]
    start_pos: np.ndarray          # int32 [n]  tokens already cached in that row
    cu: np.ndarray                 # int32 [n+1] offsets into the packed tokens
    k: np.ndarray                  # [T][Hkv][D] float32 or uint16 (bf16 bits)
    v: np.ndarray
    # Which logical token stream each row continues: ("seq", b) for decode
    # sequence b, ("pf", r) for prefill request r, ("prefix", 0) for the
    # shared prefix.  Row i holds that stream's positions start_pos[i]...
    owners: Tuple[Tuple[str, int], ...] = ()

    @property
    def num_tokens(self) -> int:
        return int(self.cu[-1])

    @property
    def num_rows(self) -> int:
        return int(self.start_pos.shape[0])


@dataclass
class Workload:
    spec: Spec
    seed: int
    num_pages: int
    sm_scale: np.float32
    # Decode part (may have zero sequences).
    context_lens: np.ndarray       # int32 [B]  tokens attended by each decode query
    block_tables: np.ndarray       # int32 [B][stride]
    q: np.ndarray                  # [B][Hq][D] float32 or uint16 (bf16 bits)
    # Cache contents: `setup` fills the pool before the step, `step` is appended
    # inside the step (one token per decode sequence plus the prefill chunks).
    setup: AppendBatch
    step: AppendBatch
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray] = None
    # Prefill part (mixed step only).
    pf_q: Optional[np.ndarray] = None      # [Tq][Hq][D]
    pf_cu: Optional[np.ndarray] = None     # int32 [R+1]
    pf_ctx_before: Optional[np.ndarray] = None  # int32 [R]
    pf_block_tables: Optional[np.ndarray] = None  # int32 [R][stride]
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_prefill(self) -> int:
        return 0 if self.pf_cu is None else int(self.pf_cu.shape[0] - 1)

    def poisoned_pool(self) -> Tuple[np.ndarray, np.ndarray]:
        """Fresh K and V pools [num_pages][Hkv][P][D] filled with NaN poison."""
        s = self.spec
        shape = (self.num_pages, s.num_kv_heads, s.page_size, s.head_dim)
        dt = s.kv_dtype
        if dt == "f32":
            k = np.full(shape, POISON["f32"], dtype=np.uint32).view(np.float32)
            v = np.full(shape, POISON["f32"], dtype=np.uint32).view(np.float32)
        else:
            k = np.full(shape, POISON[dt], dtype=STORAGE_NP[dt])
            v = np.full(shape, POISON[dt], dtype=STORAGE_NP[dt])
        return k, v


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (input preparation)."""
    import torch  # torch CPU cast is the RNE reference for bf16 inputs
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw_lens(spec: Spec, n: int, rng: np.random.Generator) -> np.ndarray:
    d = spec.lens
    if d.kind == "fixed":
        assert len(d.values) == n
        return np.asarray(d.values, dtype=np.int64)
    if d.kind == "uniform":
        return rng.integers(d.lo, d.hi, size=n, endpoint=True).astype(np.int64)
    if d.kind == "lognormal":
        z = rng.standard_normal(n)
        v = np.rint(np.exp(math.log(d.median) + d.sigma * z))
        return np.clip(v, d.lo, d.hi).astype(np.int64)
    raise ValueError(d.kind)


class _Filler:
    """Draws N(0,1) float32 blocks on a thread pool, one child stream per block."""

    def __init__(self, seq: np.random.SeedSequence, n_blocks: int):
        self.children = seq.spawn(max(1, n_blocks))
        self.jobs: List[Tuple[int, np.ndarray]] = []

    def add(self, idx: int, out: np.ndarray) -> None:
        self.jobs.append((idx, out))

    def run(self) -> None:
        def work(job):
            idx, out = job
            g = np.random.Generator(np.random.PCG64(self.children[idx]))
            g.standard_normal(out=out.reshape(-1), dtype=np.float32)

        if len(self.jobs) <= 1:
            for j in self.jobs:
                work(j)
        else:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(work, self.jobs))


def make_workload(spec: Spec, seed: Optional[int] = None) -> Workload:
    """Build the seeded workload for ``spec``.

    Decode sequences come first.  For each, the logical K/V rows 0..L-1 are
    drawn; the last row is the step's own token and goes into ``step`` (unless
    it lies inside a shared prefix, which is written once by ``setup``).
    """
    if seed is None:
        seed = SEED_BASE + spec.wid
    ss = np.random.SeedSequence(seed)
    s_lens, s_perm, s_q, s_kv, s_pf = ss.spawn(5)
    rng_lens = np.random.Generator(np.random.PCG64(s_lens))

    B, Hq, Hkv, D, P = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    assert Hq % Hkv == 0
    pre = _draw_lens(spec, B, rng_lens) if B > 0 else np.zeros(0, np.int64)
    ctx = pre + 1 if spec.decode_lens_are_pre_step else pre
    npre = spec.shared_prefix_pages
    prefix_tokens = npre * P

    R = len(spec.prefill_ctx)
    pf_total = [c + spec.prefill_chunk for c in spec.prefill_ctx]

    max_len = spec.max_len or int(max([*ctx.tolist(), *pf_total, 1]))
    stride = max(1, -(-max_len // P), npre)       # every row lists the whole prefix

    # ---- page ids -------------------------------------------------------
    def own_pages(L: int) -> int:
        return -(-max(0, L - prefix_tokens) // P)

    need = npre + sum(own_pages(int(L)) for L in ctx) + sum(-(-t // P) for t in pf_total)
    num_pages = spec.num_pages or max(1, math.ceil(1.25 * need))
    assert need <= num_pages, "pool too small"
    perm = np.random.Generator(np.random.PCG64(s_perm)).permutation(num_pages).astype(np.int32)
    cursor = 0

    def take(n: int) -> np.ndarray:
        nonlocal cursor
        ids = perm[cursor:cursor + n]
        cursor += n
        return ids

    prefix_ids = take(npre)
    bt = np.full((B, stride), -1, dtype=np.int32)
    for b in range(B):
        ids = np.concatenate([prefix_ids, take(own_pages(int(ctx[b])))])
        bt[b, :ids.size] = ids
    pf_bt = np.full((R, stride), -1, dtype=np.int32)
    for r in range(R):
        ids = take(-(-pf_total[r] // P))
        pf_bt[r, :ids.size] = ids

    # ---- decode queries -------------------------------------------------
    q32 = np.empty((B, Hq, D), dtype=np.float32)
    fq = _Filler(s_q, 1)
    fq.add(0, q32)
    fq.run()

    # ---- logical K/V and the two append batches -------------------------
    # Setup rows: [shared prefix], decode seq b (tokens [own_start, L-1) ),
    # prefill request r (its P_r cached tokens).  Step rows: decode seq b
    # (token L-1 when outside the prefix), prefill request r (its chunk).
    setup_rows, step_rows = [], []   # (bt_row, start, count, src, src_off)
    # sources: ("prefix", 0) | ("seq", b) | ("pf", r)
    if npre:
        setup_rows.append((np.concatenate([prefix_ids, np.full(stride - npre, -1, np.int32)]),
                           0, prefix_tokens, ("prefix", 0), 0))
    for b in range(B):
        L = int(ctx[b])
        own_start = prefix_tokens if npre else 0
        if L > own_start:
            if L - 1 > own_start:
                setup_rows.append((bt[b], own_start, L - 1 - own_start, ("seq", b), 0))
            step_rows.append((bt[b], L - 1, 1, ("seq", b), L - 1 - own_start))
    for r in range(R):
        c0 = spec.prefill_ctx[r]
        if c0 > 0:
            setup_rows.append((pf_bt[r], 0, c0, ("pf", r), 0))
        step_rows.append((pf_bt[r], c0, spec.prefill_chunk, ("pf", r), c0))

    # Per-source logical draws, each from its own child stream.
    sources = []
    if npre:
        sources.append((("prefix", 0), prefix_tokens))
    for b in range(B):
        L = int(ctx[b])
        own = L - (prefix_tokens if npre else 0)
        if own > 0:
            sources.append((("seq", b), own))
    for r in range(R):
        sources.append((("pf", r), pf_total[r]))
    fkv = _Filler(s_kv, 2 * len(sources))
    logical_k, logical_v = {}, {}
    for i, (key, n) in enumerate(sources):
        logical_k[key] = np.empty((n, Hkv, D), np.float32)
        logical_v[key] = np.empty((n, Hkv, D), np.float32)
        fkv.add(2 * i, logical_k[key])
        fkv.add(2 * i + 1, logical_v[key])
    fkv.run()

    k_scale = v_scale = None
    if spec.kv_dtype in CODE_MAX:
        ka = np.zeros(Hkv, np.float32)
        va = np.zeros(Hkv, np.float32)
        for key in logical_k:
            if logical_k[key].shape[0]:
                ka = np.maximum(ka, np.abs(logical_k[key]).max(axis=(0, 2)))
                va = np.maximum(va, np.abs(logical_v[key]).max(axis=(0, 2)))
        cmax = np.float32(CODE_MAX[spec.kv_dtype])
        k_scale = (ka / cmax).astype(np.float32)
        v_scale = (va / cmax).astype(np.float32)

    def build(rows) -> AppendBatch:
        n = len(rows)
        cu = np.zeros(n + 1, np.int32)
        for i, row in enumerate(rows):
            cu[i + 1] = cu[i] + row[2]
        T = int(cu[-1])
        k = np.empty((T, Hkv, D), np.float32)
        v = np.empty((T, Hkv, D), np.float32)
        for i, (_, start, cnt, key, off) in enumerate(rows):
            k[cu[i]:cu[i + 1]] = logical_k[key][off:off + cnt]
            v[cu[i]:cu[i + 1]] = logical_v[key][off:off + cnt]
        if spec.kv_in_dtype == "bf16":
            k, v = bf16_bits_rne(k), bf16_bits_rne(v)
        btr = np.stack([r[0] for r in rows]) if n else np.zeros((0, stride), np.int32)
        return AppendBatch(block_tables=np.ascontiguousarray(btr, dtype=np.int32),
                           start_pos=np.array([r[1] for r in rows], dtype=np.int32),
                           cu=cu, k=k, v=v, owners=tuple(r[3] for r in rows))

    setup = build(setup_rows)
    step = build(step_rows)
    del logical_k, logical_v

    q = bf16_bits_rne(q32) if spec.q_dtype == "bf16" else q32

    wl = Workload(spec=spec, seed=seed, num_pages=num_pages,
                  sm_scale=np.float32(1.0 / math.sqrt(D)),
                  context_lens=ctx.astype(np.int32), block_tables=bt, q=q,
                  setup=setup, step=step, k_scale=k_scale, v_scale=v_scale)

    if R:
        C = spec.prefill_chunk
        pq = np.empty((R * C, Hq, D), np.float32)
        fp = _Filler(s_pf, 1)
        fp.add(0, pq)
        fp.run()
        wl.pf_q = bf16_bits_rne(pq) if spec.q_dtype == "bf16" else pq
        wl.pf_cu = (np.arange(R + 1, dtype=np.int32) * C).astype(np.int32)
        wl.pf_ctx_before = np.asarray(spec.prefill_ctx, dtype=np.int32)
        wl.pf_block_tables = pf_bt
    return wl


def logical_kv(wl: Workload, kind: str, idx: int, length: int) -> Tuple[np.ndarray, np.ndarray]:
    """The K/V rows of positions 0..length-1 of one token stream, as drawn.

    Reassembled from the two append batches (shared-prefix rows count for
    every decode sequence); used to check pages against unpaged data."""
    spec = wl.spec
    k = np.empty((length, spec.num_kv_heads, spec.head_dim), wl.setup.k.dtype)
    v = np.empty_like(k)
    filled = np.zeros(length, bool)
    for batch in (wl.setup, wl.step):
        for i, own in enumerate(batch.owners):
            if own == (kind, idx) or (kind == "seq" and own[0] == "prefix"):
                s0 = int(batch.start_pos[i])
                n = int(batch.cu[i + 1] - batch.cu[i])
                hi = min(length, s0 + n)
                if hi > s0:
                    k[s0:hi] = batch.k[batch.cu[i]:batch.cu[i] + hi - s0]
                    v[s0:hi] = batch.v[batch.cu[i]:batch.cu[i] + hi - s0]
                    filled[s0:hi] = True
    assert filled.all(), "stream not fully drawn"
    return k, v


def decode_step_tokens(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """The step's decode tokens as one row per sequence, [B][Hkv][D] in the
    input dtype: row b is the step-batch token that goes to position L_b - 1
    of sequence b (zero rows for empty sequences).  Raises ValueError when a
    non-empty sequence has no token of its own in the step (its last
    position lies in a shared prefix)."""
    st, s = wl.step, wl.spec
    k = np.zeros((wl.num_seqs, s.num_kv_heads, s.head_dim), st.k.dtype)
    v = np.zeros_like(k)
    have = np.zeros(wl.num_seqs, bool)
    for i, o in enumerate(st.owners):
        if o[0] != "seq":
            continue
        b = o[1]
        if st.cu[i + 1] - st.cu[i] != 1 or st.start_pos[i] != wl.context_lens[b] - 1:
            raise ValueError(f"step row {i} is not sequence {b}'s last token")
        k[b], v[b], have[b] = st.k[st.cu[i]], st.v[st.cu[i]], True
    if not np.array_equal(have, wl.context_lens > 0):
        raise ValueError("some sequences end inside a shared prefix: no token of their own")
    return k, v


def custom_spec(lens: Sequence[int], *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                page_size: int, q_dtype: str = "bf16", kv_dtype: str = "bf16",
                out_dtype: Optional[str] = None, shared_prefix_pages: int = 0,
                prefill_ctx: Sequence[int] = (), prefill_chunk: int = 0,
                num_pages: Optional[int] = None, wid: int = 100,
                max_len: Optional[int] = None) -> Spec:
    """A workload with explicit decode lengths (edge cases, small parity runs)."""
    return Spec(wid, "custom", len(lens), num_q_heads, num_kv_heads, head_dim, page_size,
                q_dtype, kv_dtype, out_dtype or q_dtype,
                LenDist("fixed", values=tuple(int(x) for x in lens)),
                num_pages=num_pages, shared_prefix_pages=shared_prefix_pages,
                prefill_ctx=tuple(prefill_ctx), prefill_chunk=prefill_chunk, max_len=max_len)


def decode_bytes(spec: Spec, context_lens: np.ndarray, unique_prefix: bool = True) -> int:
    """Algorithmic HBM bytes of one decode attention pass.

    K and V of every attended token once (shared prefix pages once when
    ``unique_prefix``), Q read, O written, block-table entries and lengths,
    fp8 scales.
    """
    e_kv = DTYPE_BYTES[spec.kv_dtype]
    row = spec.num_kv_heads * spec.head_dim * e_kv * 2
    L = context_lens.astype(np.int64)
    tok = int(L.sum())
    if unique_prefix and spec.shared_prefix_pages:
        pt = spec.shared_prefix_pages * spec.page_size
        tok = int(np.maximum(L - pt, 0).sum()) + int(min(pt, int(L.max()) if L.size else 0))
    B = int(L.shape[0])
    qo = B * spec.num_q_heads * spec.head_dim * (DTYPE_BYTES[spec.q_dtype] + DTYPE_BYTES[spec.out_dtype])
    bt = 4 * (B + int((-(-L // spec.page_size)).sum()))
    sc = 8 * spec.num_kv_heads if spec.kv_dtype in CODE_MAX else 0
    return tok * row + qo + bt + sc


def prefill_flops(spec: Spec, ctx_before: np.ndarray, cu: np.ndarray) -> int:
    """Algorithmic FLOPs of causal chunked prefill: 4*Hq*D per (query, key) pair."""
    pairs = 0
    for r in range(ctx_before.shape[0]):
        P = int(ctx_before[r])
        C = int(cu[r + 1] - cu[r])
        pairs += C * P + C * (C + 1) // 2
    return 4 * spec.num_q_heads * spec.head_dim * pairs


def request_tensors(seed: int, req_id: int, length: int, num_q_heads: int, num_kv_heads: int,
                    head_dim: int):
    """Seeded per-request token data for scheduler-driven runs: q [length][Hq][D]
    and k, v [length][Hkv][D] as bf16 bits, standard normal, drawn from
    SeedSequence((seed, req_id)) so a request recomputed after eviction sees
    the same tokens again."""
    rng = np.random.default_rng(np.random.SeedSequence((seed, req_id)))
    q = rng.standard_normal((length, num_q_heads, head_dim), dtype=np.float32)
    k = rng.standard_normal((length, num_kv_heads, head_dim), dtype=np.float32)
    v = rng.standard_normal((length, num_kv_heads, head_dim), dtype=np.float32)
    return bf16_bits_rne(q), bf16_bits_rne(k), bf16_bits_rne(v)


def variant(name: str) -> Spec:
    """A workload of CONFIGS with another KV format: "<id>-int8" or "<id>-fp8"
    (same shapes, lengths and seed stream; the scales follow the format)."""
    import dataclasses
    wid, kv = name.split("-")
    base = CONFIGS[int(wid)]
    tag = {"int8": "int8kv", "fp8": "fp8kv"}[kv]
    stem = base.name.replace("_fp8kv", "").replace("_bf16", "")
    return dataclasses.replace(base, kv_dtype=kv, name=f"{stem}_{tag}")

