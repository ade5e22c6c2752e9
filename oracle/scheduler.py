"""Step scheduling with a paged KV cache, written out plainly (test infrastructure
only: the library's scheduler is checked against it; nothing in the product
imports it).

Sources ("TensorRT-LLM框架解析与高性能推理优化实践"): §4.2 the KV-cache manager
gives each sequence a list of pages, allocated on demand and freed when it
leaves, prefix pages shared; §5.1 capacity scheduling in a conservative mode
(running requests are guaranteed to finish) or an aggressive one; §5.2 LIFO
preemption — while a request lacks pages, evict the most recently admitted
running request and put it back at the front of the waiting queue, out of
memory when nothing is left to evict; §5.3 long prompts in chunks interleaved
with decodes; §4.1 one compute slot per running request.

Readings where the pages leave a step open (the library follows the same):
  * eviction is triggered only by the growth of running requests; admission
    never evicts and never skips the queue front;
  * conservative admission reserves the worst case of every running request
    and of the new one (prompt + max_new - 1 cached tokens), aggressive
    admission only the pages of the new request's next chunk;
  * an evicted request loses its cached K/V and is recomputed from its
    (shared) prefix when resumed;
  * a running request holds the lowest free slot.

Pages are counted, not named: which page ids a request gets is the
allocator's business and is checked for validity separately.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

PREFILL, DECODE = 0, 1


def pages_for(tokens: int, page_size: int) -> int:
    return -(-tokens // page_size)


@dataclass
class Req:
    rid: int
    prompt: int
    max_new: int
    prefix: Optional[int] = None
    prefix_tokens: int = 0
    generated: int = 0
    num_tokens: int = 0
    computed: int = 0
    pages: int = 0            # pages held, prefix pages included
    slot: int = -1


@dataclass
class OracleScheduler:
    num_pages: int
    page_size: int
    max_batch: int
    max_tokens: int
    chunk: int
    conservative: bool
    free: int = 0
    waiting: List[Req] = field(default_factory=list)     # index 0 = front
    running: List[Req] = field(default_factory=list)     # admission order
    reqs: Dict[int, Req] = field(default_factory=dict)
    prefixes: Dict[int, int] = field(default_factory=dict)   # id -> tokens
    slots: List[bool] = field(default_factory=list)
    plan: List[Tuple[int, int, int, int, int]] = field(default_factory=list)
    preemptions: int = 0

    def __post_init__(self):
        self.free = self.num_pages
        self.slots = [False] * self.max_batch

    # -- the request's page needs -----------------------------------------------
    def worst_own_pages(self, r: Req) -> int:
        last = r.prompt + r.max_new - 1            # the final token is never cached
        return pages_for(last, self.page_size) - pages_for(r.prefix_tokens, self.page_size)

    def add_prefix(self, pid: int, tokens: int) -> None:
        assert tokens > 0 and tokens % self.page_size == 0 and pid not in self.prefixes
        n = tokens // self.page_size
        assert n <= self.free
        self.free -= n
        self.prefixes[pid] = tokens

    def add_request(self, rid: int, prompt: int, max_new: int, prefix: Optional[int] = None) -> bool:
        """False when the request could never fit (refused)."""
        r = Req(rid, prompt, max_new, prefix, self.prefixes[prefix] if prefix is not None else 0,
                num_tokens=prompt)
        pinned = sum(t // self.page_size for t in self.prefixes.values())
        if self.worst_own_pages(r) + pinned > self.num_pages:
            return False
        self.reqs[rid] = r
        self.waiting.append(r)
        return True

    # -- eviction and admission ---------------------------------------------------
    def _release(self, r: Req) -> None:
        # shared prefix pages stay with the prefix; the request's own go back
        own = r.pages - (r.prefix_tokens // self.page_size if r.pages else 0)
        self.free += own
        r.pages = 0
        if r.slot >= 0:
            self.slots[r.slot] = False
        r.slot = -1

    def _evict(self, v: Req, evicted: List[int]) -> None:
        self._release(v)
        v.computed = 0
        self.running.remove(v)
        self.waiting.insert(0, v)
        evicted.append(v.rid)
        self.preemptions += 1

    def _tokens_this_step(self, r: Req, budget: int) -> int:
        pending = r.num_tokens - r.computed
        n = min(self.chunk, pending) if pending > 1 else 1
        return min(n, budget)

    def schedule(self) -> Tuple[List[Tuple[int, int, int, int, int]], List[int]]:
        """One step: [(rid, slot, kind, start_pos, n)], [evicted rids]."""
        plan, evicted = [], []
        budget = self.max_tokens
        i = 0
        while i < len(self.running) and budget > 0:
            r = self.running[i]
            n = self._tokens_this_step(r, budget)
            need = max(0, pages_for(r.computed + n, self.page_size) - r.pages)
            gone = False
            while self.free < need:
                v = self.running[-1]                 # most recently admitted
                self._evict(v, evicted)
                if v is r:
                    gone = True
                    break
            if gone:
                break
            self.free -= need
            r.pages += need
            kind = PREFILL if r.num_tokens - r.computed > 1 else DECODE
            plan.append((r.rid, r.slot, kind, r.computed, n))
            budget -= n
            i += 1
        while self.waiting and budget > 0 and len(self.running) < self.max_batch:
            r = self.waiting[0]
            start = r.prefix_tokens
            pending = r.num_tokens - start
            n = min(min(self.chunk, pending) if pending > 1 else 1, budget)
            first = pages_for(start + n, self.page_size) - pages_for(start, self.page_size)
            if self.conservative:
                need = self.worst_own_pages(r)
                for q in self.running:
                    need += pages_for(q.prompt + q.max_new - 1, self.page_size) - q.pages
            else:
                need = first
            if self.free < need:
                break
            self.waiting.pop(0)
            r.computed = start
            r.pages = start // self.page_size + first
            self.free -= first
            r.slot = self.slots.index(False)
            self.slots[r.slot] = True
            self.running.append(r)
            kind = PREFILL if r.num_tokens - r.computed > 1 else DECODE
            plan.append((r.rid, r.slot, kind, r.computed, n))
            budget -= n
        self.plan = plan
        return plan, evicted

    def commit(self) -> List[int]:
        finished = []
        for rid, _slot, _kind, _start, n in self.plan:
            r = self.reqs[rid]
            r.computed += n
            if r.computed == r.num_tokens:
                r.generated += 1
                r.num_tokens += 1
                if r.generated == r.max_new:
                    self._release(r)
                    self.running.remove(r)
                    del self.reqs[rid]
                    finished.append(rid)
        self.plan = []
        return finished

    def finish(self, rid: int) -> None:
        r = self.reqs.pop(rid)
        self._release(r)
        if r in self.running:
            self.running.remove(r)
        if r in self.waiting:
            self.waiting.remove(r)
