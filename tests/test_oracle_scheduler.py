"""Pins for the scheduling oracle (oracle/scheduler.py): small traces whose
every step is worked out by hand from the rules of
"TensorRT-LLM框架解析与高性能推理优化实践" §5.1-§5.3 (capacity scheduling, LIFO
preemption, chunked context) and §4.2 (pages on demand, shared prefixes).
Items are (request, slot, kind, start_pos, tokens); kind 0 = prefill chunk,
1 = decode."""
from oracle.scheduler import DECODE as D
from oracle.scheduler import PREFILL as P
from oracle.scheduler import OracleScheduler


def make(num_pages, page=4, batch=4, budget=100, chunk=100, conservative=False):
    return OracleScheduler(num_pages, page, batch, budget, chunk, conservative)


def test_lifo_evicts_the_most_recent_and_requeues_it_first():
    s = make(6)
    assert s.add_request(1, 8, 10) and s.add_request(2, 8, 10) and s.add_request(3, 4, 10)
    # step 1: all three fit (2 + 2 + 1 pages of 6)
    assert s.schedule() == ([(1, 0, P, 0, 8), (2, 1, P, 0, 8), (3, 2, P, 0, 4)], [])
    assert s.commit() == [] and s.free == 1
    # step 2: request 1 takes the last page for its 9th token; request 2 needs
    # one more, so request 3 (admitted last) is evicted and waits at the front
    assert s.schedule() == ([(1, 0, D, 8, 1), (2, 1, D, 8, 1)], [3])
    s.commit()
    assert [r.rid for r in s.waiting] == [3] and s.reqs[3].computed == 0
    # steps 3-5: decodes within the held pages; request 3 (needs 2 pages) waits
    for start in (9, 10, 11):
        assert s.schedule() == ([(1, 0, D, start, 1), (2, 1, D, start, 1)], [])
        s.commit()
    # step 6: request 1's 13th token needs a 4th page: request 2 is now the
    # newest running request and is evicted, going ahead of request 3
    assert s.schedule() == ([(1, 0, D, 12, 1)], [2])
    assert [r.rid for r in s.waiting] == [2, 3]
    assert s.preemptions == 2


def test_newest_request_evicts_itself_and_is_recomputed_on_resume():
    s = make(3)
    assert s.add_request(1, 6, 3) and s.add_request(2, 4, 3)
    assert s.schedule() == ([(1, 0, P, 0, 6), (2, 1, P, 0, 4)], [])
    s.commit()
    # request 2 (the newest) needs a second page for its 5th token: none free,
    # nothing newer to evict -> it evicts itself; it cannot come back yet
    assert s.schedule() == ([(1, 0, D, 6, 1)], [2])
    s.commit()
    assert s.schedule() == ([(1, 0, D, 7, 1)], [])
    assert s.commit() == [1]                       # 3 tokens generated
    # resumed into the freed slot 0: prompt (4) + 1 generated token recomputed
    assert s.schedule() == ([(2, 0, P, 0, 5)], [])
    s.commit()
    assert s.schedule() == ([(2, 0, D, 5, 1)], [])
    assert s.commit() == [2]
    assert s.free == 3


def test_conservative_reserves_worst_cases_and_never_evicts():
    s = make(6, conservative=True)
    assert s.add_request(1, 8, 10) and s.add_request(2, 8, 10)
    # request 1 reserves 5 pages (8 + 10 - 1 = 17 tokens); request 2 would
    # need its own 5 plus request 1's remaining 3 > 4 free
    assert s.schedule() == ([(1, 0, P, 0, 8)], [])
    steps = 1
    while s.reqs or s.waiting:
        s.commit()
        s.schedule()
        steps += 1
        assert steps < 100
    assert s.preemptions == 0 and s.free == 6


def test_long_prompt_in_chunks_interleaved_with_decodes():
    s = make(100, chunk=4)
    assert s.add_request(1, 10, 3) and s.add_request(2, 2, 4)
    assert s.schedule() == ([(1, 0, P, 0, 4), (2, 1, P, 0, 2)], [])
    s.commit()
    assert s.schedule() == ([(1, 0, P, 4, 4), (2, 1, D, 2, 1)], [])
    s.commit()
    assert s.schedule() == ([(1, 0, P, 8, 2), (2, 1, D, 3, 1)], [])
    s.commit()
    assert s.schedule() == ([(1, 0, D, 10, 1), (2, 1, D, 4, 1)], [])
    assert s.commit() == [2]
    assert s.schedule() == ([(1, 0, D, 11, 1)], [])
    assert s.commit() == [1]


def test_token_budget_splits_prefill_and_delays_admission():
    s = make(100, budget=5)
    assert s.add_request(1, 8, 2) and s.add_request(2, 8, 2)
    assert s.schedule() == ([(1, 0, P, 0, 5)], [])
    s.commit()
    assert s.schedule() == ([(1, 0, P, 5, 3), (2, 1, P, 0, 2)], [])
    s.commit()
    assert s.schedule() == ([(1, 0, D, 8, 1), (2, 1, P, 2, 4)], [])
    assert s.commit() == [1]
    assert s.schedule() == ([(2, 1, P, 6, 2)], [])
    s.commit()
    assert s.schedule() == ([(2, 1, D, 8, 1)], [])
    assert s.commit() == [2]


def test_requests_that_can_never_fit_are_refused():
    s = make(4)
    assert not s.add_request(1, 10, 8)            # 17 cached tokens -> 5 pages > 4
    assert s.add_request(2, 10, 7)                # 16 tokens -> 4 pages
    # a pinned prefix reduces what any request may use
    s2 = make(4)
    s2.add_prefix(9, 8)                           # 2 pages pinned
    assert not s2.add_request(3, 12, 6, prefix=9)  # 17 tokens: 5 pages, 3 own + 2 pinned > 4
    assert s2.add_request(4, 12, 5, prefix=9)      # 16 tokens: 4 pages, 2 own + 2 pinned
    assert not s2.add_request(5, 8, 2)             # 9 tokens: 3 own + 2 pinned > 4


def test_shared_prefix_pages_start_cached():
    s = make(10)
    s.add_prefix(7, 8)                            # 2 pages
    assert s.free == 8
    assert s.add_request(1, 10, 2, prefix=7) and s.add_request(2, 13, 2, prefix=7)
    # both start with 8 cached tokens; only their own pages are allocated
    assert s.schedule() == ([(1, 0, P, 8, 2), (2, 1, P, 8, 5)], [])
    assert s.free == 8 - 1 - 2
    s.commit()
    assert s.schedule() == ([(1, 0, D, 10, 1), (2, 1, D, 13, 1)], [])
    assert s.commit() == [1, 2]
    assert s.free == 8                            # the prefix stays pinned
