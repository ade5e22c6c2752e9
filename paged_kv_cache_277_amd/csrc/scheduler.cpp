// Host KV-cache manager and step scheduler for in-flight batching.
//
// What it does ("TensorRT-LLM框架解析与高性能推理优化实践"):
//   §4.2  KVCacheManager: each sequence owns a list of cache pages (its block
//         table), pages are allocated on demand and freed when it leaves;
//         pages of a shared prompt prefix are reused by reference.
//   §5.1  CapacityScheduler admits requests by remaining KV capacity, in a
//         conservative mode (running requests are guaranteed to finish) or
//         an aggressive one (more requests in flight, preemption when pages
//         run out); the micro-batch side mixes new (prefill), generating
//         (decode) and long-context (chunked) requests in one step.
//   §5.2  LIFO preemption: while a request lacks pages, the most recently
//         admitted running request is evicted — its pages freed, the request
//         put back at the front of the waiting queue; with nothing left to
//         evict the request cannot run (out of memory).
//   §5.3  Long prompts are computed in chunks interleaved with decode steps.
//   §4.1  SequenceSlotManager: each running request holds a compute slot.
//
// Readings (where the pages leave a step open):
//   * Eviction is triggered by the growth of running requests (next decode
//     token or prefill chunk).  Admission from the waiting queue never
//     evicts: an arrival that evicts a running request which then, re-queued
//     at the front, evicts the arrival on the next step would alternate
//     forever.  Admission is first-come first-served (the queue front waits
//     until it fits).
//   * Conservative admission reserves every running request's worst case
//     (prompt + max_new_tokens - 1 cached tokens) so growth never runs out
//     and nothing is evicted; aggressive admission needs only the pages of
//     the request's next chunk.
//   * An evicted request is recomputed from its prefix on resume (its pages
//     were freed): its prompt and the tokens generated so far are prefilled
//     again in chunks.
//
// Token accounting per request: num_tokens = prompt + generated tokens;
// num_computed = tokens whose K/V are in the cache.  A step computes
// n = min(chunk_size, pending, budget) tokens of a request with pending =
// num_tokens - num_computed > 1 (a prefill chunk), or its one pending token
// (a decode).  Commit adds n to num_computed; when the cache has caught up
// with num_tokens the model has produced one more token (generated + 1); at
// max_new_tokens the request finishes and its pages are freed.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace pkv_detail {
void set_error(const std::string& s);
}

namespace {

struct Request {
  int64_t id;
  int32_t prompt_len, max_new, generated = 0;
  int32_t num_tokens, num_computed = 0;
  int64_t prefix_id = -1;
  int32_t prefix_tokens = 0;
  int32_t slot = -1;
  std::vector<int32_t> pages;          // block table (prefix pages first)
};

struct Prefix {
  int32_t tokens;
  std::vector<int32_t> pages;
  int32_t users = 0;                   // requests (waiting or running) referencing it
};

struct Scheduler {
  std::mutex mu;
  pkv_sched_config cfg;
  void* alloc = nullptr;
  std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
  std::deque<Request*> waiting;        // front = next to admit
  std::vector<Request*> running;       // admission order (back = newest)
  std::vector<uint8_t> slot_used;
  std::unordered_map<int64_t, Prefix> prefixes;
  std::vector<pkv_sched_item> plan;    // scheduled, not yet committed
  bool planned = false;
  int64_t preemptions = 0;

  ~Scheduler() { if (alloc) pkv_allocator_destroy(alloc); }

  int32_t pages_for(int64_t tokens) const {
    return (int32_t)((tokens + cfg.page_size - 1) / cfg.page_size);
  }
  // Cached tokens at the request's end: the last generated token is never computed.
  int32_t max_cached(const Request& r) const { return r.prompt_len + r.max_new - 1; }
  int32_t worst_private_pages(const Request& r) const {
    return pages_for(max_cached(r)) - pages_for(r.prefix_tokens);
  }
  int32_t free_pages() const { return pkv_num_free_pages(alloc); }

  void release_pages(Request& r) {
    if (!r.pages.empty()) pkv_free_pages(alloc, (int32_t)r.pages.size(), r.pages.data());
    r.pages.clear();
  }
  void take_slot(Request& r) {
    for (size_t i = 0; i < slot_used.size(); ++i)
      if (!slot_used[i]) { slot_used[i] = 1; r.slot = (int32_t)i; return; }
  }
  void drop_slot(Request& r) {
    if (r.slot >= 0) slot_used[r.slot] = 0;
    r.slot = -1;
  }
  // Pages the request holds on (re)admission: the shared prefix, if any.
  void attach_prefix(Request& r) {
    if (r.prefix_id < 0) return;
    const Prefix& p = prefixes.at(r.prefix_id);
    pkv_share_pages(alloc, (int32_t)p.pages.size(), p.pages.data());
    r.pages = p.pages;
    r.num_computed = p.tokens;
  }
  void evict(Request* v, std::vector<int64_t>& evicted) {
    release_pages(*v);
    drop_slot(*v);
    v->num_computed = 0;
    running.erase(std::find(running.begin(), running.end(), v));
    waiting.push_front(v);
    evicted.push_back(v->id);
    ++preemptions;
  }
  // Tokens the request would compute this step within `budget`.
  int32_t step_tokens(const Request& r, int32_t budget) const {
    const int32_t pending = r.num_tokens - r.num_computed;
    const int32_t n = pending > 1 ? std::min(cfg.chunk_size, pending) : 1;
    return std::min(n, budget);
  }
  int32_t extra_pages(const Request& r, int32_t n) const {
    return std::max(0, pages_for((int64_t)r.num_computed + n) - (int32_t)r.pages.size());
  }
  bool grow(Request& r, int32_t need) {
    if (need == 0) return true;
    std::vector<int32_t> ids(need);
    if (pkv_alloc_pages(alloc, need, ids.data()) != PKV_OK) return false;
    r.pages.insert(r.pages.end(), ids.begin(), ids.end());
    return true;
  }
};

pkv_status err(pkv_status st, const std::string& m) {
  pkv_detail::set_error(m);
  return st;
}

}  // namespace

extern "C" {

pkv_status pkv_sched_create(const pkv_sched_config* cfg, void** out) {
  if (!out) return err(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg) return err(PKV_ERR_INVALID_ARG, "config is NULL");
  if (cfg->num_pages <= 0 || cfg->page_size <= 0 || cfg->max_batch_size <= 0 ||
      cfg->max_num_tokens <= 0 || cfg->chunk_size <= 0)
    return err(PKV_ERR_INVALID_ARG, "scheduler sizes must be positive");
  if (cfg->policy != PKV_SCHED_CONSERVATIVE && cfg->policy != PKV_SCHED_AGGRESSIVE)
    return err(PKV_ERR_INVALID_ARG, "unknown policy " + std::to_string(cfg->policy));
  std::unique_ptr<Scheduler> s(new (std::nothrow) Scheduler);
  if (!s) return err(PKV_ERR_INVALID_ARG, "out of host memory");
  s->cfg = *cfg;
  pkv_status st = pkv_allocator_create(cfg->num_pages, &s->alloc);
  if (st != PKV_OK) return st;
  s->slot_used.assign(cfg->max_batch_size, 0);
  *out = s.release();
  return PKV_OK;
}

void pkv_sched_destroy(void* sched) { delete static_cast<Scheduler*>(sched); }

pkv_status pkv_sched_add_prefix(void* sched, int64_t prefix_id, int32_t num_tokens,
                                int32_t* out_pages) {
  Scheduler* s = static_cast<Scheduler*>(sched);
  if (!s || !out_pages) return err(PKV_ERR_INVALID_ARG, "NULL scheduler or out_pages");
  std::lock_guard<std::mutex> lk(s->mu);
  if (prefix_id < 0 || s->prefixes.count(prefix_id))
    return err(PKV_ERR_INVALID_ARG, "prefix id " + std::to_string(prefix_id) + " invalid or taken");
  if (num_tokens <= 0 || num_tokens % s->cfg.page_size != 0)
    return err(PKV_ERR_INVALID_ARG, "a shared prefix covers whole pages (" +
                                    std::to_string(num_tokens) + " tokens)");
  Prefix p;
  p.tokens = num_tokens;
  p.pages.resize(num_tokens / s->cfg.page_size);
  pkv_status st = pkv_alloc_pages(s->alloc, (int32_t)p.pages.size(), p.pages.data());
  if (st != PKV_OK) return st;
  std::copy(p.pages.begin(), p.pages.end(), out_pages);
  s->prefixes.emplace(prefix_id, std::move(p));
  return PKV_OK;
}

pkv_status pkv_sched_remove_prefix(void* sched, int64_t prefix_id) {
  Scheduler* s = static_cast<Scheduler*>(sched);
  if (!s) return err(PKV_ERR_INVALID_ARG, "NULL scheduler");
  std::lock_guard<std::mutex> lk(s->mu);
  auto it = s->prefixes.find(prefix_id);
  if (it == s->prefixes.end()) return err(PKV_ERR_INVALID_ARG, "unknown prefix");
  if (it->second.users > 0)
    return err(PKV_ERR_INVALID_ARG, "prefix still referenced by " +
                                    std::to_string(it->second.users) + " request(s)");
  pkv_free_pages(s->alloc, (int32_t)it->second.pages.size(), it->second.pages.data());
  s->prefixes.erase(it);
  return PKV_OK;
}

pkv_status pkv_sched_add_request(void* sched, int64_t req_id, int32_t prompt_len,
                                 int32_t max_new_tokens, int64_t prefix_id) {
  Scheduler* s = static_cast<Scheduler*>(sched);
  if (!s) return err(PKV_ERR_INVALID_ARG, "NULL scheduler");
  std::lock_guard<std::mutex> lk(s->mu);
  if (s->reqs.count(req_id)) return err(PKV_ERR_INVALID_ARG, "request id in use");
  if (prompt_len <= 0 || max_new_tokens <= 0)
    return err(PKV_ERR_INVALID_ARG, "prompt_len and max_new_tokens must be positive");
  int32_t prefix_tokens = 0, prefix_pages = 0;
  if (prefix_id >= 0) {
    auto it = s->prefixes.find(prefix_id);
    if (it == s->prefixes.end()) return err(PKV_ERR_INVALID_ARG, "unknown prefix");
    prefix_tokens = it->second.tokens;
    prefix_pages = (int32_t)it->second.pages.size();
    if (prompt_len <= prefix_tokens)
      return err(PKV_ERR_INVALID_ARG, "prompt must extend past its shared prefix");
  }
  std::unique_ptr<Request> r(new Request);
  r->id = req_id;
  r->prompt_len = prompt_len;
  r->max_new = max_new_tokens;
  r->num_tokens = prompt_len;
  r->prefix_id = prefix_id;
  r->prefix_tokens = prefix_tokens;
  // A request that could not fit even in an otherwise empty pool would stall
  // the queue for ever: refuse it now.
  int32_t pinned = 0;
  for (const auto& kv : s->prefixes) pinned += (int32_t)kv.second.pages.size();
  const int32_t own = s->worst_private_pages(*r);
  if (own + pinned > s->cfg.num_pages)
    return err(PKV_ERR_OUT_OF_PAGES, "request needs " + std::to_string(own + prefix_pages) +
                                         " pages; the pool has " +
                                         std::to_string(s->cfg.num_pages - pinned + prefix_pages));
  if (prefix_id >= 0) ++s->prefixes.at(prefix_id).users;
  s->waiting.push_back(r.get());
  s->reqs.emplace(req_id, std::move(r));
  return PKV_OK;
}

pkv_status pkv_sched_schedule(void* sched, pkv_sched_item* items, int32_t items_cap,
                              int32_t* num_items, int64_t* preempted, int32_t preempted_cap,
                              int32_t* num_preempted) {
  Scheduler* s = static_cast<Scheduler*>(sched);
  if (!s || !num_items || !num_preempted) return err(PKV_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(s->mu);
  if (s->planned) return err(PKV_ERR_INVALID_ARG, "previous step not committed");
  if (items_cap < s->cfg.max_batch_size || (preempted_cap < s->cfg.max_batch_size))
    return err(PKV_ERR_INVALID_ARG, "item and preemption buffers must hold max_batch_size entries");
  if ((s->cfg.max_batch_size > 0 && !items) || !preempted)
    return err(PKV_ERR_INVALID_ARG, "NULL buffers");
  s->plan.clear();
  std::vector<int64_t> evicted;
  int32_t budget = s->cfg.max_num_tokens;

  // 1. running requests, oldest first; a shortfall evicts the newest (LIFO)
  for (size_t i = 0; i < s->running.size() && budget > 0;) {
    Request* r = s->running[i];
    const int32_t n = s->step_tokens(*r, budget);
    const int32_t need = s->extra_pages(*r, n);
    bool self_evicted = false;
    while (s->free_pages() < need) {
      Request* v = s->running.back();
      s->evict(v, evicted);
      if (v == r) { self_evicted = true; break; }
    }
    if (self_evicted) break;               // r was the newest: nothing after it remains
    s->grow(*r, need);
    const int32_t kind = (r->num_tokens - r->num_computed) > 1 ? PKV_WORK_PREFILL : PKV_WORK_DECODE;
    s->plan.push_back(pkv_sched_item{r->id, r->slot, kind, r->num_computed, n});
    budget -= n;
    ++i;
  }

  // 2. admit from the front of the waiting queue while it fits (no eviction)
  while (!s->waiting.empty() && budget > 0 &&
         (int32_t)s->running.size() < s->cfg.max_batch_size) {
    Request* r = s->waiting.front();
    const int32_t start = r->prefix_tokens;   // cached on admission (shared pages)
    const int32_t pending = r->num_tokens - start;
    const int32_t n = std::min(pending > 1 ? std::min(s->cfg.chunk_size, pending) : 1, budget);
    const int32_t first = s->pages_for((int64_t)start + n) - s->pages_for(start);
    int32_t need = first;
    if (s->cfg.policy == PKV_SCHED_CONSERVATIVE) {
      need = s->worst_private_pages(*r);
      for (const Request* q : s->running)
        need += s->pages_for(s->max_cached(*q)) - (int32_t)q->pages.size();
    }
    if (s->free_pages() < need) break;
    s->waiting.pop_front();
    s->attach_prefix(*r);
    s->grow(*r, first);
    s->take_slot(*r);
    s->running.push_back(r);
    const int32_t kind = (r->num_tokens - r->num_computed) > 1 ? PKV_WORK_PREFILL : PKV_WORK_DECODE;
    s->plan.push_back(pkv_sched_item{r->id, r->slot, kind, r->num_computed, n});
    budget -= n;
  }

  // An evicted request was running (<= max_batch_size of them); report all.
  *num_items = (int32_t)s->plan.size();
  std::copy(s->plan.begin(), s->plan.end(), items);
  *num_preempted = (int32_t)evicted.size();
  std::copy(evicted.begin(), evicted.end(), preempted);
  if (s->plan.empty() && !s->waiting.empty() && s->running.empty())
    return err(PKV_ERR_OUT_OF_PAGES, "the front request cannot be admitted into an empty batch");
  s->planned = true;
  return PKV_OK;
}

int32_t pkv_sched_block_table(const void* sched, int64_t req_id, int32_t* out, int32_t cap) {
  const Scheduler* s = static_cast<const Scheduler*>(sched);
  if (!s) return -1;
  std::lock_guard<std::mutex> lk(const_cast<Scheduler*>(s)->mu);
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return -1;
  const std::vector<int32_t>& p = it->second->pages;
  if (out) std::copy(p.begin(), p.begin() + std::min<size_t>(p.size(), std::max(cap, 0)), out);
  return (int32_t)p.size();
}

pkv_status pkv_sched_commit(void* sched, int64_t* finished, int32_t finished_cap,
                            int32_t* num_finished) {
  Scheduler* s = static_cast<Scheduler*>(sched);
  if (!s || !num_finished) return err(PKV_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(s->mu);
  if (!s->planned) return err(PKV_ERR_INVALID_ARG, "nothing scheduled");
  if (finished_cap < (int32_t)s->plan.size() || (!s->plan.empty() && !finished))
    return err(PKV_ERR_INVALID_ARG, "finished buffer must hold one entry per scheduled item");
  int32_t nf = 0;
  for (const pkv_sched_item& it : s->plan) {
    Request* r = s->reqs.at(it.req_id).get();
    r->num_computed += it.num_tokens;
    if (r->num_computed == r->num_tokens) {   // the model produced the next token
      ++r->generated;
      ++r->num_tokens;
      if (r->generated == r->max_new) {
        s->release_pages(*r);
        s->drop_slot(*r);
        s->running.erase(std::find(s->running.begin(), s->running.end(), r));
        if (r->prefix_id >= 0) --s->prefixes.at(r->prefix_id).users;
        finished[nf++] = r->id;
        s->reqs.erase(it.req_id);
      }
    }
  }
  *num_finished = nf;
  s->plan.clear();
  s->planned = false;
  return PKV_OK;
}

pkv_status pkv_sched_finish(void* sched, int64_t req_id) {
  Scheduler* s = static_cast<Scheduler*>(sched);
  if (!s) return err(PKV_ERR_INVALID_ARG, "NULL scheduler");
  std::lock_guard<std::mutex> lk(s->mu);
  if (s->planned) return err(PKV_ERR_INVALID_ARG, "commit the scheduled step first");
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return err(PKV_ERR_INVALID_ARG, "unknown request");
  Request* r = it->second.get();
  s->release_pages(*r);
  s->drop_slot(*r);
  auto rit = std::find(s->running.begin(), s->running.end(), r);
  if (rit != s->running.end()) s->running.erase(rit);
  auto wit = std::find(s->waiting.begin(), s->waiting.end(), r);
  if (wit != s->waiting.end()) s->waiting.erase(wit);
  if (r->prefix_id >= 0) --s->prefixes.at(r->prefix_id).users;
  s->reqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_sched_query(const void* sched, int64_t req_id, pkv_sched_request_state* out) {
  const Scheduler* s = static_cast<const Scheduler*>(sched);
  if (!s || !out) return err(PKV_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(const_cast<Scheduler*>(s)->mu);
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return err(PKV_ERR_INVALID_ARG, "unknown request");
  const Request& r = *it->second;
  const bool run = std::find(s->running.begin(), s->running.end(), &r) != s->running.end();
  *out = pkv_sched_request_state{r.num_tokens, r.num_computed, r.generated,
                                 (int32_t)r.pages.size(), r.slot, run ? 1 : 0};
  return PKV_OK;
}

pkv_status pkv_sched_stats(const void* sched, pkv_sched_counts* out) {
  const Scheduler* s = static_cast<const Scheduler*>(sched);
  if (!s || !out) return err(PKV_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(const_cast<Scheduler*>(s)->mu);
  *out = pkv_sched_counts{(int32_t)s->waiting.size(), (int32_t)s->running.size(),
                          s->free_pages(), s->preemptions};
  return PKV_OK;
}

}  // extern "C"
