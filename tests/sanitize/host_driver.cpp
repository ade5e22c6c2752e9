// Host-only replay driver for the library's page allocator and step
// scheduler (csrc/allocator.cpp, csrc/scheduler.cpp), built by the test
// suite with AddressSanitizer and UndefinedBehaviorSanitizer.
//
// It reads one command per line on stdin, calls the C ABI, and prints one
// response line per command; the test compares the responses with those the
// regular library gave to the same commands (which the scheduler tests have
// matched against the scheduling oracle).  Commands:
//
//   S_create pages page_size batch budget chunk policy  -> status
//   S_prefix id tokens        -> status page ids (tokens / page_size of them)
//   S_remove id               -> status
//   S_add id prompt max_new prefix_id   -> status
//   S_schedule                -> status n (req slot kind start tokens)* m evicted*
//   S_table id                -> count ids...
//   S_commit                  -> status n finished*
//   S_finish id               -> status
//   S_query id                -> status tokens computed generated pages slot running
//   S_stats                   -> status waiting running free preemptions
//   S_destroy
//   A_create pages            -> status
//   A_alloc n                 -> status ids...
//   A_share n ids...          -> status
//   A_free n ids...           -> status
//   A_nfree                   -> count
//   A_ref id                  -> refcount
//   A_destroy
//   A_threads threads rounds seed -> "ok" or a message: concurrent
//                               allocate / share / free on one allocator
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <random>
#include <sstream>
#include <string>
#include <thread>
#include <vector>

#include "../../include/pagedkv.h"

// The library's error-message hook (api.cpp in the full build).
namespace pkv_detail {
void set_error(const std::string& s) {
  thread_local std::string last;
  last = s;
}
}  // namespace pkv_detail

namespace {

std::string threads_stress(int nthreads, int rounds, unsigned seed) {
  void* a = nullptr;
  const int pages = 64 * nthreads;
  if (pkv_allocator_create(pages, &a) != PKV_OK) return "create failed";
  std::vector<std::thread> ts;
  std::vector<std::string> errs(nthreads);
  for (int t = 0; t < nthreads; ++t) {
    ts.emplace_back([&, t] {
      std::mt19937 rng(seed + 7919u * t);
      std::vector<int32_t> mine;
      for (int r = 0; r < rounds; ++r) {
        const int n = int(rng() % 24);
        std::vector<int32_t> got(n);
        const pkv_status st = pkv_alloc_pages(a, n, got.data());
        if (st == PKV_OK) {
          if (n && rng() % 2) {                     // share, then drop the extra reference
            if (pkv_share_pages(a, n, got.data()) != PKV_OK) errs[t] = "share failed";
            if (pkv_free_pages(a, n, got.data()) != PKV_OK) errs[t] = "free of a share failed";
          }
          mine.insert(mine.end(), got.begin(), got.end());
        } else if (st != PKV_ERR_OUT_OF_PAGES) {
          errs[t] = "alloc failed";
        }
        if (mine.size() > 40 || (rng() % 3 == 0 && !mine.empty())) {
          if (pkv_free_pages(a, int32_t(mine.size()), mine.data()) != PKV_OK) errs[t] = "free failed";
          mine.clear();
        }
      }
      if (!mine.empty() && pkv_free_pages(a, int32_t(mine.size()), mine.data()) != PKV_OK)
        errs[t] = "final free failed";
    });
  }
  for (auto& th : ts) th.join();
  std::string out = "ok";
  for (const auto& e : errs)
    if (!e.empty()) out = e;
  if (out == "ok" && pkv_num_free_pages(a) != pages) out = "pages lost";
  for (int32_t id = 0; out == "ok" && id < pages; ++id)
    if (pkv_page_refcount(a, id) != 0) out = "refcount left";
  pkv_allocator_destroy(a);
  return out;
}

}  // namespace

int main() {
  void* sched = nullptr;
  void* alloc = nullptr;
  int32_t batch = 0, page_size = 0;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    std::ostringstream out;
    if (cmd == "S_create") {
      pkv_sched_config c{};
      in >> c.num_pages >> c.page_size >> c.max_batch_size >> c.max_num_tokens >> c.chunk_size >>
          c.policy;
      batch = c.max_batch_size;
      page_size = c.page_size;
      out << pkv_sched_create(&c, &sched);
    } else if (cmd == "S_prefix") {
      int64_t id;
      int32_t tokens;
      in >> id >> tokens;
      const int32_t npages = page_size > 0 && tokens > 0 ? tokens / page_size : 0;
      std::vector<int32_t> ids(npages > 0 ? npages : 1);
      const pkv_status st = pkv_sched_add_prefix(sched, id, tokens, ids.data());
      out << st;
      if (st == PKV_OK)
        for (int32_t i = 0; i < npages; ++i) out << ' ' << ids[i];
    } else if (cmd == "S_remove") {
      int64_t id;
      in >> id;
      out << pkv_sched_remove_prefix(sched, id);
    } else if (cmd == "S_add") {
      int64_t id, prefix;
      int32_t prompt, max_new;
      in >> id >> prompt >> max_new >> prefix;
      out << pkv_sched_add_request(sched, id, prompt, max_new, prefix);
    } else if (cmd == "S_schedule") {
      std::vector<pkv_sched_item> items(batch > 0 ? batch : 1);
      std::vector<int64_t> ev(batch > 0 ? batch : 1);
      int32_t n = 0, m = 0;
      const pkv_status st = pkv_sched_schedule(sched, items.data(), batch, &n, ev.data(), batch, &m);
      out << st;
      if (st == PKV_OK) {
        out << ' ' << n;
        for (int32_t i = 0; i < n; ++i)
          out << ' ' << items[i].req_id << ' ' << items[i].slot << ' ' << items[i].kind << ' '
              << items[i].start_pos << ' ' << items[i].num_tokens;
        out << ' ' << m;
        for (int32_t i = 0; i < m; ++i) out << ' ' << ev[i];
      }
    } else if (cmd == "S_table") {
      int64_t id;
      in >> id;
      const int32_t n = pkv_sched_block_table(sched, id, nullptr, 0);
      out << n;
      if (n > 0) {
        std::vector<int32_t> ids(n);
        pkv_sched_block_table(sched, id, ids.data(), n);
        for (int32_t p : ids) out << ' ' << p;
      }
    } else if (cmd == "S_commit") {
      std::vector<int64_t> fin(batch > 0 ? batch : 1);
      int32_t n = 0;
      const pkv_status st = pkv_sched_commit(sched, fin.data(), batch, &n);
      out << st;
      if (st == PKV_OK) {
        out << ' ' << n;
        for (int32_t i = 0; i < n; ++i) out << ' ' << fin[i];
      }
    } else if (cmd == "S_finish") {
      int64_t id;
      in >> id;
      out << pkv_sched_finish(sched, id);
    } else if (cmd == "S_query") {
      int64_t id;
      in >> id;
      pkv_sched_request_state s{};
      const pkv_status st = pkv_sched_query(sched, id, &s);
      out << st;
      if (st == PKV_OK)
        out << ' ' << s.num_tokens << ' ' << s.num_computed << ' ' << s.generated << ' '
            << s.num_pages << ' ' << s.slot << ' ' << s.running;
    } else if (cmd == "S_stats") {
      pkv_sched_counts c{};
      const pkv_status st = pkv_sched_stats(sched, &c);
      out << st << ' ' << c.waiting << ' ' << c.running << ' ' << c.free_pages << ' '
          << c.preemptions;
    } else if (cmd == "S_destroy") {
      pkv_sched_destroy(sched);
      sched = nullptr;
      out << 0;
    } else if (cmd == "A_create") {
      int32_t n;
      in >> n;
      out << pkv_allocator_create(n, &alloc);
    } else if (cmd == "A_alloc") {
      int32_t n;
      in >> n;
      std::vector<int32_t> ids(n > 0 ? n : 1);
      const pkv_status st = pkv_alloc_pages(alloc, n, ids.data());
      out << st;
      if (st == PKV_OK)
        for (int32_t i = 0; i < n; ++i) out << ' ' << ids[i];
    } else if (cmd == "A_share" || cmd == "A_free") {
      int32_t n;
      in >> n;
      std::vector<int32_t> ids(n > 0 ? n : 1);
      for (int32_t i = 0; i < n; ++i) in >> ids[i];
      out << (cmd == "A_share" ? pkv_share_pages(alloc, n, ids.data())
                               : pkv_free_pages(alloc, n, ids.data()));
    } else if (cmd == "A_nfree") {
      out << pkv_num_free_pages(alloc);
    } else if (cmd == "A_ref") {
      int32_t id;
      in >> id;
      out << pkv_page_refcount(alloc, id);
    } else if (cmd == "A_destroy") {
      pkv_allocator_destroy(alloc);
      alloc = nullptr;
      out << 0;
    } else if (cmd == "A_threads") {
      int nthreads, rounds;
      unsigned seed;
      in >> nthreads >> rounds >> seed;
      out << threads_stress(nthreads, rounds, seed);
    } else {
      out << "unknown " << cmd;
    }
    std::cout << out.str() << '\n';
  }
  if (sched) pkv_sched_destroy(sched);
  if (alloc) pkv_allocator_destroy(alloc);
  return 0;
}
