// Host page allocator for the paged KV cache.
//
// The cache is a pool of fixed-size pages handed out on demand and returned
// when a request leaves; pages of a repeated prompt prefix are shared between
// sequences ("TensorRT-LLM框架解析与高性能推理优化实践" §4.2: KVCacheManager with
// allocate_blocks / free_blocks, block reuse and prefix sharing; §4.1: the
// slot manager guarantees safe concurrent access).  Exhaustion is reported,
// not hidden (§5.2: an out-of-memory error when nothing can be freed).
//
// Design: a LIFO free stack of page ids (the most recently freed page is
// handed out first, so a hot page is reused while it may still sit in cache)
// plus a refcount per page.  All-or-nothing allocation; every mutation is
// checked in full before anything changes, so a failed call leaves the state
// untouched.  One mutex serialises all calls.
#include <cstdint>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

struct Allocator {
  std::mutex mu;
  std::vector<int32_t> free_stack;   // ids, top = back
  std::vector<int32_t> refcount;     // 0 = free
};

}  // namespace

// The thread-local message behind pkv_last_error() lives in api.cpp.
namespace pkv_detail {
void set_error(const std::string& s);
}

extern "C" {

pkv_status pkv_allocator_create(int32_t num_pages, void** out_alloc) {
  if (!out_alloc) { pkv_detail::set_error("out_alloc is NULL"); return PKV_ERR_INVALID_ARG; }
  *out_alloc = nullptr;
  if (num_pages <= 0) {
    pkv_detail::set_error("num_pages must be positive, got " + std::to_string(num_pages));
    return PKV_ERR_INVALID_ARG;
  }
  Allocator* a = new (std::nothrow) Allocator;
  if (!a) { pkv_detail::set_error("out of host memory"); return PKV_ERR_INVALID_ARG; }
  a->refcount.assign(num_pages, 0);
  a->free_stack.reserve(num_pages);
  for (int32_t i = num_pages - 1; i >= 0; --i) a->free_stack.push_back(i);  // 0 on top
  *out_alloc = a;
  return PKV_OK;
}

void pkv_allocator_destroy(void* alloc) { delete static_cast<Allocator*>(alloc); }

pkv_status pkv_alloc_pages(void* alloc, int32_t n, int32_t* out_ids) {
  Allocator* a = static_cast<Allocator*>(alloc);
  if (!a) { pkv_detail::set_error("allocator is NULL"); return PKV_ERR_INVALID_ARG; }
  if (n < 0) { pkv_detail::set_error("negative page count"); return PKV_ERR_INVALID_ARG; }
  if (n > 0 && !out_ids) { pkv_detail::set_error("out_ids is NULL"); return PKV_ERR_INVALID_ARG; }
  std::lock_guard<std::mutex> lk(a->mu);
  if ((size_t)n > a->free_stack.size()) {
    pkv_detail::set_error("out of pages: " + std::to_string(n) + " requested, " +
                          std::to_string(a->free_stack.size()) + " free");
    return PKV_ERR_OUT_OF_PAGES;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = a->free_stack.back();
    a->free_stack.pop_back();
    a->refcount[id] = 1;
    out_ids[i] = id;
  }
  return PKV_OK;
}

pkv_status pkv_share_pages(void* alloc, int32_t n, const int32_t* ids) {
  Allocator* a = static_cast<Allocator*>(alloc);
  if (!a) { pkv_detail::set_error("allocator is NULL"); return PKV_ERR_INVALID_ARG; }
  if (n < 0 || (n > 0 && !ids)) { pkv_detail::set_error("bad id list"); return PKV_ERR_INVALID_ARG; }
  std::lock_guard<std::mutex> lk(a->mu);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || (size_t)id >= a->refcount.size() || a->refcount[id] == 0) {
      pkv_detail::set_error("share: page " + std::to_string(id) + " is not allocated");
      return PKV_ERR_INVALID_ARG;
    }
  }
  for (int32_t i = 0; i < n; ++i) ++a->refcount[ids[i]];
  return PKV_OK;
}

pkv_status pkv_free_pages(void* alloc, int32_t n, const int32_t* ids) {
  Allocator* a = static_cast<Allocator*>(alloc);
  if (!a) { pkv_detail::set_error("allocator is NULL"); return PKV_ERR_INVALID_ARG; }
  if (n < 0 || (n > 0 && !ids)) { pkv_detail::set_error("bad id list"); return PKV_ERR_INVALID_ARG; }
  std::lock_guard<std::mutex> lk(a->mu);
  // Check first (an id may repeat in the list: count the releases per id).
  std::unordered_map<int32_t, int32_t> releases;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || (size_t)id >= a->refcount.size()) {
      pkv_detail::set_error("free: page id " + std::to_string(id) + " out of range");
      return PKV_ERR_INVALID_ARG;
    }
    if (++releases[id] > a->refcount[id]) {
      pkv_detail::set_error("free: page " + std::to_string(id) +
                            " released more often than referenced (double free)");
      return PKV_ERR_INVALID_ARG;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (--a->refcount[id] == 0) a->free_stack.push_back(id);
  }
  return PKV_OK;
}

int32_t pkv_num_free_pages(const void* alloc) {
  const Allocator* a = static_cast<const Allocator*>(alloc);
  if (!a) return -1;
  std::lock_guard<std::mutex> lk(const_cast<Allocator*>(a)->mu);
  return (int32_t)a->free_stack.size();
}

int32_t pkv_page_refcount(const void* alloc, int32_t id) {
  const Allocator* a = static_cast<const Allocator*>(alloc);
  if (!a) return -1;
  std::lock_guard<std::mutex> lk(const_cast<Allocator*>(a)->mu);
  if (id < 0 || (size_t)id >= a->refcount.size()) return -1;
  return a->refcount[id];
}

}  // extern "C"
