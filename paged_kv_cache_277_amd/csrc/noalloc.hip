// pkv_paged_attn_decode_noalloc: the decode call with its partials in a
// fixed device array of the library instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy from module load until the process ends.  Host code
// must not use the array's name as a device address: its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; the kernels receive that address as their workspace.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/pagedkv.h"

namespace pkv_detail {
void set_error(const std::string& s);
}

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];          // device address of `scratch`, per device

// The device address of the current device's array (looked up on the first
// call on the device).  The kernels run on `stream`'s device, so that must be
// the current device: the array of another device is not this one.
pkv_status scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    pkv_detail::set_error(std::string("decode_noalloc: current device: ") + hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    pkv_detail::set_error("decode_noalloc: device index out of range");
    return PKV_ERR_UNSUPPORTED;
  }
  hipDevice_t sdev = -1;
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) {
    pkv_detail::set_error(std::string("decode_noalloc: stream's device: ") + hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  if (sdev != dev) {
    pkv_detail::set_error("decode_noalloc: the stream belongs to device " + std::to_string(sdev) +
                          " but device " + std::to_string(dev) +
                          " is current; make the stream's device current first");
    return PKV_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      pkv_detail::set_error(std::string("decode_noalloc: scratch address: ") +
                            hipGetErrorString(e));
      return PKV_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_decode_noalloc(const pkv_cache_desc* cache, const void* q,
                                         int32_t q_dtype, void* out, int32_t out_dtype,
                                         float* lse, const int32_t* block_tables,
                                         int32_t bt_stride, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t num_q_heads,
                                         int32_t max_context_len, float sm_scale,
                                         int32_t split_tokens, void* stream) {
  // Size first: a call whose partials exceed the array is refused before
  // anything touches the device.  (Invalid arguments give 0 here and are
  // reported by the decode call's own checks below.)
  const size_t need = pkv_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_context_len,
                                                 split_tokens);
  if (need > kScratchBytes) {
    pkv_detail::set_error("decode_noalloc: the call needs " + std::to_string(need) +
                          " bytes of partials, more than the " + std::to_string(kScratchBytes) +
                          "-byte scratch array (use pkv_paged_attn_decode with a workspace, or "
                          "longer split_tokens)");
    return PKV_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  pkv_status st = scratch_on_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st != PKV_OK) return st;
  return pkv_paged_attn_decode(cache, q, q_dtype, out, out_dtype, lse, block_tables, bt_stride,
                               context_lens, num_seqs, num_q_heads, max_context_len, sm_scale,
                               split_tokens, ws, kScratchBytes, stream);
}

}  // extern "C"
