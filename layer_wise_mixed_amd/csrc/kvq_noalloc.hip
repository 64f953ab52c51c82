// kvq_noalloc.hip -- decode attention for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation): kvq_decode_attention with its split-partials workspace
// taken from a fixed array of device memory that the library holds, instead
// of from the caller.
//
// The array is a file-scope __device__ variable, so each GPU the library runs
// on holds its own copy until the process ends. Host code never passes the
// variable's name to a kernel (in host code that name is only a stand-in, not
// a device address): the first call on a device, with that device current,
// looks up the device address with hipGetSymbolAddress and keeps it for that
// device. Every call on a device shares its array: calls that overlap on one
// GPU (launched on different streams and running at the same time) race on
// it. The split pass writes every partial it reads back in the merge pass, so
// nothing in the array needs to start at zero.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

static __device__ __align__(256) unsigned char scratch[size_t(16) << 20];

namespace {

constexpr size_t kScratchBytes = sizeof(scratch);  // 16 MiB: batch * Hq * splits <= 32520 rows of 129 fp32

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch` (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof msg, "hipGetDevice: %s", hipGetErrorString(e));
    return kvq::set_error(KVQ_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return kvq::set_error(KVQ_ERR_UNSUPPORTED, "device index beyond 64");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
      return kvq::set_error(KVQ_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" int kvq_decode_attention_noalloc(const kvq_plan* plan, int32_t layer, const void* cache,
                                            const uint16_t* q, const int32_t* seq_lens, int32_t batch,
                                            int32_t max_seq_len, float softmax_scale, void* out, int32_t out_dtype,
                                            float* lse_out, int32_t num_splits, const kvq_pages* pages,
                                            kvq_stream_t stream) {
  if (!plan) return kvq::set_error(KVQ_ERR_INVALID_ARG, "plan is NULL");
  if (num_splits < 0 || num_splits > 1024 || batch < 0 || max_seq_len < 0)
    return kvq::set_error(KVQ_ERR_INVALID_ARG, "num_splits, batch or max_seq_len out of range");
  const size_t need = kvq_decode_workspace_bytes(plan, batch, max_seq_len, num_splits);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "the split partials need %zu bytes, more than the %zu bytes of the library's scratch array "
             "(fewer splits or a smaller batch fit; kvq_decode_attention takes a workspace of any size)",
             need, kScratchBytes);
    return kvq::set_error(KVQ_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  return kvq_decode_attention(plan, layer, cache, q, seq_lens, batch, max_seq_len, softmax_scale, out, out_dtype,
                              lse_out, ws, kScratchBytes, num_splits, pages, stream);
}
