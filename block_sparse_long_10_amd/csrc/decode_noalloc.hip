// msa_decode_noalloc: msa_decode for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// The decode kernels' scratch (pooled index scores, per-block partial
// outputs, the hand-off counters and the selection) lives in the file-scope
// device array below instead of a caller-provided workspace.
//
// The array exists once per GPU the library runs on and stays allocated until
// the process ends.  Host code never uses its name as an address (on the host
// it is only a handle): on each device's first call, with that device
// current, hipGetSymbolAddress gives the device address, which is kept per
// device and passed to the kernels.  Every call on a GPU shares that GPU's
// array, so calls that overlap in time on one GPU race.  Nothing in it needs
// to start at zero: the index launch clears the hand-off counters itself.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "msa.h"
#include "msa_api_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per
// device); nullptr with the error text set on failure.
void* scratch_for_current_device(msa_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "msa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    *st = msa::set_error(MSA_ERR_HIP, msg);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = msa::set_error(MSA_ERR_UNSUPPORTED, "msa_decode_noalloc: device index beyond 63");
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      char msg[256];
      std::snprintf(msg, sizeof msg, "msa_decode_noalloc: hipGetSymbolAddress(scratch): %s",
                    hipGetErrorString(e));
      *st = msa::set_error(MSA_ERR_HIP, msg);
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" msa_status msa_decode_noalloc(const msa_params* params, const msa_paged_kv* kv,
                                         const void* q, const void* idx_q,
                                         const int32_t* seq_lens, int32_t batch,
                                         int32_t max_seq_len, float* out, int32_t* sel,
                                         void* stream) {
  try {
    if (kv == nullptr) return msa::set_error(MSA_ERR_INVALID_ARGUMENT, "kv is NULL");
    const size_t need = msa_decode_workspace_bytes(params, batch, kv->max_blocks_per_seq);
    if (need == 0)  // invalid parameters: let the shared path report them
      return msa::decode_impl(params, kv, q, idx_q, seq_lens, batch, max_seq_len, out, sel,
                              nullptr, 0, stream, nullptr);
    if (need > kScratchBytes) {
      char msg[256];
      std::snprintf(msg, sizeof msg,
                    "msa_decode_noalloc: batch %d x max_blocks_per_seq %d needs %zu bytes of "
                    "scratch; the static scratch holds %zu (use msa_decode with a workspace)",
                    (int)batch, (int)kv->max_blocks_per_seq, need, kScratchBytes);
      return msa::set_error(MSA_ERR_WORKSPACE, msg);
    }
    msa_status st = MSA_OK;
    void* ws = scratch_for_current_device(&st);
    if (ws == nullptr) return st;
    return msa::decode_impl(params, kv, q, idx_q, seq_lens, batch, max_seq_len, out, sel, ws,
                            kScratchBytes, stream, nullptr);
  } catch (...) {
    return msa::set_error(MSA_ERR_HIP, "unexpected internal error");
  }
}
