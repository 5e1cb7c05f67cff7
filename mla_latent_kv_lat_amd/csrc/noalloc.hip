// mla_decode_noalloc: mla_decode for callers that cannot allocate device memory.
//
// The decode kernels' partial results (the pieces of sequences cut by the split plan and
// the batch's tile prefix) live in a workspace.  Here it is a static device array: every
// GPU the library runs on holds its own copy, for the life of the process, and every call
// on that GPU shares it.  The array's name is a host-side stand-in in host code, so its
// device address is looked up once per device (with that device current) and only that
// address is handed to the kernels.  Nothing in the array needs to start at zero: the
// kernels write every entry they read in the same call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace {

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first call there).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return int(e);
      if (!p) return int(hipErrorInvalidSymbol);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return 0;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" mla_status mla_decode_noalloc(const mla_dims* d, const void* q_lat, const void* q_rope,
                                         mla_dtype q_dt, const void* c_kv, mla_dtype kv_dt,
                                         const float* kv_scale, const void* k_rope, mla_dtype rope_dt,
                                         int32_t T, const int32_t* seq_lens, void* o_lat, mla_dtype o_dt,
                                         float* lse, void* stream) {
  DecodeArgs a;
  DecodePlan p;
  mla_status st = prepare_decode(d, q_lat, q_rope, q_dt, c_kv, kv_dt, kv_scale, k_rope, rope_dt, T,
                                 seq_lens, o_lat, o_dt, lse, &a, &p);
  if (st != MLA_OK) return st;
  // Plans whose partial results exceed the static array are refused before any HIP call.
  if (p.workspace > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p.workspace > 0) {
    const int err = scratch_ptr(&ws);
    if (err) return hip_error_status(err);
  }
  st = attach_workspace(&a, p, ws, MLA_NOALLOC_SCRATCH_BYTES);
  if (st != MLA_OK) return st;
  return run_decode(a, p, static_cast<hipStream_t>(stream));
}
