// dreamer_seq_attn_noalloc: dreamer_seq_attn without a caller-supplied workspace, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  Its scratch is a fixed file-scope device
// array, one copy per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dreamer.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = DREAMER_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The fixed scratch.  In host code this name is only a host-side stand-in for the device
// symbol: every host use goes through the device address that scratch_ptr() looks up.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];

// This device's address of `scratch`, looked up once per device with that device current
// (each GPU holds its own copy of the array at its own address).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return dreamer::api_fail(DREAMER_E_HIP, "seq_attn_noalloc: no current device");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return dreamer::api_fail(DREAMER_E_HIP, "seq_attn_noalloc: scratch address: %s",
                               hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return DREAMER_OK;
}

}  // namespace

extern "C" int dreamer_seq_attn_noalloc(int dtype, int B, int q_len, int H, int d,
                                        int64_t pos0, const void* q, const void* k_new,
                                        const void* v_new, void* k_cache, void* v_cache,
                                        int64_t cap, void* out, const float* cos_s,
                                        const float* sin_s, float scale, int sa_rope,
                                        dreamer_stream_t stream) {
  // sizes the validation of dreamer_seq_attn rejects are left to it (DREAMER_E_INVAL)
  if (B >= 0 && q_len >= 0 && H > 0 && d > 0 && pos0 >= 0) {
    const size_t need = dreamer_seq_attn_ws_bytes(dtype, B, q_len, H, d, pos0);
    if (need > kScratchBytes)
      return dreamer::api_fail(DREAMER_E_WORKSPACE,
                               "seq_attn_noalloc: this shape needs %zu bytes of scratch, more "
                               "than the fixed %zu (use dreamer_seq_attn with a workspace)",
                               need, kScratchBytes);
  }
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc) return rc;
  return dreamer_seq_attn(dtype, B, q_len, H, d, pos0, q, k_new, v_new, k_cache, v_cache,
                          cap, out, cos_s, sin_s, scale, sa_rope, ws, kScratchBytes, stream);
}
