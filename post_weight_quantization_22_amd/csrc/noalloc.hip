// gptq_quantize_layer without any allocation: the column loop's scratch (the
// working copy W' of the weights, the block errors, codes in processing
// order, the inverse order) lives in a fixed-size array of device memory
// that belongs to the library, one copy per GPU, for callers that cannot
// allocate (code under HIP graph capture, tight loops, harnesses that forbid
// hipMalloc).  The kernels are those of gptq_quantize_layer, given that
// array as their workspace.
#include <mutex>

#include "kernels.hpp"

namespace {

// The scratch array.  In host code its name is only a stand-in for the
// symbol: the device address of this GPU's copy comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[GPTQ_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch[64] = {};

// This device's copy of `scratch` (looked up on the first call on the device,
// with that device current).
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

gptq_status gptq_quantize_layer_noalloc(const void* W, gptq_dtype wdt, int64_t m, int64_t n,
                                        int64_t ldw, const float* U, int64_t ldu,
                                        const int32_t* perm, const uint8_t* dead,
                                        const gptq_config* cfg, uint8_t* codes, float* scales,
                                        float* zeros, int32_t* g_idx, float* row_err,
                                        int32_t* info, hipStream_t stream) {
  if (!cfg) return GPTQ_ERR_INVALID_ARG;
  if (m < 0 || n < 0) return GPTQ_ERR_INVALID_ARG;
  // a layer whose workspace exceeds the fixed scratch is refused before any work
  if (m > 0 && n > 0 && (cfg->desc_act == 0 || cfg->desc_act == 1) &&
      gptq::quantize_ws_bytes(m, n, cfg->desc_act) > (size_t)GPTQ_NOALLOC_SCRATCH_BYTES)
    return GPTQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return GPTQ_ERR_HIP;
  return gptq::quantize_layer_checked(W, wdt, m, n, ldw, U, ldu, perm, dead, cfg, codes, scales,
                                      zeros, g_idx, row_err, info, ws,
                                      (size_t)GPTQ_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
