// dit_block_forward without a caller workspace: the block's intermediates live in a file-scope
// device array of fixed size, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation). The entry point
// allocates nothing itself; it runs dit_block_forward's kernels on that array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/avdit.h"
#include "kernels.hpp"

// One copy per GPU, held from the module's load until the process ends.
static __device__ __align__(256) unsigned char scratch[DIT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = (size_t)DIT_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once per device. The
// array's name in host code is only a handle for the runtime, never an address to pass on.
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int dit_block_forward_noalloc(const dit_dims* dims, const dit_layout* layout,
                                         const dit_block_weights* weights, const float* temb,
                                         const uint16_t* x_in, uint16_t* x_out, int32_t attn_mode,
                                         void* stream) {
  // The size check comes first and touches no device. dit_workspace_size is 0 only for dims or
  // a layout that dit_block_forward rejects during validation, before any device work: let it
  // report them with its own status and message.
  const size_t need = dit_workspace_size(dims, layout, 0, nullptr);
  if (need == 0)
    return dit_block_forward(dims, layout, weights, temb, x_in, x_out, attn_mode, nullptr, 0,
                             stream);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "dit_block_forward_noalloc: the block needs %zu bytes of intermediates; the "
             "built-in scratch holds %zu (use dit_block_forward with a workspace)",
             need, kScratchBytes);
    return avdit::set_last_error(DIT_ERR_UNSUPPORTED, msg);
  }
  void* ws = nullptr;
  const hipError_t e = scratch_for_current_device(&ws);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "dit_block_forward_noalloc: no scratch on the current device: %s",
             hipGetErrorString(e));
    return avdit::set_last_error(DIT_ERR_DEVICE, msg);
  }
  return dit_block_forward(dims, layout, weights, temb, x_in, x_out, attn_mode, ws, kScratchBytes,
                           stream);
}
