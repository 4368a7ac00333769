// moe_lora_forward_noalloc: align + forward with the workspace in a static
// device array owned by the library, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The kernels are the ones moe_lora_align and
// moe_lora_forward launch; only where their workspace lives differs.
#include <atomic>

#include "internal.h"

namespace moelora {

namespace {

// The workspace of every call on one GPU.  Each GPU the library runs on
// holds its own copy until the process ends.  On the host this name is a
// stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[MOE_LORA_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, looked up once per device
// (with that device current); nullptr when the lookup fails.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);  // same value from every thread
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

}  // namespace moelora

using namespace moelora;

extern "C" int moe_lora_forward_noalloc(const moe_lora_shape* shape, const uint16_t* x,
                                        const int32_t* topk_ids, const float* topk_weights,
                                        const int32_t* lora_ids, const uint16_t* W_gu,
                                        const uint16_t* W_down, const uint16_t* A_gu,
                                        const uint16_t* B_gu, const uint16_t* A_down,
                                        const uint16_t* B_down, uint16_t* y, void* stream) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (L.total > (size_t)MOE_LORA_NOALLOC_WORKSPACE_BYTES) return MOE_LORA_EWORKSPACE;
  if (L.T == 0) return MOE_LORA_OK;
  const void* ptrs[] = {x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu, A_down, B_down, y};
  for (const void* p : ptrs)
    if (!p) return MOE_LORA_EINVAL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_LORA_EALIGN;
  void* ws = scratch_ptr();
  if (!ws) return MOE_LORA_EHIP;
  // the align rewrites every align output and clears the split-K shrink
  // accumulators, so what the previous call left in the scratch is never read
  rc = moe_lora_align(shape, topk_ids, lora_ids, ws, L.total, stream);
  if (rc) return rc;
  return moe_lora_forward(shape, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu, A_down,
                          B_down, ws, L.total, y, stream);
}
