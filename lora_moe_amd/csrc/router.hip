// Router kernel: top-k experts per token from fp32 logits, and their
// weights; one wavefront per token (route_token in router_device.h holds the
// choice and its reading of the pages).
#include "device_util.h"
#include "internal.h"
#include "router_device.h"

namespace moelora {

namespace {

template <int R>
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                     int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wavefront
  int e;
  float wt;
  route_token<R>(logits + (size_t)t * E, E, k, &e, &wt);
  const int lane = threadIdx.x & 63;
  if (lane < k) {
    ids[(size_t)t * k + lane] = e;
    w[(size_t)t * k + lane] = wt;
  }
}

}  // namespace

int launch_router(const Layout& L, const float* logits, int32_t* ids, float* w, hipStream_t st) {
  const int grid = (L.T + 3) / 4;
  if (L.E <= 512)
    router_kernel<8><<<grid, 256, 0, st>>>(logits, L.T, L.E, L.k, ids, w);
  else
    router_kernel<0><<<grid, 256, 0, st>>>(logits, L.T, L.E, L.k, ids, w);
  return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

}  // namespace moelora
