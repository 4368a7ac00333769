// Top-k combine: y[t][:] = sum_j d[row(t, j)][:] (d already carries the pair's
// top-k weight), rounded to bf16.  The router sends each token to several
// experts and the layer then sums their outputs (vLLM blog "Multi-LoRA for
// MoE models", section "Implementing multi-LoRA inference for MoE models in
// vLLM").  Summation runs over j in ascending order, so y is deterministic for
// a given d.  One thread produces 8 consecutive outputs (one 16-byte store).
#include "device_util.h"
#include "internal.h"

namespace moelora {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ d,
                                                      const int32_t* __restrict__ pos, int T,
                                                      int H, int k, int nslab, int64_t slab,
                                                      uint16_t* __restrict__ y) {
  const int per_row = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx - (int64_t)t * per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int row = pos[(size_t)t * k + j];
    if (row < 0) continue;  // dropped pair (invalid expert id)
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // the pair's output: its K-split slabs in order
    for (int sl = 0; sl < nslab; ++sl) {
      const float4* src = reinterpret_cast<const float4*>(d + sl * slab + (size_t)row * H + c);
      const float4 v0 = src[0], v1 = src[1];
      v[0] += v0.x; v[1] += v0.y; v[2] += v0.z; v[3] += v0.w;
      v[4] += v1.x; v[5] += v1.y; v[6] += v1.z; v[7] += v1.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  u32x4_t out;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    out[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(y + (size_t)t * H + c) = out;
}

}  // namespace

int launch_combine(const Layout& L, void* ws, uint16_t* y, hipStream_t st) {
  WsPtrs w = ws_ptrs(ws, L);
  const int64_t n = (int64_t)L.T * (L.H / 8);
  const int grid = (int)((n + 255) / 256);
  combine_kernel<<<grid, 256, 0, st>>>(w.d, w.pos, L.T, L.H, L.k, L.dsplit, L.cap_rows * (int64_t)L.H, y);
  return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

}  // namespace moelora
