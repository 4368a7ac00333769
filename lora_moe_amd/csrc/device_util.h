// Device helpers for gfx950 (CDNA4): bf16 conversions, the bf16 MFMA used by
// every contraction, and workgroup scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16) on one wavefront.
// Lane l supplies A[m = l%16][k = 8*(l/16) .. +8] and B[k = 8*(l/16) .. +8][n = l%16];
// it receives D[m = 4*(l/16) + i][n = l%16], i = 0..3.  Only the pairing of
// A and B k-slots matters for the sum, so callers may permute K freely as
// long as both operands use the same permutation.
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D(32x32, fp32) += A(32x16) * B(16x32), bf16.  Lane l supplies
// A[m = l%32][k = 8*(l/32) .. +8] and B[k = 8*(l/32) .. +8][n = l%32] and
// receives D[8*(v/4) + 4*(l/32) + v%4][l%32] in element v = 0..15.
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Buffer resource over [base, base + bytes), bytes < 2^31, for 16-byte loads
// whose offset may point past the end: such a load returns zeros (also when
// it copies into LDS) and touches no memory, so padding rows of a tile cost no
// traffic.  Word 3 is the gfx9 raw-buffer setting (32-bit data format).
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
constexpr uint32_t kBufNone = 0x80000000u;  // an offset past the end of every such buffer
__device__ __forceinline__ buf_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t ld16_buf(buf_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// 16-byte load of data read once (a weight stream): marked non-temporal so it
// streams through the caches without displacing lines that are reused
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ u32x4_t zero4() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + __expf(-v)); }

// Workgroup barrier that orders LDS traffic only: each wavefront waits for
// its own LDS operations, not for its outstanding global stores (for kernels
// whose threads never read back global data written by other threads of the
// workgroup; the stores still complete before the kernel ends).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0); vmcnt, expcnt unrestricted
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool LDS_ONLY>
__device__ __forceinline__ void wg_barrier() {
  if (LDS_ONLY)
    lds_barrier();
  else
    __syncthreads();
}

// Exclusive scan of one int per thread across a workgroup of `nthreads`
// (multiple of 64, <= 1024).  `lds` needs 16 ints.  Returns the exclusive
// prefix; *total receives the workgroup sum.  All threads must call it.
// LDS_ONLY: its barriers order LDS traffic only (see lds_barrier).
template <bool LDS_ONLY = false>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  wg_barrier<LDS_ONLY>();
  if (wave == 0) {
    int w = lane < nw ? lds[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int y = __shfl_up(w, o, 64);
      if (lane >= o) w += y;
    }
    if (lane < nw) lds[lane] = w;  // inclusive wave sums
  }
  wg_barrier<LDS_ONLY>();
  int before = wave ? lds[wave - 1] : 0;
  *total = lds[nw - 1];
  wg_barrier<LDS_ONLY>();
  return before + x - v;
}

}  // namespace moelora
