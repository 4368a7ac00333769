// LoRA expand inside a grouped-GEMM epilogue, for the LDS-tiled GEMM
// families: the expand output z * B is added to the base output on the
// accumulators of the same kernel (vLLM blog "Multi-LoRA for MoE models",
// sections "Implementing multi-LoRA inference for MoE models in vLLM" and
// "Kernel optimizations").
#pragma once

#include "device_util.h"
#include "internal.h"

namespace moelora {

// acc[mi][ni] += s * z[rows] * B[l][e][cols]^T for every (expert e, adapter
// l) segment that meets the wavefront's rows [wrow0, wrow0 + 32*MI).
//
// Operand layout (bf16 MFMA 32x32x16): row block mi covers sorted rows
// wrow0 + 32*mi + lane%32 on the z side; column block ni covers the tile
// columns whose weight rows are ncol[ni] (lane%32 picks one).  WA: the weight
// side is the MFMA's first operand (the accumulators hold the tile
// transposed); otherwise z is.
//
// Each rank slice of 16 is one MFMA K step.  z (fp32) of the lane's rows is
// read and split into a bf16 pair hi + lo (hi = rne(s*z), lo = rne(s*z - hi))
// once per slice and then masked per segment; the B rows of up to NB
// segments are loaded together, so a batch waits for memory once.  Segments
// are found with one load per adapter id across the lanes and a ballot.
template <int MI, int NI, bool WA, int NB = 8>
__device__ __forceinline__ void lora_expand(f32x16_t (&acc)[MI][NI], const GemmParams& p, int e,
                                            int wrow0, const int (&ncol)[NI]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, khalf = lane >> 5;
  const int S = p.L + 1;
  const int wrow1 = wrow0 + 32 * MI;
  for (int l0 = 0; l0 < p.L; l0 += 64) {
    const int lj = l0 + lane;
    int st = 0, cnt = 0;
    if (lj < p.L) {
      st = p.segstart[e * S + lj];
      cnt = p.segcnt[e * S + lj];
    }
    const uint64_t hit = __ballot(cnt > 0 && st < wrow1 && st + cnt > wrow0);
    if (!hit) continue;
    for (int q0 = 0; q0 < p.r; q0 += 16) {
      const int qa = q0 + 8 * khalf;
      const bool qok = qa < p.r;
      u32x4_t zh[MI], zl[MI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        zh[mi] = zero4();
        zl[mi] = zero4();
        if (qok) {
          const float4* zp = reinterpret_cast<const float4*>(p.z + (size_t)(wrow0 + 32 * mi + l32) * p.r + qa);
          const float4 z0 = zp[0], z1 = zp[1];
          float zv[8];
          zv[0] = p.s * z0.x; zv[1] = p.s * z0.y; zv[2] = p.s * z0.z; zv[3] = p.s * z0.w;
          zv[4] = p.s * z1.x; zv[5] = p.s * z1.y; zv[6] = p.s * z1.z; zv[7] = p.s * z1.w;
          split8(zv, zh[mi], zl[mi]);
        }
      }
      uint64_t pending = hit;
      while (pending) {
        int ids[NB];
        int nb = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          ids[b] = 0;
          if (pending) {
            ids[b] = __builtin_ctzll(pending);
            pending &= pending - 1;
            nb = b + 1;
          }
        }
        u32x4_t bfr[NB][NI];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nb) {
            const uint16_t* Bl = p.B + ((size_t)(l0 + ids[b]) * p.E + e) * p.N * p.r;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bfr[b][ni] = qok ? ld16(Bl + (size_t)ncol[ni] * p.r + qa) : zero4();
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nb) {
            const int sst = __builtin_amdgcn_readlane(st, ids[b]);
            const int send = sst + __builtin_amdgcn_readlane(cnt, ids[b]);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
              const int sub0 = wrow0 + 32 * mi;
              if (sub0 >= send || sub0 + 32 <= sst) continue;  // this 32-row block misses the segment
              const int row = sub0 + l32;
              const bool in = row >= sst && row < send;
              const u32x4_t h = in ? zh[mi] : zero4(), lo = in ? zl[mi] : zero4();
#pragma unroll
              for (int ni = 0; ni < NI; ++ni) {
                if (WA) {
                  acc[mi][ni] = mfma_32x32x16(bfr[b][ni], h, acc[mi][ni]);
                  acc[mi][ni] = mfma_32x32x16(bfr[b][ni], lo, acc[mi][ni]);
                } else {
                  acc[mi][ni] = mfma_32x32x16(h, bfr[b][ni], acc[mi][ni]);
                  acc[mi][ni] = mfma_32x32x16(lo, bfr[b][ni], acc[mi][ni]);
                }
              }
            }
          }
        }
      }
    }
  }
}

}  // namespace moelora
