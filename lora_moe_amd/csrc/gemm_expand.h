// LoRA expand from registers inside the LDS-tiled GEMMs: the expand output
// z * B is added to the base output on the accumulators of the same kernel
// (vLLM blog "Multi-LoRA for MoE models", sections "Implementing multi-LoRA
// inference for MoE models in vLLM" and "Kernel optimizations").  This is the
// form for ranks below 32 (or when the shape asks for it); from rank 32 the
// tiled GEMMs run the expand as extra K stages of their own ring instead.
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
// Segments are found with one load per adapter id across the lanes and a
// ballot, and taken NB at a time.  For each batch and each rank slice of 16
// (one MFMA K step) the slice of z of the lane's rows and the B rows of the
// batch's segments are loaded together -- one memory round trip per slice --
// then s*z is rounded to bf16 (the shrink result enters the product at bf16
// precision, like every other operand) and masked per segment.  The expand
// runs once per tile with one workgroup per CU, so its round trips are time
// the MFMA pipes wait: loading z and B together halved them.
template <int MI, int NI, bool WA, int NB = 8>
__device__ __forceinline__ void lora_expand(f32x16_t (&acc)[MI][NI], const GemmParams& p, int e,
                                            int wrow0, const int (&ncol)[NI], int lbeg = 0) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, khalf = lane >> 5;
  const int S = p.L + 1;
  const int wrow1 = wrow0 + 32 * MI;
  for (int l0 = lbeg; l0 < p.L; l0 += 64) {
    const int lj = l0 + lane;
    int st = 0, cnt = 0;
    if (lj < p.L) {
      st = p.segstart[e * S + lj];
      cnt = p.segcnt[e * S + lj];
    }
    uint64_t pending = __ballot(cnt > 0 && st < wrow1 && st + cnt > wrow0);
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
      for (int q0 = 0; q0 < p.r; q0 += 16) {
        const int qa = q0 + 8 * khalf;
        const bool qok = qa < p.r;
        float4 z0[MI], z1[MI];
        u32x4_t bfr[NB][NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          z0[mi] = make_float4(0.f, 0.f, 0.f, 0.f);
          z1[mi] = z0[mi];
          if (qok) {
            const float4* zp = reinterpret_cast<const float4*>(p.z + (size_t)(wrow0 + 32 * mi + l32) * p.r + qa);
            z0[mi] = zp[0];
            z1[mi] = zp[1];
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nb) {
            const uint16_t* Bl = p.B + ((size_t)(l0 + ids[b]) * p.E + e) * p.N * p.r;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bfr[b][ni] = qok ? ld16(Bl + (size_t)ncol[ni] * p.r + qa) : zero4();
          }
        }
        u32x4_t zh[MI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const float zv[8] = {p.s * z0[mi].x, p.s * z0[mi].y, p.s * z0[mi].z, p.s * z0[mi].w,
                               p.s * z1[mi].x, p.s * z1[mi].y, p.s * z1[mi].z, p.s * z1[mi].w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            zh[mi][i] = (uint32_t)f32_to_bf16(zv[2 * i]) | ((uint32_t)f32_to_bf16(zv[2 * i + 1]) << 16);
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
              const u32x4_t h = (row >= sst && row < send) ? zh[mi] : zero4();
#pragma unroll
              for (int ni = 0; ni < NI; ++ni) {
                if (WA)
                  acc[mi][ni] = mfma_32x32x16(bfr[b][ni], h, acc[mi][ni]);
                else
                  acc[mi][ni] = mfma_32x32x16(h, bfr[b][ni], acc[mi][ni]);
              }
            }
          }
        }
      }
    }
  }
}

// The same expand as work items spread over a K loop, for adapters
// [lbeg, lbeg + 64): item i is (segment i / ns in ascending adapter order,
// rank slice i % ns, ns = r / 16) over the nseg segments that meet the
// wavefront's rows; when the items outnumber the K stages, the loop keeps
// the first whole segments and leaves the rest to the batched expand
// (expand_items_cap).  A loaded item holds s*z of the lane's rows for the slice (bf16,
// from the shrink) and the segment's B rows at the lane's columns; its
// masked MFMAs run a K stage after its loads, so their latency passes under
// the main loop's work instead of stalling the epilogue (one workgroup per
// CU at 256 x 256 tiles leaves nothing else to run).  Weight side first, as
// in lora_expand<..., WA = true>.
template <int MI, int NI>
struct ExpandItems {
  uint64_t hit;  // bit l: adapter lbeg + l has a segment meeting the rows
  int nseg, nitems, next;
  int lrest;     // first adapter left to the batched expand (lbeg + 64: none)
  int st, cnt;   // segment of adapter lbeg + lane
  int l;         // adapter bit of the loaded item
  u32x4_t z[MI];
  u32x4_t b[NI];
};

template <int MI, int NI>
__device__ __forceinline__ void expand_items_init(ExpandItems<MI, NI>& it, const GemmParams& p, int e,
                                                  int wrow0, int lbeg) {
  const int lane = threadIdx.x & 63, S = p.L + 1, lj = lbeg + lane;
  it.st = 0;
  it.cnt = 0;
  if (lj < p.L) {
    it.st = p.segstart[e * S + lj];
    it.cnt = p.segcnt[e * S + lj];
  }
  it.hit = __ballot(it.cnt > 0 && it.st < wrow0 + 32 * MI && it.st + it.cnt > wrow0);
  it.nseg = __builtin_popcountll(it.hit);
  it.nitems = it.nseg * ((p.r + 15) >> 4);
  it.next = 0;
  it.l = 0;
  it.lrest = lbeg + 64;
}

// Keep the first whole segments whose items fit in `cap` (items run segment
// by segment, rank slices within a segment); the rest go to the batched
// expand from the adapter of the first segment left out.
template <int MI, int NI>
__device__ __forceinline__ void expand_items_cap(ExpandItems<MI, NI>& it, const GemmParams& p, int lbeg, int cap) {
  const int ns = (p.r + 15) >> 4;
  if (it.nitems <= cap) return;
  const int keep = cap / ns;  // whole segments
  uint64_t m = it.hit;
  for (int k = 0; k < keep; ++k) m &= m - 1;
  it.lrest = lbeg + __builtin_ctzll(m);
  it.nitems = keep * ns;
}

template <int MI, int NI>
__device__ __forceinline__ void expand_item_load(ExpandItems<MI, NI>& it, const GemmParams& p, int e,
                                                 int wrow0, int lbeg, const int (&ncol)[NI]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, khalf = lane >> 5;
  const int ns = (p.r + 15) >> 4;
  const int j = it.next / ns, q = it.next - j * ns;  // segment j, rank slice q
  uint64_t m = it.hit;
  for (int k = 0; k < j; ++k) m &= m - 1;
  it.l = __builtin_ctzll(m);
  const int qa = 16 * q + 8 * khalf;
  const bool qok = qa < p.r;
  // z only for the row blocks the segment meets (the others skip their
  // MFMAs): DeepSeek-like layer 8.20 -> 8.12 ms, down GEMM 2.77 -> 2.71
  const int sst = __builtin_amdgcn_readlane(it.st, it.l);
  const int send = sst + __builtin_amdgcn_readlane(it.cnt, it.l);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int sub0 = wrow0 + 32 * mi;
    it.z[mi] = zero4();
    if (qok && sub0 < send && sub0 + 32 > sst) it.z[mi] = ld16(p.zb + (size_t)(sub0 + l32) * p.r + qa);
  }
  const uint16_t* Bl = p.B + ((size_t)(lbeg + it.l) * p.E + e) * p.N * p.r;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) it.b[ni] = qok ? ld16(Bl + (size_t)ncol[ni] * p.r + qa) : zero4();
  ++it.next;
}

template <int MI, int NI>
__device__ __forceinline__ void expand_item_mfma(const ExpandItems<MI, NI>& it, f32x16_t (&acc)[MI][NI],
                                                 int wrow0) {
  const int l32 = threadIdx.x & 31;
  const int sst = __builtin_amdgcn_readlane(it.st, it.l);
  const int send = sst + __builtin_amdgcn_readlane(it.cnt, it.l);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int sub0 = wrow0 + 32 * mi;
    if (sub0 >= send || sub0 + 32 <= sst) continue;  // this 32-row block misses the segment
    const int row = sub0 + l32;
    const u32x4_t h = (row >= sst && row < send) ? it.z[mi] : zero4();
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma_32x32x16(it.b[ni], h, acc[mi][ni]);
  }
}

}  // namespace moelora
