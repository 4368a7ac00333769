// Grouped GEMM over the sorted (expert, adapter) rows, with the LoRA expand
// and the activation or the top-k weight fused into the epilogue.
//
// The base projections run as one GEMM per expert over the rows routed to it
// (vLLM blog "Multi-LoRA for MoE models", section "Implementing multi-LoRA
// inference for MoE models in vLLM": fused_moe runs the projections as a
// group GEMM).  The LoRA expand z * B is added to the base output inside the
// same kernel rather than by a separate add (section "Kernel optimizations":
// the add of the LoRA result to the base result is fused into the expand).
//
// mode 0 (gate_up): a workgroup owns 32 columns j0..j0+31 of the
//   intermediate and computes both the gate rows j and the up rows I+j of
//   W_gu, so the SiLU gate h = silu(gate) * up is formed in registers:
//   the lane holding gate(row, j) also holds up(row, j).  h is stored bf16.
// mode 1 (down): a workgroup owns 64 output columns; the epilogue adds the
//   expand and multiplies by the pair's top-k weight; d is stored fp32.
//
// A workgroup (4 wavefronts) takes one tile of 16*RF rows -- rows of a single
// expert, since expert runs are padded to block_m, a multiple of the tile --
// by 64 columns.  The wavefronts split K in interleaved 64-wide steps and each
// accumulates the whole tile with bf16 MFMA 16x16x32; operands come straight
// from global memory into registers (every weight element is used by exactly
// one workgroup per row tile, so staging them in LDS buys nothing at decode
// row counts).  Each lane loads 32 contiguous bytes of a row per step and
// feeds them to two MFMAs, so the K order inside a step is permuted
// identically for both operands.  Partial tiles are added through LDS and
// wavefront 0 runs the epilogue.
#include "device_util.h"
#include "internal.h"

namespace moelora {

namespace {


// s * sum_q z[q] * B[q] with z fp32 and B a bf16 row of length r (r % 8 == 0)
__device__ __forceinline__ float expand_dot(const float* __restrict__ z,
                                            const uint16_t* __restrict__ b, int r) {
  float acc = 0.f;
  for (int q = 0; q < r; q += 8) {
    const u32x4_t bv = ld16(b + q);
    const float4 z0 = *reinterpret_cast<const float4*>(z + q);
    const float4 z1 = *reinterpret_cast<const float4*>(z + q + 4);
    acc += z0.x * bf16_lo(bv[0]) + z0.y * bf16_hi(bv[0]) + z0.z * bf16_lo(bv[1]) +
           z0.w * bf16_hi(bv[1]) + z1.x * bf16_lo(bv[2]) + z1.y * bf16_hi(bv[2]) +
           z1.z * bf16_lo(bv[3]) + z1.w * bf16_hi(bv[3]);
  }
  return acc;
}

template <int MODE, int RF, bool EVEN>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmParams p) {
  constexpr int MT = RF * 16;
  __shared__ float red[2][MT][64 + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, kq = lane >> 4;
  const int row0 = blockIdx.y * MT;
  if (row0 >= p.hdr[HDR_NUM_PADDED]) return;
  const int e = p.bexp[row0 / p.bm];

  // operand rows
  const uint16_t* arow[RF];
#pragma unroll
  for (int rf = 0; rf < RF; ++rf) {
    const int row = row0 + rf * 16 + m;
    if (MODE == 0) {
      const int pr = p.sorted[row];
      const int t = pr < p.P ? pr / p.topk : 0;  // pad rows read token 0; their output is dropped
      arow[rf] = p.in + (size_t)t * p.K;
    } else {
      arow[rf] = p.in + (size_t)row * p.K;
    }
  }
  const uint16_t* wrow[4];
  const uint16_t* Wexp = p.W + (size_t)e * p.N * p.K;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int n;
    if (MODE == 0) {
      const int j = min(blockIdx.x * 32 + (f & 1) * 16 + m, p.I - 1);
      n = (f < 2) ? j : p.I + j;
    } else {
      n = min(blockIdx.x * 64 + f * 16 + m, p.N - 1);
    }
    wrow[f] = Wexp + (size_t)n * p.K;
  }

  f32x4_t acc[RF][4];
#pragma unroll
  for (int rf = 0; rf < RF; ++rf)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[rf][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = 2;  // K steps in flight per wavefront
  for (int ks = wave; ks < p.nsteps; ks += 4 * U) {
    u32x4_t a0[U][RF], a1[U][RF], b0[U][4], b1[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = (ks + 4 * u) * 64 + kq * 16;
      const bool live = ks + 4 * u < p.nsteps;
      const bool v0 = live && (EVEN || kb < p.K), v1 = live && (EVEN || kb + 8 < p.K);
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) {
        a0[u][rf] = v0 ? ld16(arow[rf] + kb) : zero4();
        a1[u][rf] = v1 ? ld16(arow[rf] + kb + 8) : zero4();
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        b0[u][f] = v0 ? ld16(wrow[f] + kb) : zero4();
        b1[u][f] = v1 ? ld16(wrow[f] + kb + 8) : zero4();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          acc[rf][f] = mfma_16x16x32(a0[u][rf], b0[u][f], acc[rf][f]);
          acc[rf][f] = mfma_16x16x32(a1[u][rf], b1[u][f], acc[rf][f]);
        }
  }

  // add the four partial tiles: (2,3) -> (0,1) -> 0
  if (wave >= 2) {
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 2][rf * 16 + 4 * kq + i][f * 16 + m] = acc[rf][f][i];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rf][f][i] += red[wave][rf * 16 + 4 * kq + i][f * 16 + m];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[0][rf * 16 + 4 * kq + i][f * 16 + m] = acc[rf][f][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int rf = 0; rf < RF; ++rf)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rf][f][i] += red[0][rf * 16 + 4 * kq + i][f * 16 + m];

  // epilogue: rows rf*16 + 4*kq + i, columns f*16 + m
#pragma unroll
  for (int rf = 0; rf < RF; ++rf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + rf * 16 + 4 * kq + i;
      const int pr = p.sorted[row];
      const bool real = pr < p.P;
      int l = -1;
      if (real) {
        l = p.lora_ids[pr / p.topk];
        if (!(l >= 0 && l < p.L)) l = -1;
      }
      const float* zr = p.z + (size_t)row * p.r;
      const uint16_t* Bl = l >= 0 ? p.B + ((size_t)l * p.E + e) * p.N * p.r : nullptr;
      if (MODE == 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int j = blockIdx.x * 32 + f * 16 + m;
          if (j >= p.I) continue;
          float gate = acc[rf][f][i], up = acc[rf][f + 2][i];
          if (l >= 0) {
            gate += p.s * expand_dot(zr, Bl + (size_t)j * p.r, p.r);
            up += p.s * expand_dot(zr, Bl + (size_t)(p.I + j) * p.r, p.r);
          }
          const float hv = real ? silu_f32(gate) * up : 0.f;
          p.h_out[(size_t)row * p.I + j] = f32_to_bf16(hv);
        }
      } else {
        if (!real) continue;
        const float w = p.topk_w[pr];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int n = blockIdx.x * 64 + f * 16 + m;
          if (n >= p.N) continue;
          float v = acc[rf][f][i];
          if (l >= 0) v += p.s * expand_dot(zr, Bl + (size_t)n * p.r, p.r);
          p.d_out[(size_t)row * p.H + n] = v * w;
        }
      }
    }
}

template <int MODE, int RF>
void launch_t(const GemmParams& gp, bool even, dim3 grid, hipStream_t st) {
  if (even)
    grouped_gemm_kernel<MODE, RF, true><<<grid, 256, 0, st>>>(gp);
  else
    grouped_gemm_kernel<MODE, RF, false><<<grid, 256, 0, st>>>(gp);
}

}  // namespace

int launch_gemm(const Layout& L, int mode, const uint16_t* in, const int32_t* lora_ids,
                const float* topk_weights, const uint16_t* W, const uint16_t* B, void* ws,
                hipStream_t st) {
  WsPtrs w = ws_ptrs(ws, L);
  GemmParams gp;
  gp.in = mode == 0 ? in : w.h;
  gp.W = W;
  gp.B = B;
  gp.z = mode == 0 ? w.zgu : w.zd;
  gp.sorted = w.sorted;
  gp.bexp = w.bexp;
  gp.segstart = w.segstart;
  gp.segcnt = w.segcnt;
  gp.hdr = w.hdr;
  gp.lora_ids = lora_ids;
  gp.topk_w = topk_weights;
  gp.h_out = w.h;
  gp.d_out = w.d;
  gp.K = mode == 0 ? L.H : L.I;
  gp.N = mode == 0 ? 2 * L.I : L.H;
  gp.I = L.I;
  gp.H = L.H;
  gp.E = L.E;
  gp.L = L.L;
  gp.r = L.r;
  gp.topk = L.k;
  gp.P = (int)L.P;
  gp.bm = L.bm;
  gp.nsteps = (gp.K + 63) / 64;
  gp.s = L.s;
  if (L.bm >= 128) {
    launch_gemm_tiled(gp, mode, L.cap_rows, st);
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  const int RF = L.bm >= 64 ? 4 : L.bm / 16;
  const int MT = RF * 16;
  const int ncol = mode == 0 ? (L.I + 31) / 32 : (L.H + 63) / 64;
  dim3 grid(ncol, (unsigned)((L.cap_rows + MT - 1) / MT));
  const bool even = gp.K % 64 == 0;
  if (mode == 0) {
    if (RF == 4) launch_t<0, 4>(gp, even, grid, st);
    else if (RF == 2) launch_t<0, 2>(gp, even, grid, st);
    else launch_t<0, 1>(gp, even, grid, st);
  } else {
    if (RF == 4) launch_t<1, 4>(gp, even, grid, st);
    else if (RF == 2) launch_t<1, 2>(gp, even, grid, st);
    else launch_t<1, 1>(gp, even, grid, st);
  }
  return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

}  // namespace moelora
