// Grouped GEMM for prefill-sized batches (block_m = 256): 256 x 256 tiles.
//
// Same contract as the other two families (one GEMM per expert over its
// sorted rows; the LoRA expand z * B added to the base output in the same
// kernel -- vLLM blog "Multi-LoRA for MoE models", sections "Implementing
// multi-LoRA inference for MoE models in vLLM" and "Kernel optimizations"),
// sized for MFMA throughput rather than for a weight stream:
//
//   * a 256 x 256 tile halves the L2 -> LDS traffic per flop of a 128 x 128
//     tile (64 KB per 64-deep K step for 8.4 MFLOP);
//   * 8 wavefronts in a 2 x 4 grid, each owning 128 x 64 outputs = 4 x 2 bf16
//     MFMA 32x32x16 tiles, so each 16-byte LDS fragment read feeds two or
//     four MFMAs; the fragments of K sub-step kk+1 are read while kk
//     multiplies;
//   * A (x rows gathered by token, or h rows) and W tiles go global ->
//     registers -> LDS, double-buffered (2 x 64 KB): the loads of K step q+1
//     are in flight while step q multiplies; 16-byte chunks of each 128-byte
//     LDS row are XOR-swizzled (chunk ^ ((row >> 1) & 7)) so that fragment
//     reads and tile stores are free of bank conflicts;
//   * epilogue as in the 128 x 128 family: the expand as masked MFMAs per
//     (expert, adapter) segment with z split into bf16 hi + lo, then the SiLU
//     gate (mode 0, gate and up columns in the same lane) or the top-k weight
//     (mode 1).
// A wavefront whose 128 rows are all padding skips its MFMAs and stores.
#include "device_util.h"
#include "internal.h"

namespace moelora {

namespace {

constexpr int PBM = 256, PBN = 256, PBK = 64;
constexpr int PROW = PBK * 2;          // bytes per tile row in LDS
constexpr int PTILE = PBM * PROW;      // 32 KB (A and W tiles alike)
constexpr int PLDS = 4 * PTILE;        // two buffers of (A, W)

__device__ __forceinline__ int pswz(int row, int chunk) {
  return row * PROW + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void grouped_gemm_prefill_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, khalf = lane >> 5;
  const int mtile = blockIdx.x / p.ncol, ntc = blockIdx.x - mtile * p.ncol;
  const int row0 = mtile * PBM;
  if (row0 >= p.hdr[HDR_NUM_PADDED]) return;
  const int e = p.bexp[row0 / p.bm];

  // Output column of tile column c (0..255).  mode 0: columns [64w, 64w+64)
  // are gate j0+32w+[0,32) followed by up I+j0+32w+[0,32), j0 = 128*ntc.
  auto tile_col = [&](int c) -> int {
    if (MODE == 0) {
      const int w = c >> 6, ni = (c >> 5) & 1;
      const int j = min(ntc * 128 + w * 32 + (c & 31), p.I - 1);
      return ni ? p.I + j : j;
    }
    return min(ntc * PBN + c, p.N - 1);
  };

  // global -> LDS: chunk c = tid + 512*i (i < 4) is tile row c/8, K offset
  // 8*(c%8) (the same for every i)
  const int kc = tid & 7;
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  const uint16_t* Wexp = p.W + (size_t)e * p.N * p.K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid + 512 * i) >> 3;
    const int grow = row0 + r;
    if (MODE == 0) {
      const int pr = p.sorted[grow];
      const int t = pr < p.P ? pr / p.topk : 0;  // padding rows read token 0; output dropped
      a_src[i] = p.in + (size_t)t * p.K + kc * 8;
    } else {
      a_src[i] = p.in + (size_t)grow * p.K + kc * 8;
    }
    b_src[i] = Wexp + (size_t)tile_col(r) * p.K + kc * 8;
  }

  const int ntile = (p.K + PBK - 1) / PBK;  // the last one may be partial (masked)
  u32x4_t ra[4], rb[4];
  auto load = [&](int q) {
    const int k = q * PBK + kc * 8;
    const bool ok = k < p.K;
    const int koff = (ok ? k : p.K - 8) - kc * 8;  // clamped: always a valid address
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t va = ld16(a_src[i] + koff), vb = ld16(b_src[i] + koff);
      ra[i] = ok ? va : zero4();
      rb[i] = ok ? vb : zero4();
    }
  };
  auto store = [&](int buf) {
    char* A = smem + buf * 2 * PTILE;
    char* B = A + PTILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid + 512 * i) >> 3;
      *reinterpret_cast<u32x4_t*>(A + pswz(r, kc)) = ra[i];
      *reinterpret_cast<u32x4_t*>(B + pswz(r, kc)) = rb[i];
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  const bool live = p.sorted[row0 + wm * 128] < p.P;  // any real row in this wavefront's 128
  auto mma = [&](int buf) {
    if (!live) return;
    const char* A = smem + buf * 2 * PTILE;
    const char* B = A + PTILE;
    u32x4_t af[2][4], bf[2][2];
    auto frag = [&](int kk, int s) {
      const int ch = 2 * kk + khalf;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[s][mi] = *reinterpret_cast<const u32x4_t*>(A + pswz(wm * 128 + mi * 32 + l32, ch));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[s][ni] = *reinterpret_cast<const u32x4_t*>(B + pswz(wn * 64 + ni * 32 + l32, ch));
    };
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < PBK / 16; ++kk) {
      if (kk + 1 < PBK / 16) frag(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = mfma_32x32x16(af[kk & 1][mi], bf[kk & 1][ni], acc[mi][ni]);
    }
  };

  load(0);
  store(0);
  __syncthreads();
  for (int q = 0; q < ntile; ++q) {
    const bool more = q + 1 < ntile;
    if (more) load(q + 1);
    mma(q & 1);
    if (more) store((q + 1) & 1);
    __syncthreads();
  }
  if (!live) return;

  // LoRA expand: acc += s * z[rows of segment] * B[l][e][cols]^T per segment
  const int S = p.L + 1;
  const int wrow0 = row0 + wm * 128;
  int ncol[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) ncol[ni] = tile_col(wn * 64 + ni * 32 + l32);
  for (int l = 0; l < p.L; ++l) {
    const int cnt = p.segcnt[e * S + l];
    if (cnt == 0) continue;
    const int st = p.segstart[e * S + l];
    const int lo = max(st, wrow0), hi = min(st + cnt, wrow0 + 128);
    if (lo >= hi) continue;
    const uint16_t* Bl = p.B + ((size_t)l * p.E + e) * p.N * p.r;
    for (int q0 = 0; q0 < p.r; q0 += 16) {
      const int qa = q0 + 8 * khalf;
      const bool qok = qa < p.r;
      u32x4_t bfr[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = qok ? ld16(Bl + (size_t)ncol[ni] * p.r + qa) : zero4();
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int sub0 = wrow0 + mi * 32;
        if (sub0 >= hi || sub0 + 32 <= lo) continue;  // this 32-row block misses the segment
        const int grow = sub0 + l32;
        u32x4_t zh = zero4(), zl = zero4();
        if (qok && grow >= lo && grow < hi) {
          float zv[8];
          const float4* zp = reinterpret_cast<const float4*>(p.z + (size_t)grow * p.r + qa);
          const float4 z0 = zp[0], z1 = zp[1];
          zv[0] = p.s * z0.x; zv[1] = p.s * z0.y; zv[2] = p.s * z0.z; zv[3] = p.s * z0.w;
          zv[4] = p.s * z1.x; zv[5] = p.s * z1.y; zv[6] = p.s * z1.z; zv[7] = p.s * z1.w;
          split8(zv, zh, zl);
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          acc[mi][ni] = mfma_32x32x16(zh, bfr[ni], acc[mi][ni]);
          acc[mi][ni] = mfma_32x32x16(zl, bfr[ni], acc[mi][ni]);
        }
      }
    }
  }

  // epilogue: element v of acc[mi][ni] is row 8*(v/4) + 4*khalf + v%4 of the
  // 32-row block, column l32 of the 32-column block
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wrow0 + mi * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
      const int pr = p.sorted[row];
      if (pr >= p.P) continue;  // padding row
      if (MODE == 0) {
        const int j = ntc * 128 + wn * 32 + l32;
        if (j < p.I)
          p.h_out[(size_t)row * p.I + j] = f32_to_bf16(silu_f32(acc[mi][0][v]) * acc[mi][1][v]);
      } else {
        const float w = p.topk_w[pr];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int n = ntc * PBN + wn * 64 + ni * 32 + l32;
          if (n < p.N) p.d_out[(size_t)row * p.H + n] = acc[mi][ni][v] * w;
        }
      }
    }
}

}  // namespace

int launch_gemm_prefill(const GemmParams& gp_in, int mode, int64_t cap_rows, hipStream_t st) {
  static bool attr_set[2] = {false, false};
  GemmParams gp = gp_in;
  gp.ncol = mode == 0 ? (gp.I + 127) / 128 : (gp.N + PBN - 1) / PBN;
  gp.nrowt = (int)((cap_rows + PBM - 1) / PBM);
  const unsigned grid = (unsigned)gp.ncol * (unsigned)gp.nrowt;
  const void* fn = mode == 0 ? reinterpret_cast<const void*>(&grouped_gemm_prefill_kernel<0>)
                             : reinterpret_cast<const void*>(&grouped_gemm_prefill_kernel<1>);
  if (!attr_set[mode]) {  // more than the default 64 KB of dynamic LDS
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, PLDS) != hipSuccess)
      return MOE_LORA_EHIP;
    attr_set[mode] = true;
  }
  if (mode == 0)
    grouped_gemm_prefill_kernel<0><<<grid, 512, PLDS, st>>>(gp);
  else
    grouped_gemm_prefill_kernel<1><<<grid, 512, PLDS, st>>>(gp);
  return MOE_LORA_OK;
}

}  // namespace moelora
