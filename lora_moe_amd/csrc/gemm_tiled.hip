// LDS-tiled grouped GEMM for many rows per expert (prefill-sized batches),
// with the LoRA expand and the SiLU gate or the top-k weight in the epilogue.
//
// Same contract as the register-streaming family in gemm.hip (one GEMM per
// expert over its sorted rows; the expand z * B added to the base output in
// the same kernel -- vLLM blog "Multi-LoRA for MoE models", sections
// "Implementing multi-LoRA inference for MoE models in vLLM" and "Kernel
// optimizations"), organised for reuse instead of streaming:
//
//   * workgroup tile 128 rows x 128 columns, K in steps of 64; 4 wavefronts in
//     a 2 x 2 grid, each owning 64 x 64 = 2 x 2 tiles of the bf16 MFMA
//     32x32x16;
//   * A (gathered x rows or h rows) and W tiles go global -> registers ->
//     LDS, double-buffered, so the loads of step k+1 are in flight while step
//     k multiplies; each 128-byte LDS row stores its eight 16-byte chunks in
//     XOR-swizzled order (chunk ^ (row & 7)) so that both the row-wise stores
//     and the column-wise 16-byte fragment reads are free of bank conflicts;
//   * the expand runs as extra MFMAs over the rank dimension after the main
//     loop: for each (expert, adapter) segment that meets the wavefront's rows,
//     the A operand is z of those rows (zero elsewhere) and the B operand the
//     adapter's B rows for the tile's columns.  z is fp32; it enters the MFMA
//     as a bf16 pair hi + lo (hi = rne(z), lo = rne(z - hi)), which keeps ~16
//     significant bits of z;
//   * mode 0 pairs gate column j and up column I + j in the same lane (the
//     wavefront's 64 columns are 32 gate + 32 up), so h = silu(gate) * up is
//     formed in registers and stored bf16; mode 1 scales by the top-k weight
//     and stores fp32 d.
// A wavefront whose 64 rows are all padding skips its MFMAs and stores
// (expert runs put real rows first, padding last).
#include "device_util.h"
#include "internal.h"

namespace moelora {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D(32x32, fp32) += A(32x16) * B(16x32), bf16.  Lane l supplies
// A[m = l%32][k = 8*(l/32) .. +8] and B[k = 8*(l/32) .. +8][n = l%32] and
// receives D[8*(v/4) + 4*(l/32) + v%4][l%32] in element v = 0..15.
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int TBM = 128, TBN = 128, TBK = 64;
constexpr int ROW_BYTES = TBK * 2;              // one tile row in LDS
constexpr int TILE_BYTES = TBM * ROW_BYTES;     // 16 KB (A and B tiles alike)

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ (row & 7)) << 4);
}

// 8 fp32 values -> bf16 hi and lo parts, packed two per word
__device__ __forceinline__ void split8(const float* v, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    const uint16_t l0 = f32_to_bf16(v[2 * i] - bf16_to_f32(h0));
    const uint16_t l1 = f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1));
    hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
}

template <int MODE, bool EVEN>
__global__ __launch_bounds__(256, 2) void grouped_gemm_tiled_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][TILE_BYTES];  // [buffer][A, W]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, khalf = lane >> 5;
  const int row0 = blockIdx.y * TBM;
  if (row0 >= p.hdr[HDR_NUM_PADDED]) return;
  const int e = p.bexp[row0 / p.bm];

  // Output column of tile column c (0..127).  mode 0: columns [64*wn, 64*wn+64)
  // are gate j0+32*wn+[0,32) followed by up I+j0+32*wn+[0,32).
  auto tile_col = [&](int c) -> int {
    if (MODE == 0) {
      const int w = c >> 6, ni = (c >> 5) & 1;
      const int j = min(blockIdx.x * 64 + w * 32 + (c & 31), p.I - 1);
      return ni ? p.I + j : j;
    }
    return min(blockIdx.x * TBN + c, p.N - 1);
  };

  // global -> LDS assignment: 16-byte chunk c = tid + 256*i (i < 4) is tile
  // row c/8, K offset 8*(c%8); the same K offset for every i
  const int kc = tid & 7;
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  const uint16_t* Wexp = p.W + (size_t)e * p.N * p.K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid + 256 * i) >> 3;
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

  u32x4_t ra[4], rb[4];
  auto load = [&](int kt) {
    const int k = kt * TBK;
    const bool ok = EVEN || k + kc * 8 < p.K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ok ? ld16(a_src[i] + k) : zero4();
      rb[i] = ok ? ld16(b_src[i] + k) : zero4();
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid + 256 * i) >> 3;
      *reinterpret_cast<u32x4_t*>(&lds[buf][0][swz(r, kc)]) = ra[i];
      *reinterpret_cast<u32x4_t*>(&lds[buf][1][swz(r, kc)]) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  const bool live = p.sorted[row0 + wm * 64] < p.P;  // any real row in this wavefront's 64
  const int nkt = (p.K + TBK - 1) / TBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) load(kt + 1);
    if (live) {
#pragma unroll
      for (int kk = 0; kk < TBK / 16; ++kk) {
        const int ch = 2 * kk + khalf;
        u32x4_t af[2], bf[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          af[mi] = *reinterpret_cast<const u32x4_t*>(&lds[cur][0][swz(wm * 64 + mi * 32 + l32, ch)]);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bf[ni] = *reinterpret_cast<const u32x4_t*>(&lds[cur][1][swz(wn * 64 + ni * 32 + l32, ch)]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma_32x32x16(af[mi], bf[ni], acc[mi][ni]);
      }
    }
    if (kt + 1 < nkt) store(cur ^ 1);
    __syncthreads();
  }
  if (!live) return;

  // LoRA expand: acc += s * z[rows of segment] * B[l][e][cols]^T per segment
  const int S = p.L + 1;
  const int wrow0 = row0 + wm * 64;
  int ncol[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) ncol[ni] = tile_col(wn * 64 + ni * 32 + l32);
  for (int l = 0; l < p.L; ++l) {
    const int cnt = p.segcnt[e * S + l];
    if (cnt == 0) continue;
    const int st = p.segstart[e * S + l];
    const int lo = max(st, wrow0), hi = min(st + cnt, wrow0 + 64);
    if (lo >= hi) continue;
    const uint16_t* Bl = p.B + ((size_t)l * p.E + e) * p.N * p.r;
    for (int q0 = 0; q0 < p.r; q0 += 16) {
      const int qa = q0 + 8 * khalf;
      const bool qok = qa < p.r;
      u32x4_t bfr[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = qok ? ld16(Bl + (size_t)ncol[ni] * p.r + qa) : zero4();
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
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
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wrow0 + mi * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
      const int pr = p.sorted[row];
      if (pr >= p.P) continue;  // padding row
      if (MODE == 0) {
        const int j = blockIdx.x * 64 + wn * 32 + l32;
        if (j < p.I)
          p.h_out[(size_t)row * p.I + j] = f32_to_bf16(silu_f32(acc[mi][0][v]) * acc[mi][1][v]);
      } else {
        const float w = p.topk_w[pr];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int n = blockIdx.x * TBN + wn * 64 + ni * 32 + l32;
          if (n < p.N) p.d_out[(size_t)row * p.H + n] = acc[mi][ni][v] * w;
        }
      }
    }
}

}  // namespace

void launch_gemm_tiled(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st) {
  const int ncol = mode == 0 ? (gp.I + 63) / 64 : (gp.N + TBN - 1) / TBN;
  dim3 grid(ncol, (unsigned)((cap_rows + TBM - 1) / TBM));
  const bool even = gp.K % TBK == 0;
  if (mode == 0) {
    if (even) grouped_gemm_tiled_kernel<0, true><<<grid, 256, 0, st>>>(gp);
    else grouped_gemm_tiled_kernel<0, false><<<grid, 256, 0, st>>>(gp);
  } else {
    if (even) grouped_gemm_tiled_kernel<1, true><<<grid, 256, 0, st>>>(gp);
    else grouped_gemm_tiled_kernel<1, false><<<grid, 256, 0, st>>>(gp);
  }
}

}  // namespace moelora
