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
//     LDS: tile q multiplies from one LDS buffer while tile q+1 waits in
//     registers and tile q+2 is in flight; each 128-byte LDS row stores its
//     eight 16-byte chunks XOR-swizzled (chunk ^ ((row >> 1) & 7)) so that
//     both the row-wise stores and the column-wise fragment reads avoid bank
//     conflicts; the K remainder is one masked tile;
//   * the MFMAs take the W tile as their first operand, so the accumulators
//     hold the tile transposed and each lane ends with runs of 4 adjacent
//     output columns of one row (one 8- or 16-byte store each);
//   * the expand runs as extra MFMAs over the rank dimension after the main
//     loop (lora_expand): for each (expert, adapter) segment that meets the
//     wavefront's rows, z of those rows (zero elsewhere) times the adapter's B
//     rows for the tile's columns.  z is fp32; it enters the MFMA as a bf16
//     pair hi + lo (hi = rne(z), lo = rne(z - hi)), which keeps ~16
//     significant bits of z;
//   * mode 0 pairs gate column j and up column I + j in the same lane (the
//     wavefront's 64 columns are 32 gate + 32 up), so h = silu(gate) * up is
//     formed in registers and stored bf16; mode 1 scales by the top-k weight
//     and stores fp32 d.  The rows' validity and top-k weights are staged in
//     LDS at the start.
// A wavefront whose 64 rows are all padding skips its MFMAs and stores
// (expert runs put real rows first, padding last).
#include "device_util.h"
#include "gemm_expand.h"
#include "internal.h"

namespace moelora {

namespace {

#ifndef MOELORA_TILED_ROTATE
#define MOELORA_TILED_ROTATE 0  // rotate the K-tile order per workgroup
#endif

constexpr int TBM = 128, TBN = 128, TBK = 64;
constexpr int ROW_BYTES = TBK * 2;              // one tile row in LDS
constexpr int TILE_BYTES = TBM * ROW_BYTES;     // 16 KB (A and B tiles alike)

// A 16-lane phase of a 16-byte LDS access covers 64 banks; rows are 32
// banks wide, so rows 2i and 2i+1 sit on the two bank halves and chunk c of
// row r goes to slot c ^ ((r >> 1) & 7): sixteen consecutive rows reading the
// same chunk (MFMA fragments) and two rows written chunk by chunk (tile
// stores) both hit sixteen different 4-bank groups.
#ifndef MOELORA_TILED_SWZ
#define MOELORA_TILED_SWZ 1
#endif
__device__ __forceinline__ int swz(int row, int chunk) {
#if MOELORA_TILED_SWZ
  return row * ROW_BYTES + ((chunk ^ ((row >> 1) & 7)) << 4);
#else
  return row * ROW_BYTES + ((chunk ^ (row & 7)) << 4);
#endif
}

#ifndef MOELORA_TILED_GROUP_M
#define MOELORA_TILED_GROUP_M 0  // 0: plain order; n: groups of n row tiles per XCD range
#endif

// Workgroup -> (row tile, column tile).  Consecutive workgroup ids land on
// different XCDs (each with its own L2), so ids are first regrouped so that
// every XCD owns a contiguous range of the logical order; the logical order
// then walks groups of GROUP_M row tiles column by column, so the workgroups
// that run together on one XCD share a few A tiles and a few W tiles.
__device__ __forceinline__ void tile_of(int ncol, int nrow, int* mt, int* nt) {
  const int total = ncol * nrow;
  const int id = blockIdx.x;
  if (MOELORA_TILED_GROUP_M == 0) {  // plain order: column tiles of one row tile in a row
    *mt = id / ncol;
    *nt = id - *mt * ncol;
    return;
  }
  const int per = total / 8;
  const int logical = id < per * 8 ? (id % 8) * per + id / 8 : id;
  const int GM = MOELORA_TILED_GROUP_M > 0 ? MOELORA_TILED_GROUP_M : 1;
  const int gsz = GM * ncol;
  const int g = logical / gsz, in = logical - g * gsz;
  const int first = g * GM;
  const int gm = min(GM, nrow - first);
  *mt = first + in % gm;
  *nt = in / gm;
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void grouped_gemm_tiled_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][TILE_BYTES];  // [buffer][A, W]
  __shared__ int row_ok[TBM];    // the tile's rows: real (1) or padding (0)
  __shared__ float row_w[TBM];   // and their top-k weight (mode 1)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, khalf = lane >> 5;
  int mtile, ntile_col;
  tile_of(p.ncol, p.nrowt, &mtile, &ntile_col);
  const int row0 = mtile * TBM;
  if (row0 >= p.hdr[HDR_NUM_PADDED]) return;
  const int e = p.bexp[row0 / p.bm];
  int my_ok = 0;
  float my_w = 0.f;
  if (tid < TBM) {
    const int pr = p.sorted[row0 + tid];
    my_ok = pr < p.P;
    if (MODE == 1 && my_ok) my_w = p.topk_w[pr];
  }

  // Output column of tile column c (0..127).  mode 0: columns [64*wn, 64*wn+64)
  // are gate j0+32*wn+[0,32) followed by up I+j0+32*wn+[0,32).
  auto tile_col = [&](int c) -> int {
    if (MODE == 0) {
      const int w = c >> 6, ni = (c >> 5) & 1;
      const int j = min(ntile_col * 64 + w * 32 + (c & 31), p.I - 1);
      return ni ? p.I + j : j;
    }
    return min(ntile_col * TBN + c, p.N - 1);
  };

  // global -> LDS assignment: 16-byte chunk c = tid + 256*i (i < 4) is tile
  // row c/8, K offset 8*(c%8); the same K offset for every i
  // A rows come through a buffer resource: padding rows get an offset past
  // the end and load zeros without touching memory.
  const int kc = tid & 7;
  uint32_t a_off[4];  // byte offsets into the A buffer (x or h)
  const uint16_t* b_src[4];
  const uint16_t* Wexp = p.W + (size_t)e * p.N * p.K;
  const buf_rsrc_t a_rs = make_rsrc(p.in, p.in_bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid + 256 * i) >> 3;
    const int grow = row0 + r;
    const int pr = p.sorted[grow];
    const int arow = MODE == 0 ? pr / p.topk : grow;  // x row of the token, or the h row
    a_off[i] = pr < p.P ? (uint32_t)(arow * p.K + kc * 8) * 2u : kBufNone;
    b_src[i] = Wexp + (size_t)tile_col(r) * p.K + kc * 8;
  }

  // K tiles: the full 64-wide tiles (optionally in an order rotated per
  // workgroup, which spreads HBM channels but desynchronises workgroups that
  // share an A or W tile in L2), then the remainder tile (K % 64, a multiple
  // of 8) masked
  const int nfull = p.K / TBK, krem = p.K - nfull * TBK;
  const int ntile = nfull + (krem ? 1 : 0);
  const int rot = (MOELORA_TILED_ROTATE && nfull) ? (int)((ntile_col * 7u + mtile * 3u) % (unsigned)nfull) : 0;
  auto tile_k0 = [&](int q) { return q < nfull ? ((q + rot) % nfull) * TBK : nfull * TBK; };

  // two register stages; loads are unconditional (a remainder piece past K
  // reads a clamped address and is replaced by zeros) so that waiting for
  // one stage never drains the other
  u32x4_t ra[2][4], rb[2][4];
  auto load = [&](int q, int set) {
    const int k = tile_k0(q) + kc * 8;
    const bool ok = k < p.K;
    const int koff = (ok ? k : p.K - 8) - kc * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4_t va = ld16_buf(a_rs, a_off[i] + (uint32_t)koff * 2u), vb = ld16(b_src[i] + koff);
      ra[set][i] = ok ? va : zero4();
      rb[set][i] = ok ? vb : zero4();
    }
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid + 256 * i) >> 3;
      *reinterpret_cast<u32x4_t*>(&lds[buf][0][swz(r, kc)]) = ra[set][i];
      *reinterpret_cast<u32x4_t*>(&lds[buf][1][swz(r, kc)]) = rb[set][i];
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
  auto mma = [&](int buf) {
    if (!live) return;
#pragma unroll
    for (int kk = 0; kk < TBK / 16; ++kk) {
      const int ch = 2 * kk + khalf;
      u32x4_t af[2], bf[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const u32x4_t*>(&lds[buf][0][swz(wm * 64 + mi * 32 + l32, ch)]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *reinterpret_cast<const u32x4_t*>(&lds[buf][1][swz(wn * 64 + ni * 32 + l32, ch)]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma_32x32x16(bf[ni], af[mi], acc[mi][ni]);
    }
  };

  // pipeline: tile q multiplies from LDS buffer q&1 while tile q+1 waits in
  // registers and tile q+2 is being loaded
  load(0, 0);
  if (ntile > 1) load(1, 1);
  store(0, 0);
  if (tid < TBM) {
    row_ok[tid] = my_ok;
    row_w[tid] = my_w;
  }
  __syncthreads();
  int q = 0;
  for (; q + 3 < ntile; q += 2) {  // steady state, two tiles per trip (static register sets)
    load(q + 2, 0);
    mma(0);
    store(1, 1);
    __syncthreads();
    load(q + 3, 1);
    mma(1);
    store(0, 0);
    __syncthreads();
  }
  // the last (at most three) tiles; q is even here
  if (q + 2 < ntile) {
    load(q + 2, 0);
    mma(0);
    store(1, 1);
    __syncthreads();
    mma(1);
    store(0, 0);
    __syncthreads();
    mma(0);
  } else if (q + 1 < ntile) {
    mma(0);
    store(1, 1);
    __syncthreads();
    mma(1);
  } else {
    mma(0);
  }
  if (!live) return;

  // LoRA expand: acc += s * z[rows of segment] * B[l][e][cols]^T per segment
  const int wrow0 = row0 + wm * 64;
  int ncol[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) ncol[ni] = tile_col(wn * 64 + ni * 32 + l32);
  lora_expand<2, 2, true>(acc, p, e, wrow0, ncol);

  // epilogue: element v of acc[mi][ni] is row l32 of the 32-row block and
  // column 8*(v/4) + 4*khalf + v%4 of the 32-column block; each group of 4
  // elements is 4 adjacent outputs of one row, stored at once (N, I and H
  // are multiples of 8, so a group is in range when its first column is)
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int lrow = wm * 64 + mi * 32 + l32;
    if (!row_ok[lrow]) continue;  // padding row
    const int row = row0 + lrow;
    if (MODE == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = ntile_col * 64 + wn * 32 + 8 * g + 4 * khalf;
        if (j < p.I) {
          uint32_t hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            hv[i] = f32_to_bf16(silu_f32(acc[mi][0][4 * g + i]) * acc[mi][1][4 * g + i]);
          uint2 pk;
          pk.x = hv[0] | (hv[1] << 16);
          pk.y = hv[2] | (hv[3] << 16);
          *reinterpret_cast<uint2*>(p.h_out + (size_t)row * p.I + j) = pk;
        }
      }
    } else {
      const float w = row_w[lrow];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = ntile_col * TBN + wn * 64 + ni * 32 + 8 * g + 4 * khalf;
          if (n < p.N) {
            float4 o;
            o.x = acc[mi][ni][4 * g] * w;
            o.y = acc[mi][ni][4 * g + 1] * w;
            o.z = acc[mi][ni][4 * g + 2] * w;
            o.w = acc[mi][ni][4 * g + 3] * w;
            *reinterpret_cast<float4*>(p.d_out + (size_t)row * p.H + n) = o;
          }
        }
    }
  }
}

}  // namespace

void launch_gemm_tiled(const GemmParams& gp_in, int mode, int64_t cap_rows, hipStream_t st) {
  GemmParams gp = gp_in;
  gp.ncol = mode == 0 ? (gp.I + 63) / 64 : (gp.N + TBN - 1) / TBN;
  gp.nrowt = (int)((cap_rows + TBM - 1) / TBM);
  const unsigned grid = (unsigned)gp.ncol * (unsigned)gp.nrowt;
  if (mode == 0)
    grouped_gemm_tiled_kernel<0><<<grid, 256, 0, st>>>(gp);
  else
    grouped_gemm_tiled_kernel<1><<<grid, 256, 0, st>>>(gp);
}

}  // namespace moelora
