// LoRA shrink: z[row][q] = sum_i in[row][i] * A[l][e][q][i]  (h_in -> r).
//
// The pages' shrink computes z = xA with A of shape h_in x r (vLLM blog
// "Multi-LoRA for MoE models", section "Implementing multi-LoRA inference for
// MoE models in vLLM").  Each of the r outputs is a long sum over h_in while
// there are only a few dozen outputs, so the sum is split over K across
// workgroups and the partial sums are combined with relaxed atomic adds
// (section "Kernel optimizations", split-K).  Reading A so that neighbouring
// output columns share cache lines is the pages' CTA-swizzle concern; here A
// is stored [r][h_in] and one workgroup reads whole [r x K-slice] slabs of it,
// every row as contiguous 32-byte pieces per lane.
//
// One work item = (tile of <= 16*RFS rows of one (expert, adapter) segment,
// K split, block of z columns: all r, or 16 when work items are few).  A workgroup of 4 wavefronts walks the split's 64-wide K steps
// interleaved by wavefront, issuing the loads of 2 or 4 of its steps before
// their MFMAs; each wavefront accumulates the whole tile
// [16*RFS x 16*NFR] with bf16 MFMA 16x16x32.  The four partial tiles are added
// through LDS, then one wavefront stores (single split) or atomically adds
// (several splits) into z.  mode 0 gathers the input rows of x by token
// (gate_up shrink); mode 1 reads the SiLU-gate output h by row (down shrink).
#include <algorithm>

#include "device_util.h"
#include "internal.h"

namespace moelora {

namespace {

struct ShrinkParams {
  const uint16_t* in;  // mode 0: x [T][K]; mode 1: h [cap_rows][K]
  const uint16_t* A;   // [L][E][r][K]
  const int32_t* sorted;
  const LoraTile* tiles;
  const int32_t* hdr;
  float* z;            // [cap_rows][r]
  uint16_t* zb;        // [cap_rows][r] bf16(s * z), or nullptr
  float s;
  int K, E, r, topk, splits, steps_per_split, nsteps, use_atomic;
  int ncb, cpb;        // column blocks per tile, z columns per block
};

// U = K steps of one wavefront whose loads are issued together before their
// MFMAs (registers: U * 2 * (RFS + NFR) 16-byte fragments); the host picks
// it from the steps each wavefront has, up to this register bound
template <int RFS, int NFR>
constexpr int shrink_max_unroll() { return RFS + NFR <= 3 ? 4 : RFS + NFR <= 5 ? 2 : 1; }

template <int MODE, int RFS, int NFR, bool EVEN, int U>
__global__ __launch_bounds__(256) void lora_shrink_kernel(ShrinkParams p) {
  __shared__ float red[2][RFS * 16][NFR * 16 + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, kq = lane >> 4;
  const int nitems = p.hdr[HDR_NTILES] * p.splits * p.ncb;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int cb = item % p.ncb, rest = item / p.ncb;
    const int ti = rest / p.splits, sp = rest - ti * p.splits;
    const int q0 = cb * p.cpb;  // first z column of this item
    const LoraTile tl = p.tiles[ti];

    const uint16_t* arow[RFS];
#pragma unroll
    for (int rf = 0; rf < RFS; ++rf) {
      const int row = tl.row0 + min(rf * 16 + m, tl.n - 1);  // rows past the tile repeat a valid one
      if (MODE == 0) {
        const int t = p.sorted[row] / p.topk;
        arow[rf] = p.in + (size_t)t * p.K;
      } else {
        arow[rf] = p.in + (size_t)row * p.K;
      }
    }
    const uint16_t* brow[NFR];
#pragma unroll
    for (int nf = 0; nf < NFR; ++nf) {
      const int q = min(q0 + nf * 16 + m, p.r - 1);  // columns past r repeat a valid one
      brow[nf] = p.A + (((size_t)tl.l * p.E + tl.e) * p.r + q) * p.K;
    }

    f32x4_t acc[RFS][NFR];
#pragma unroll
    for (int rf = 0; rf < RFS; ++rf)
#pragma unroll
      for (int nf = 0; nf < NFR; ++nf) acc[rf][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // this wavefront's steps ks0 + wave + 4j, U at a time: all loads of a
    // group are issued before its MFMAs (addresses of steps past the split or
    // pieces past K are clamped to valid ones and their values zeroed, so no
    // load sits under a branch)
    const int ks0 = sp * p.steps_per_split;
    const int ks1 = min(p.nsteps, ks0 + p.steps_per_split);
    for (int ks = ks0 + wave; ks < ks1; ks += 4 * U) {
      u32x4_t a0[U][RFS], a1[U][RFS], b0[U][NFR], b1[U][NFR];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool sv = ks + 4 * u < ks1;
        const int kb = (sv ? ks + 4 * u : ks) * 64 + kq * 16;
        const bool v0 = sv && (EVEN || kb < p.K), v1 = sv && (EVEN || kb + 8 < p.K);
        const int k0 = EVEN || kb < p.K ? kb : 0, k1 = EVEN || kb + 8 < p.K ? kb + 8 : 0;
#pragma unroll
        for (int rf = 0; rf < RFS; ++rf) {
          const u32x4_t x0 = ld16(arow[rf] + k0), x1 = ld16(arow[rf] + k1);
          a0[u][rf] = v0 ? x0 : zero4();
          a1[u][rf] = v1 ? x1 : zero4();
        }
#pragma unroll
        for (int nf = 0; nf < NFR; ++nf) {
          const u32x4_t y0 = ld16(brow[nf] + k0), y1 = ld16(brow[nf] + k1);
          b0[u][nf] = v0 ? y0 : zero4();
          b1[u][nf] = v1 ? y1 : zero4();
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int rf = 0; rf < RFS; ++rf)
#pragma unroll
          for (int nf = 0; nf < NFR; ++nf) {
            acc[rf][nf] = mfma_16x16x32(a0[u][rf], b0[u][nf], acc[rf][nf]);
            acc[rf][nf] = mfma_16x16x32(a1[u][rf], b1[u][nf], acc[rf][nf]);
          }
    }

    // add the four wavefronts' partial tiles: (2,3) -> (0,1) -> 0
    if (wave >= 2) {
#pragma unroll
      for (int rf = 0; rf < RFS; ++rf)
#pragma unroll
        for (int nf = 0; nf < NFR; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wave - 2][rf * 16 + 4 * kq + i][nf * 16 + m] = acc[rf][nf][i];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int rf = 0; rf < RFS; ++rf)
#pragma unroll
        for (int nf = 0; nf < NFR; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rf][nf][i] += red[wave][rf * 16 + 4 * kq + i][nf * 16 + m];
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int rf = 0; rf < RFS; ++rf)
#pragma unroll
        for (int nf = 0; nf < NFR; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[0][rf * 16 + 4 * kq + i][nf * 16 + m] = acc[rf][nf][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int rf = 0; rf < RFS; ++rf)
#pragma unroll
        for (int nf = 0; nf < NFR; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = rf * 16 + 4 * kq + i, q = q0 + nf * 16 + m;
            if (row < tl.n && q < p.r && q < q0 + p.cpb) {
              const float v = acc[rf][nf][i] + red[0][row][nf * 16 + m];
              float* dst = p.z + (size_t)(tl.row0 + row) * p.r + q;
              if (p.use_atomic) {
                __hip_atomic_fetch_add(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              } else {
                *dst = v;
                if (p.zb) p.zb[(size_t)(tl.row0 + row) * p.r + q] = f32_to_bf16(p.s * v);
              }
            }
          }
    }
    __syncthreads();  // red is reused by the next item
  }
}

// zb = bf16(s * z) for every row, after split-K shrinks (8 values per thread)
__global__ __launch_bounds__(256) void zb_convert_kernel(const float* __restrict__ z, int64_t n8, float s,
                                                         uint16_t* __restrict__ zb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(z)[2 * i], b = reinterpret_cast<const float4*>(z)[2 * i + 1];
  u32x4_t o;
  o[0] = (uint32_t)f32_to_bf16(s * a.x) | ((uint32_t)f32_to_bf16(s * a.y) << 16);
  o[1] = (uint32_t)f32_to_bf16(s * a.z) | ((uint32_t)f32_to_bf16(s * a.w) << 16);
  o[2] = (uint32_t)f32_to_bf16(s * b.x) | ((uint32_t)f32_to_bf16(s * b.y) << 16);
  o[3] = (uint32_t)f32_to_bf16(s * b.z) | ((uint32_t)f32_to_bf16(s * b.w) << 16);
  reinterpret_cast<u32x4_t*>(zb)[i] = o;
}

template <int MODE, int RFS, int NFR, int U>
void launch_u(const ShrinkParams& sp, bool even, int grid, hipStream_t st) {
  if (even)
    lora_shrink_kernel<MODE, RFS, NFR, true, U><<<grid, 256, 0, st>>>(sp);
  else
    lora_shrink_kernel<MODE, RFS, NFR, false, U><<<grid, 256, 0, st>>>(sp);
}

template <int MODE, int RFS, int NFR>
void launch_t(const ShrinkParams& sp, bool even, int grid, hipStream_t st) {
  // steps per wavefront in one split
  const int spw = (sp.steps_per_split + 3) / 4;
  const int u = std::min(shrink_max_unroll<RFS, NFR>(), spw >= 4 ? 4 : spw >= 2 ? 2 : 1);
  constexpr int mu = shrink_max_unroll<RFS, NFR>();
  if (u >= 4) launch_u<MODE, RFS, NFR, mu>(sp, even, grid, st);
  else if (u == 2) launch_u<MODE, RFS, NFR, (mu >= 2 ? 2 : 1)>(sp, even, grid, st);
  else launch_u<MODE, RFS, NFR, 1>(sp, even, grid, st);
}

template <int MODE, int RFS>
void launch_nfr(const ShrinkParams& sp, bool even, int grid, hipStream_t st) {
  switch ((sp.cpb + 15) / 16) {
    case 1: launch_t<MODE, RFS, 1>(sp, even, grid, st); break;
    case 2: launch_t<MODE, RFS, 2>(sp, even, grid, st); break;
    case 3: launch_t<MODE, RFS, 3>(sp, even, grid, st); break;
    case 4: launch_t<MODE, RFS, 4>(sp, even, grid, st); break;
    case 5: launch_t<MODE, 1, 5>(sp, even, grid, st); break;
    case 6: launch_t<MODE, 1, 6>(sp, even, grid, st); break;
    case 7: launch_t<MODE, 1, 7>(sp, even, grid, st); break;
    default: launch_t<MODE, 1, 8>(sp, even, grid, st); break;
  }
}

}  // namespace

// Tiles are at most TS rows; ranks above 64 use 16-row tiles (LDS budget).
static int shrink_row_frags(const Layout& L) {
  if (L.r > 64) return 1;
  return (int)(L.TS / 16);
}

// Expected number of shrink tiles: at most one per touched (expert, adapter)
// segment plus one per TS adapter rows.
static int64_t shrink_tiles_est(const Layout& L) {
  return std::max<int64_t>(1, std::min<int64_t>(L.max_tiles, std::min<int64_t>(L.P, (int64_t)L.E * L.L)));
}

// Blocks of z columns per tile, each a work item of its own.  With few work
// items (under 4 per CU) each tile's columns become items of 16 columns,
// reading their own rows of A (A is [r][K]) and the tile's x rows again: the
// CUs that drew two whole tiles bound the kernel, and at the GPT-OSS-like
// shape (364 tiles, r = 32) the two shrinks went 21.4 + 22.0 -> 18.7 + 20.0 us.
static int shrink_col_blocks(const Layout& L, int splits) {
  if (L.shrink_zblocks > 0) return L.shrink_zblocks;  // set by the shape (validated: r / blocks % 8 == 0)
  return (L.r % 16 == 0 && shrink_tiles_est(L) * splits < 1024) ? L.r / 16 : 1;
}

ShrinkPlan plan_shrink(const Layout& L, int K) {
  ShrinkPlan sp;
  const int nsteps = (K + 63) / 64;
  const int64_t est = shrink_tiles_est(L);
  // K splits only while the tiles alone leave the chip short of work: with
  // 384 or more tiles (1.5 per CU) a single split measured as fast or faster
  // (no atomics, and the align then has no accumulators to clear)
  int splits = est >= 384 ? 1 : (int)std::max<int64_t>(1, 2048 / est);
  splits = std::min(splits, std::max(1, nsteps / 4));  // >= 4 steps: one per wavefront
  if (L.shrink_splits > 0) splits = std::min(L.shrink_splits, nsteps);  // set by the shape
  sp.splits = splits;
  const int64_t items = L.max_tiles * splits * shrink_col_blocks(L, splits);
  sp.grid = (int)std::max<int64_t>(1, std::min<int64_t>(items, 4096));
  return sp;
}

int launch_shrink(const Layout& L, int mode, const uint16_t* in, const uint16_t* A, float* z, uint16_t* zb,
                  void* ws, hipStream_t st) {
  WsPtrs w = ws_ptrs(ws, L);
  const int K = mode == 0 ? L.H : L.I;
  ShrinkPlan pl = plan_shrink(L, K);
  ShrinkParams sp;
  sp.in = in;
  sp.A = A;
  sp.sorted = w.sorted;
  sp.tiles = w.tiles;
  sp.hdr = w.hdr;
  sp.z = z;
  sp.K = K;
  sp.E = L.E;
  sp.r = L.r;
  sp.topk = L.k;
  sp.splits = pl.splits;
  sp.nsteps = (K + 63) / 64;
  sp.steps_per_split = (sp.nsteps + pl.splits - 1) / pl.splits;
  sp.use_atomic = pl.splits > 1;
  const bool want_zb = tiled_expand(L, mode);
  sp.zb = want_zb && !sp.use_atomic ? zb : nullptr;
  sp.s = L.s;
  sp.ncb = shrink_col_blocks(L, pl.splits);
  sp.cpb = L.r / sp.ncb;
  const bool even = (K % 64) == 0;
  const int rfs = shrink_row_frags(L);
  if (mode == 0) {
    if (rfs == 4) launch_nfr<0, 4>(sp, even, pl.grid, st);
    else if (rfs == 2) launch_nfr<0, 2>(sp, even, pl.grid, st);
    else launch_nfr<0, 1>(sp, even, pl.grid, st);
  } else {
    if (rfs == 4) launch_nfr<1, 4>(sp, even, pl.grid, st);
    else if (rfs == 2) launch_nfr<1, 2>(sp, even, pl.grid, st);
    else launch_nfr<1, 1>(sp, even, pl.grid, st);
  }
  if (want_zb && sp.use_atomic) {  // the split sums are complete only now
    const int64_t n8 = L.cap_rows * (int64_t)L.r / 8;
    zb_convert_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(z, n8, L.s, zb);
  }
  return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

}  // namespace moelora
