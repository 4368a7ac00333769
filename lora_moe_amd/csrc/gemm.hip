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
// mode 0 (gate_up): a workgroup owns 8 * NWV columns j0.. of the
//   intermediate (32 or 64) and computes both the gate rows j and the up
//   rows I+j of W_gu, so the SiLU gate h = silu(gate) * up is formed in
//   registers: the lane holding gate(row, j) also holds up(row, j).  h is
//   stored bf16.
// mode 1 (down): a workgroup owns 64 output columns of one K split; the
//   epilogue adds the expand (first split only) and multiplies by the pair's
//   top-k weight; d is stored fp32, one slab per K split.
//
// This family serves small row counts per expert (block_m <= 32, decode):
// every weight byte is used by one row tile only, so the kernel is a weight
// stream and is organised around HBM efficiency -- see the kernel comment.
// Row tiles hold 16 or 32 rows of a single expert (expert runs are padded to
// block_m, the tile's row count).
#include <algorithm>
#include <type_traits>

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

// Tile: 16*RF rows x (16*NWV) weight rows per workgroup of NWV wavefronts,
// 16 weight rows per wavefront.  mode 0: wavefront w owns gate rows
// j0+8w..j0+8w+7 and the matching up rows I+j0+8w.., so one MFMA column
// fragment holds 8 gate and 8 up columns; mode 1: wavefront w owns output
// columns n0+16w..n0+16w+15.
//
// The kernel is a weight stream.  What bounds it is the rate at which each
// CU can have 128-byte lines fetched through its L1, so every byte a CU asks
// for besides the weights (the row fragments) costs weight bandwidth:
//  * each wavefront streams its 16 weight rows in chunks of KC = 128 K
//    elements; a load instruction covers 4 rows x 256 contiguous bytes (whole
//    128-byte lines), non-temporal (each weight byte is read once); each
//    chunk is written to a wavefront-private LDS slice with its 16-byte
//    pieces XOR-swizzled (piece ^ row), so the MFMA fragment reads (16 rows,
//    same K piece) spread over all banks.  The next chunk's loads are issued
//    before this chunk's MFMAs (a second chunk in flight measured no faster);
//  * the row fragments of a chunk (16*RF rows x 128 K of x gathered by
//    token, or of h) are fetched once per workgroup, one or two 16-byte
//    pieces per thread, into a double-buffered LDS tile shared by all its
//    wavefronts: fetched per wavefront they cost up to twice the weight
//    traffic when every row is real (a dense layer's 32 tokens), and halved
//    that case's speed.  So the wavefronts of a workgroup walk K together,
//    one barrier per chunk;
//  * each workgroup starts at its own K chunk and wraps around: weight rows
//    lie K*2 bytes apart, so workgroups walking K in lockstep would hit the
//    same HBM channels at once;
//  * padding rows point at the tile's first row (their outputs are dropped);
//  * steady-state loads are unconditional (full chunks; the K remainder is
//    one masked chunk at the end): a load under a branch makes the compiler
//    drain all outstanding loads before it.
// NWV = 8 (gate_up with 32-row tiles, every down GEMM) halves the
// row-fragment traffic per weight byte again: with 4 wavefronts the dense
// layer's down GEMM (32 real rows) fetched half a byte of h per weight byte
// and ran at 4 TB/s; with 8 its time fell 64 -> 58 us.  With 16-row tiles
// and 8 wavefronts each thread stages 8 bytes instead of 16.
//
// HL (mode 1 only): h arrives as a bf16 pair hi (p.in) + lo (p.in_lo) and
// each weight fragment meets both, so the product carries h to about 16
// significant bits; the lo fragments are staged beside the hi ones.
template <int MODE, int RF, int NWV, bool HL>
__global__ __launch_bounds__(64 * NWV) void grouped_gemm_kernel(GemmParams p) {
  static_assert(!HL || MODE == 1, "the hi + lo pair feeds the down GEMM only");
  constexpr int KC = 128;
  // row-fragment pieces staged per thread per chunk; with more threads than
  // 16-byte pieces (16 rows, 8 wavefronts) each thread stages 8 bytes
  constexpr bool HALF = RF * 4 < NWV;
  constexpr int XPT = HALF ? 1 : RF * 4 / NWV;
  static_assert(HALF ? RF * 8 == NWV : XPT * NWV == RF * 4, "row tile pieces must divide over the threads");
  __shared__ __attribute__((aligned(16))) uint16_t wl[NWV][16 * KC];
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][RF * 16 * KC];
  __shared__ __attribute__((aligned(16))) uint16_t xll[HL ? 2 : 1][HL ? RF * 16 * KC : 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps chunk math scalar
  const int m = lane & 15, kq = lane >> 4;
  const int row0 = blockIdx.y * (RF * 16);
  if (row0 >= p.hdr[HDR_NUM_PADDED]) return;
  // mode 1 may run on tiles smaller than block_m (h as hi + lo); padding
  // rows close an expert's run, so a tile whose first row is padding is all
  // padding and has no output
  if (MODE == 1 && p.sorted[row0] >= p.P) return;
  const int e = p.bexp[row0 / p.bm];

  // mode 0: this wavefront's column group (8 gate and 8 up columns).  With
  // gbal the ceil(I / 8) groups are spread evenly over the workgroups, up to
  // NWV each, and the wavefronts past a workgroup's count only stage row
  // fragments: a single-expert layer has one row tile, and its
  // ceil(I / 64) workgroups of 8 wavefronts (400 at I = 25600) left some
  // CUs with twice the weight bytes of others.
  int grp = (int)blockIdx.x * NWV + wave;
  bool active = true;
  if (MODE == 0 && p.gbal) {
    const int ngrp = (p.I + 7) / 8;
    const int g0 = (int)(((int64_t)blockIdx.x * ngrp) / gridDim.x);
    const int g1 = (int)(((int64_t)(blockIdx.x + 1) * ngrp) / gridDim.x);
    grp = g0 + wave;
    active = grp < g1;
  }
  // weight row held by fragment column c (0..15) of this wavefront
  auto wrow_of = [&](int c) -> int {
    if (MODE == 0) {
      const int j = min(grp * 8 + (c & 7), p.I - 1);
      return c < 8 ? j : p.I + j;
    }
    return min((int)blockIdx.x * (NWV * 16) + wave * 16 + c, p.N - 1);
  };
  const uint16_t* __restrict__ Wexp = p.W + (size_t)e * p.N * p.K;
  // instruction i covers fragment rows 4i..4i+3 (16 lanes x 16 bytes per
  // row); element offsets from the expert's base fit 32 bits
  const int piece = lane & 15;
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) woff[i] = (uint32_t)wrow_of(4 * i + (lane >> 4)) * (uint32_t)p.K;

  // staged row-fragment pieces: thread tid stages piece (tid & 15) of tile
  // rows xr[j] = (tid >> 4) + j * 4 * NWV; offsets (elements) from p.in fit
  // 32 bits (checked on the host)
  int xr[XPT];
  uint32_t aoff[XPT];
  const int xpiece = HALF ? (tid >> 1) & 15 : tid & 15;  // 16-byte piece of the chunk row
  const int xhalf = HALF ? tid & 1 : 0;                  // its 8-byte half (HALF)
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    xr[j] = HALF ? tid >> 5 : (tid >> 4) + j * 4 * NWV;
    int row = row0 + xr[j];
    int pr = p.sorted[row];
    if (pr >= p.P) {  // padding row: read the tile's first row instead
      row = row0;
      pr = p.sorted[row0];
    }
    if (MODE == 0)
      aoff[j] = (uint32_t)(pr < p.P ? pr / p.topk : 0) * (uint32_t)p.K;
    else
      aoff[j] = (uint32_t)row * (uint32_t)p.K;
  }

  // full 128-wide chunks run unmasked in rotated order; a K remainder (a
  // multiple of 8 below 128) is one masked chunk at the end.  With K splits
  // (mode 1, blockIdx.z) this workgroup takes chunks [kc0, kc0 + nfull) and
  // the last split also the remainder.
  const int split = MODE == 1 ? (int)blockIdx.z : 0;
  const int all_full = p.K / KC;
  const int cps = (all_full + p.ksplit - 1) / p.ksplit;
  const int kc0 = MODE == 1 ? min(all_full, split * cps) : 0;
  const int nfull = MODE == 1 ? min(all_full, kc0 + cps) - kc0 : all_full;
  const int krem = (MODE == 0 || split == p.ksplit - 1) ? p.K - all_full * KC : 0;
  const int kbase = kc0 * KC;  // first K element of this split
  const int rot = nfull ? (int)((blockIdx.x * 7u + blockIdx.y * 3u) % (unsigned)nfull) : 0;

  u32x4_t rw[4], rx[XPT], rxl[XPT];
  uint2 rxh, rxhl;  // HALF: this thread's 8 bytes (hi, lo)
  // ACT: the wavefront has a column group (every wavefront without gbal);
  // the others stage row fragments and meet the barriers only
  auto load = [&](int k0, bool masked, auto act_c) {
    constexpr bool ACT = decltype(act_c)::value;
    const bool ok = !masked || piece * 8 < krem;
    if constexpr (ACT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rw[i] = ok ? ld16_stream(Wexp + (woff[i] + (uint32_t)(kbase + k0 + piece * 8))) : zero4();
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j)
    {
      const bool okx = !masked || xpiece * 8 < krem;
      if (HALF) {
        const uint32_t o = aoff[j] + (uint32_t)(kbase + k0 + xpiece * 8 + xhalf * 4);
        rxh = okx ? *reinterpret_cast<const uint2*>(p.in + o) : make_uint2(0u, 0u);
        if (HL) rxhl = okx ? *reinterpret_cast<const uint2*>(p.in_lo + o) : make_uint2(0u, 0u);
      } else {
        const uint32_t o = aoff[j] + (uint32_t)(kbase + k0 + xpiece * 8);
        rx[j] = okx ? ld16(p.in + o) : zero4();
        if (HL) rxl[j] = okx ? ld16(p.in_lo + o) : zero4();
      }
    }
  };
  int buf = 0;
  uint16_t* slice = wl[wave];

  f32x4_t acc[RF];
#pragma unroll
  for (int rf = 0; rf < RF; ++rf) acc[rf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the chunk in registers -> LDS (weights to the wavefront's slice, row
  // pieces to this chunk's shared buffer), then the next chunk's loads are
  // issued, then one barrier and the MFMAs of this chunk.  The buffer written
  // here was last read a chunk ago, before the previous barrier.
  auto consume = [&](int next_k0, int next_kind, auto act_c) {  // kind: 0 none, 1 full, 2 masked remainder
    constexpr bool ACT = decltype(act_c)::value;
    if constexpr (ACT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int fr = 4 * i + (lane >> 4);
        *reinterpret_cast<u32x4_t*>(&slice[fr * KC + ((piece ^ fr) << 3)]) = rw[i];
      }
    }
    uint16_t* xb = xl[buf];
    uint16_t* xbl = xll[HL ? buf : 0];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int o = xr[j] * KC + ((xpiece ^ (xr[j] & 15)) << 3);
      if (HALF) {
        *reinterpret_cast<uint2*>(&xb[o + xhalf * 4]) = rxh;
        if (HL) *reinterpret_cast<uint2*>(&xbl[o + xhalf * 4]) = rxhl;
      } else {
        *reinterpret_cast<u32x4_t*>(&xb[o]) = rx[j];
        if (HL) *reinterpret_cast<u32x4_t*>(&xbl[o]) = rxl[j];
      }
    }
    buf ^= 1;
    if (next_kind) load(next_k0, next_kind == 2, act_c);
    lds_barrier();
    if constexpr (!ACT) return;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t b =
          *reinterpret_cast<const u32x4_t*>(&slice[m * KC + (((4 * s + kq) ^ m) << 3)]);
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) {
        const int o = (rf * 16 + m) * KC + (((4 * s + kq) ^ m) << 3);
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xb[o]);
        acc[rf] = mfma_16x16x32(a, b, acc[rf]);
        if (HL) acc[rf] = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(&xbl[o]), b, acc[rf]);
      }
    }
  };

  auto kloop = [&](auto act_c) {
    if (nfull > 0) {
      load(rot * KC, false, act_c);
      int c = rot;
      for (int q = 0; q + 1 < nfull; ++q) {  // steady state: unconditional refills
        c = c + 1 == nfull ? 0 : c + 1;
        consume(c * KC, 1, act_c);
      }
      consume(nfull * KC, krem ? 2 : 0, act_c);
    } else {
      load(0, true, act_c);
    }
    if (krem) consume(0, 0, act_c);
  };
  if (active) {
    kloop(std::integral_constant<bool, true>());
  } else {
    kloop(std::integral_constant<bool, false>());
    return;
  }

  // epilogue: lane (m, kq) holds rows rf*16 + 4*kq + i of fragment column m,
  // i.e. weight row wrow_of(m); the expand is added per lane for that row
  const int wr = wrow_of(m);
#pragma unroll 1
  for (int rf = 0; rf < RF; ++rf)
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + rf * 16 + 4 * kq + i;
      const int pr = p.sorted[row];
      const bool real = pr < p.P;
      int l = -1;
      if (real) {
        l = p.lora_ids[pr / p.topk];
        if (!(l >= 0 && l < p.L)) l = -1;
      }
      float v = acc[rf][i];
      if (l >= 0 && split == 0)  // the expand joins the first K split only
        v += p.s * expand_dot(p.z + (size_t)row * p.r,
                              p.B + (((size_t)l * p.E + e) * p.N + wr) * p.r, p.r);
      if (MODE == 0) {
        const float up = __shfl_xor(v, 8, 64);  // lane m < 8: gate; m + 8: its up
        const int j = grp * 8 + m;
        if (m < 8 && j < p.I) {
          const float hv = real ? silu_f32(v) * up : 0.f;
          const uint16_t hb = f32_to_bf16(hv);
          p.h_out[(size_t)row * p.I + j] = hb;
          if (p.hlo_out) p.hlo_out[(size_t)row * p.I + j] = f32_to_bf16(hv - bf16_to_f32(hb));
        }
      } else {
        const int n = blockIdx.x * (NWV * 16) + wave * 16 + m;
        if (real && n < p.N) p.d_out[split * p.d_slab + (size_t)row * p.H + n] = v * p.topk_w[pr];
      }
    }
}

template <int MODE, int RF, int NWV, bool HL>
void launch_nwv(const GemmParams& gp, int64_t cap_rows, hipStream_t st) {
  const int ncol = MODE == 0 ? (gp.I + NWV * 8 - 1) / (NWV * 8) : (gp.H + NWV * 16 - 1) / (NWV * 16);
  dim3 grid(ncol, (unsigned)((cap_rows + RF * 16 - 1) / (RF * 16)), MODE == 1 ? gp.ksplit : 1);
  grouped_gemm_kernel<MODE, RF, NWV, HL><<<grid, NWV * 64, 0, st>>>(gp);
}

// A single-expert gate_up whose pairs fit one 32-row tile (dense decode):
// 16-wavefront workgroups, one per CU of the MI355X's 256, each taking an
// even share (12 or 13 at I = 25600) of the ceil(I / 8) column groups.
// Dense layer (T = 32, H = 5120), gate_up with 400 workgroups of 8 against
// this (two alternating runs, us): I = 25600 109 -> 99, I = 20480 102 -> 81,
// I = 16384 (256 workgroups of 8 before) 65 -> 66.
void launch_gate_up_balanced(const GemmParams& gp_in, int64_t cap_rows, hipStream_t st) {
  constexpr int NWV = 16, kCUs = 256;
  GemmParams gp = gp_in;
  gp.gbal = 1;
  const int ngrp = (gp.I + 7) / 8;
  const int G = std::max(std::min(kCUs, ngrp), (ngrp + NWV - 1) / NWV);  // at most NWV groups each
  dim3 grid(G, (unsigned)((cap_rows + 31) / 32), 1);
  grouped_gemm_kernel<0, 2, NWV, false><<<grid, NWV * 64, 0, st>>>(gp);
}

template <int MODE, int RF, bool HL = false>
void launch_rf(const GemmParams& gp, int64_t cap_rows, hipStream_t st) {
  // 8 wavefronts (128 weight rows) share each tile's staged fragments, except
  // gate_up's 16-row tiles (measured: 233 -> 236 us with 8 at the decode
  // shape, while the down GEMM there went 120 -> 117 us)
  constexpr int NWV = MODE == 0 ? 4 * RF : 8;
  launch_nwv<MODE, RF, NWV, HL>(gp, cap_rows, st);
}

}  // namespace

int launch_gemm(const Layout& L, int mode, const uint16_t* in, const int32_t* lora_ids,
                const float* topk_weights, const uint16_t* W, const uint16_t* B, void* ws,
                hipStream_t st) {
  WsPtrs w = ws_ptrs(ws, L);
  GemmParams gp;
  gp.in = mode == 0 ? in : w.h;
  gp.in_lo = mode == 1 ? w.hlo : nullptr;
  gp.hlo_out = mode == 0 ? w.hlo : nullptr;
  gp.in_bytes = (uint32_t)((mode == 0 ? L.T * (int64_t)L.H : L.cap_rows * (int64_t)L.I) * 2);
  gp.W = W;
  gp.B = B;
  gp.z = mode == 0 ? w.zgu : w.zd;
  gp.zb = mode == 0 ? w.zbgu : w.zbd;
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
  gp.ksplit = mode == 1 ? L.dsplit : 1;
  gp.order = L.tile_order ? L.tile_order : (mode == 0 ? 1 : 2);
  gp.d_slab = L.cap_rows * (int64_t)L.H;
  gp.s = L.s;
  gp.gbal = 0;
  // the LDS-tiled GEMMs' expand as extra K stages (gemm_dma.hip) where the
  // adapters fit one lane each (L <= 64), K has no remainder and zb is
  // addressable through a buffer resource; by default from rank 32 on (at
  // most two segments share a stage), where it was measured faster (flushed
  // medians, one box, register expand -> stages): DeepSeek-like layer (r =
  // 64) 8.27 -> 8.04 ms at 256 x 256 tiles, 8.72 -> 8.54 at 192 x 256, 9.28
  // -> 8.98 at 128 x 128; GPT-OSS-like (r = 32, 64 x 128) 0.398 -> 0.391 ms.
  // At rank 16 four segments share a stage, and the Qwen3-MoE-like layer's
  // ~30 segments per 192-row tile made it slower (0.582 -> 0.624 ms).
  // expand_mode 1 keeps the register expand, 2 asks for the stages at any rank.
  const int64_t zb_bytes = L.cap_rows * (int64_t)L.r * 2;
  gp.zb_bytes = (uint32_t)std::min<int64_t>(zb_bytes, 0x7fffffff);
  const bool want_stages = L.expand_mode == 2 || (L.expand_mode == 0 && L.r >= 32);
  gp.xstages = want_stages && L.L <= 64 && gp.K % 64 == 0 && zb_bytes < (1LL << 31);
  if (mode == 1 && L.hsplit) {
    // h as hi + lo: the streaming kernel, on 16-row tiles at block_m 16 and
    // 32-row tiles otherwise (block_m is a multiple of 32 then)
    if (L.bm >= 32) launch_rf<1, 2, true>(gp, L.cap_rows, st);
    else launch_rf<1, 1, true>(gp, L.cap_rows, st);
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  // the LDS-tiled GEMMs address an expert's weights (and the A rows) through
  // buffer resources, whose offsets stay below 2 GB; an expert whose W is
  // larger runs on the streaming kernel (32-row tiles, block_m >= 64 is a
  // multiple of 32)
  if (L.bm >= 64 && !tiled_w_fits(L, mode)) {
    if (mode == 0) launch_rf<0, 2>(gp, L.cap_rows, st);
    else launch_rf<1, 2>(gp, L.cap_rows, st);
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  if (L.bm == 192) {
    const int rc = launch_gemm_dma192(gp, mode, L.cap_rows, st);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  if (L.bm >= 256) {
    const int rc = launch_gemm_prefill(gp, mode, L.cap_rows, st);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  if (L.bm >= 128) {
    const int rc = launch_gemm_dma128(gp, mode, L.cap_rows, st);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  if (L.bm == 64) {
    const int rc = launch_gemm_dma64(gp, mode, L.cap_rows, st);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  // 16- or 32-row tiles
  const int RF = L.bm >= 32 ? 2 : 1;
  if (mode == 0) {
    if (RF == 2 && L.E == 1 && L.P <= 32) launch_gate_up_balanced(gp, L.cap_rows, st);
    else if (RF == 2) launch_rf<0, 2>(gp, L.cap_rows, st);
    else launch_rf<0, 1>(gp, L.cap_rows, st);
  } else {
    if (RF == 2) launch_rf<1, 2>(gp, L.cap_rows, st);
    else launch_rf<1, 1>(gp, L.cap_rows, st);
  }
  return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

}  // namespace moelora
