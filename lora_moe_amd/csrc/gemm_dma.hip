// Grouped GEMM with LDS-DMA staging for batches with dozens of rows per
// expert or more: tiles of 64 x 128 (block_m = 64), 128 x 128 (block_m =
// 128), 192 x 256 (block_m = 192) or 256 x 256 (block_m = 256).
//
// Same contract as the register-streaming family in gemm.hip (one GEMM per
// expert over its sorted rows; the LoRA expand z * B added to the base output
// in the same kernel -- vLLM blog "Multi-LoRA for MoE models", sections
// "Implementing multi-LoRA inference for MoE models in vLLM" and "Kernel
// optimizations"), organised for reuse of the weight tile across a tile's rows:
//
//   * BN/64 x 2 wavefronts, each owning (BM/2) x 64 outputs = (BM/64) x 2 bf16
//     MFMA 32x32x16 tiles, so each 16-byte LDS fragment read feeds two or
//     more MFMAs; the fragments of the next 16-deep K slice are read while the
//     current one multiplies;
//   * A (x rows gathered by token, or h rows) and W tiles are copied global ->
//     LDS by the load unit itself (16 bytes per lane), into a ring of NS
//     stages of BK-deep K slices: NS - 1 stages are in flight while one
//     multiplies, without holding tiles in registers.  A stage is released by
//     a single workgroup barrier per K step, placed after the last fragment
//     read of the stage and before the last MFMAs that use it;
//   * A and W rows come through buffer resources (a 32-bit offset per lane;
//     the host keeps an expert's W below 2 GB here): padding rows (past an
//     expert's real pairs) get an offset past the end and copy zeros without
//     touching memory;
//   * a row tile that is its expert's only one reads the weight tile
//     non-temporally (it is not reused by another row tile);
//   * 16-byte chunks of each LDS row are XOR-swizzled so that fragment reads
//     are free of bank conflicts; since the load unit writes 16 consecutive
//     bytes per lane, the swizzle is applied on the global side (each lane
//     fetches the chunk that belongs at its LDS slot);
//   * the MFMAs take the W tile as their first operand, so the accumulator
//     holds the tile transposed: each lane ends with runs of 4 adjacent output
//     columns of one row, written with one 8-byte (h, bf16) or 16-byte (d,
//     fp32) store;
//   * the LoRA expand adds s*z*B^T on the same accumulators, in one of two
//     forms: as extra K stages through the ring (XD: 64-deep stages over the
//     (expert, adapter) segments that meet the row tile, 64 ranks of one
//     segment or several smaller-rank segments side by side; z rows of the
//     segment on the A side, its B rows on the W side), or
//     from registers as masked MFMAs per segment (gemm_expand.h: work items
//     inside the K loop, the rest after it);
//   * epilogue: the SiLU gate (mode 0, gate and up columns in the same lane)
//     or the top-k weight (mode 1); the rows' validity and weights are staged
//     in LDS at the start.
// A wavefront whose rows are all padding skips its MFMAs and stores but still
// copies its share of every stage.  Row tiles with few real rows (at most 64
// of 256, or 128 of 192) run on a ring of thin stages (those A rows + the W
// tile) that keeps two stages in flight instead of one.
#include <type_traits>

#include "device_util.h"
#include "gemm_expand.h"
#include "internal.h"

namespace moelora {

namespace {

typedef __attribute__((address_space(3))) char lds_char;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8); the fields not named are left at their maximum
constexpr int wait_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// 16-byte copy into LDS through a buffer resource over [base, base + bytes).
// (A resource built inside the kernels' generic copy lambda left this file's
// host pass without the kernels' launch stubs; built here it does not.)
__device__ __forceinline__ void buf_copy_lds(const void* base, uint32_t bytes, lds_char* dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), dst, 16, off, 0, 0, 0);
}
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Workgroup barrier without the release/acquire fence of __syncthreads (that
// fence waits for every outstanding vector load, the copies of later stages
// included).  Callers wait for their own copies and LDS writes first.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM_, int BN_, int BK_, int NS_, int TR_ = 0>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_;    // tile rows (pairs) and columns (weight rows)
  static constexpr int BK = BK_;              // K depth of one stage
  static constexpr int NS = NS_;              // stages in the LDS ring
  static constexpr int WN = BN / 64, NW = 2 * WN, NT = 64 * NW;  // wavefronts: 2 x WN
  static constexpr int MI = BM / 64, NI = 2;  // 32x32 blocks per wavefront
  static constexpr int CPR = BK / 8;          // 16-byte chunks per tile row
  static constexpr int PROW = BK * 2;         // bytes per tile row in LDS
  static constexpr int ATILE = BM * PROW;     // A tile (rows x K slice)
  static constexpr int WTILE = BN * PROW;     // W tile (weight rows x K slice)
  static constexpr int STAGE = ATILE + WTILE;
  // thin ring for row tiles with at most TR real rows (0: none): stages of
  // TR A rows and the whole W tile, three of them (two in flight) in the LDS
  // of the ring
  static constexpr int TR = TR_, TATILE = TR * PROW, TSTAGE = TATILE + WTILE;
  static constexpr int TNS = TR > 0 ? 3 : 0;
  static constexpr int RING = NS * STAGE > TNS * TSTAGE ? NS * STAGE : TNS * TSTAGE;
  static constexpr int LDS = RING + 2 * BM * 4;  // ring + per-row validity and top-k weight
  static constexpr int ROWS_PER_COPY = 1024 / PROW;
  static constexpr int AROWS = BM / NW, WROWS = BN / NW;  // tile rows each wavefront copies
  static constexpr int NCA = AROWS / ROWS_PER_COPY;       // 1 KB copies per wavefront per stage: A
  static constexpr int NCW = WROWS / ROWS_PER_COPY;       // and W
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(NCA >= 1 && NCA * ROWS_PER_COPY == AROWS && NCW * ROWS_PER_COPY == WROWS, "copy layout");
  static_assert(LDS <= 160 * 1024, "LDS ring exceeds 160 KB");
  static_assert(NS >= 2, "ring needs two stages");
  static constexpr int TNCA = TR / (NW * ROWS_PER_COPY);  // thin A copies per wavefront per stage
  static_assert(TR == 0 || (TR % 32 == 0 && TR < BM && TNCA * NW * ROWS_PER_COPY == TR), "thin ring rows");

  // chunk slot of logical chunk `chunk` in tile row `row`: consecutive 16-lane
  // phases of a fragment read cover 16 rows and all 64 banks
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row / (16 / CPR)) & (CPR - 1));
  }
  static __device__ __forceinline__ int off(int row, int chunk) { return row * PROW + (swz(row, chunk) << 4); }
};

// EVENK: K is a multiple of the stage depth, so no copy needs clamping or
// zeroing past K (and the chunk indices need not stay live in the loop).
// XD (EVENK only): the expand as extra K stages (L <= 64).
template <int MODE, class C, int WAVES_PER_SIMD, bool EVENK, bool XD>
__global__ __launch_bounds__(C::NT, WAVES_PER_SIMD) void grouped_gemm_dma_kernel(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NS = C::NS, MI = C::MI, NI = C::NI;
  constexpr int NCA = C::NCA, NCW = C::NCW, AROWS = C::AROWS, WROWS = C::WROWS;
  constexpr int RPC = C::ROWS_PER_COPY, CPR = C::CPR, PROW = C::PROW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int l32 = lane & 31, khalf = lane >> 5;
  // Tile of this workgroup.  order 1 (gate_up by default): row tile-major.
  // order 2 (down by default): workgroup i runs on XCD i mod 8, and row tile
  // m goes to XCD m mod 8 with all its column tiles, so that its A panel (h
  // rows) is fetched into one L2 only.  Down GEMMs with order 2 against
  // order 1 (two alternating runs on one box, us): GPT-OSS-like 106 -> 103,
  // Qwen3-MoE-like 212 -> 205, DeepSeek-like 3277 -> 3257; order 2 for
  // gate_up was neutral to 3 % slower.  The shape's tile_order overrides.
  int mtile, ntc;
  if (p.order == 2) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int k = j / p.ncol;
    ntc = j - k * p.ncol;
    mtile = x + 8 * k;
  } else {
    mtile = blockIdx.x / p.ncol;
    ntc = blockIdx.x - mtile * p.ncol;
  }
  const int row0 = mtile * BM;
  // (order 2 rounds the row tiles up to a multiple of 8)
  if (mtile >= p.nrowt || row0 >= p.hdr[HDR_NUM_PADDED]) return;
  int* row_ok = reinterpret_cast<int*>(smem + C::RING);
  float* row_w = reinterpret_cast<float*>(smem + C::RING + BM * 4);
  // validity and top-k weight of the tile's rows, for the epilogue
  int my_ok = 0;
  float my_w = 0.f;
  if (tid < BM) {
    const int pr = p.sorted[row0 + tid];
    my_ok = pr < p.P;
    if (MODE == 1 && my_ok) my_w = p.topk_w[pr];
  }
  const int e = p.bexp[row0 / p.bm];
  // the expert's weights are read by this row tile only (no neighbouring
  // tile of the same expert): stream them non-temporally
  const int blk = row0 / p.bm;
  const bool w_once = !(blk > 0 && p.bexp[blk - 1] == e) && !(blk + 1 < p.nrowt && p.bexp[blk + 1] == e);

  // Output column of tile column c (0..BN-1).  mode 0: columns [64w, 64w+64)
  // are gate j0+32w+[0,32) followed by up I+j0+32w+[0,32), j0 = (BN/2)*ntc.
  auto tile_col = [&](int c) -> int {
    if (MODE == 0) {
      const int w = c >> 6, ni = (c >> 5) & 1;
      const int j = min(ntc * (BN / 2) + w * 32 + (c & 31), p.I - 1);
      return ni ? p.I + j : j;
    }
    return min(ntc * BN + c, p.N - 1);
  };

  // Copies: wavefront w fills A tile rows [AROWS w, AROWS (w+1)) and W tile
  // rows [WROWS w, WROWS (w+1)), NCA and NCW copies of RPC rows each; lane l
  // lands at row R0 + l / CPR, slot l % CPR, which holds logical chunk
  // alchunk / wlchunk.
  const int lrow = lane / CPR, lslot = lane % CPR;
  uint32_t a_off[NCA];  // byte offsets into the A buffer (x or h)
  uint32_t w_off[NCW];  // byte offsets into the expert's weights (below 2^31)
  int alchunk[EVENK ? 1 : NCA], wlchunk[EVENK ? 1 : NCW];
  const uint16_t* Wexp = p.W + (size_t)e * p.N * p.K;
  // W rows come through a buffer resource too (one 32-bit offset per lane
  // instead of a 64-bit address: DeepSeek-like layer 7.93-7.98 -> 7.80-7.82
  // ms, gate_up 4.35-4.47 -> 4.24-4.26, two alternating runs on one box; the
  // host keeps an expert's W below 2 GB here)
  const buf_rsrc_t w_rs = make_rsrc(Wexp, (uint32_t)((size_t)p.N * p.K * 2));
  const buf_rsrc_t a_rs = make_rsrc(p.in, p.in_bytes);
#pragma unroll
  for (int i = 0; i < NCA; ++i) {
    const int r = wave * AROWS + i * RPC + lrow;
    const int ch = C::swz(r, lslot);  // the swizzle is an involution
    if (!EVENK) alchunk[i] = ch;
    const int grow = row0 + r;
    const int pr = p.sorted[grow];
    const int arow = MODE == 0 ? pr / p.topk : grow;  // x row of the token, or the h row
    a_off[i] = pr < p.P ? (uint32_t)(arow * p.K + ch * 8) * 2u : kBufNone;
  }
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int r = wave * WROWS + i * RPC + lrow;
    const int ch = C::swz(r, lslot);
    if (!EVENK) wlchunk[i] = ch;
    w_off[i] = ((uint32_t)tile_col(r) * (uint32_t)p.K + (uint32_t)(ch * 8)) * 2u;
  }

  // thin ring: wavefront w copies A rows [TNCA*8*w, TNCA*8*(w + 1)), W as usual
  constexpr int TNCA = C::TNCA;
  uint32_t a_off_t[TNCA > 0 ? TNCA : 1];
#pragma unroll
  for (int i = 0; i < TNCA; ++i) {
    const int r = (wave * TNCA + i) * RPC + lrow;
    const int ch = C::swz(r, lslot);
    const int pr = p.sorted[row0 + r];
    const int arow = MODE == 0 ? pr / p.topk : row0 + r;
    a_off_t[i] = pr < p.P ? (uint32_t)(arow * p.K + ch * 8) * 2u : kBufNone;
  }
  const int ntile = (p.K + BK - 1) / BK;  // the last stage may be partial
  const bool partial = !EVENK && (p.K % BK) != 0;
  // XD: after the K stages come expand stages over the (expert, adapter)
  // segments that meet the tile's rows, in ascending adapter order: a stage
  // holds 64 ranks of one segment (r >= 64: r / 64 stages per segment,
  // rounded up), or 8 / (r / 8) segments side by side (r < 64: each its r / 8
  // chunks of the 8 in a row piece).  A side: s*z of the segment's rows (bf16,
  // written by the shrink); the tile's other rows and unused chunks get an
  // offset past the end of zb and copy zeros.  W side: the segment's B rows at
  // the tile's columns.  The stages' MFMAs are the K loop's own, so the expand
  // costs stages instead of per-wavefront loads of z and B (which every
  // wavefront of a row half or column quarter repeats).  Lane g holds the
  // g-th segment's adapter, first row and row count.
  int xg_l = 0, xg_st = 0, xg_n = 0, nseg = 0, nst = ntile;  // nst: stages of the loop
  if constexpr (XD) {
    const int S = p.L + 1;
    int st = 0, cnt = 0;  // segment of adapter `lane`
    if (lane < p.L) {
      st = p.segstart[e * S + lane];
      cnt = p.segcnt[e * S + lane];
    }
    uint64_t hit = __ballot(cnt > 0 && st < row0 + BM && st + cnt > row0);
    nseg = __builtin_popcountll(hit);
    for (int g = 0; hit; ++g) {
      const int l = __builtin_ctzll(hit);
      hit &= hit - 1;
      if (lane == g) xg_l = l;
    }
    xg_st = __shfl(st, xg_l, 64);
    xg_n = __shfl(cnt, xg_l, 64);
    const int cps = p.r >> 3;  // 16-byte chunks of a segment's z row
    nst = ntile + (cps >= 8 ? nseg * ((cps + 7) >> 3) : (nseg + 8 / cps - 1) / (8 / cps));
  }
  const buf_rsrc_t z_rs = make_rsrc(XD ? (const void*)p.zb : (const void*)p.in, XD ? p.zb_bytes : p.in_bytes);
  auto issue = [&](int s, auto nt_c, auto thin_c) __attribute__((always_inline)) {
    constexpr bool NTL = decltype(nt_c)::value;
    constexpr bool THIN = decltype(thin_c)::value;
    char* A = THIN ? smem + (s % C::TNS) * C::TSTAGE : smem + (s % NS) * C::STAGE;
    char* B = A + (THIN ? C::TATILE : C::ATILE);
    if (XD && s >= ntile) {  // an expand stage
      const int j = s - ntile, cps = p.r >> 3;
      // r >= 64: ranks [64 q, 64 q + 64) of segment g (q = 0, or 1 for r = 72..128)
      const int g1 = cps > 8 ? j >> 1 : j;
      const int rc0 = cps > 8 ? (j & 1) * 8 : 0;
      const int l1 = __builtin_amdgcn_readlane(xg_l, g1), a1 = __builtin_amdgcn_readlane(xg_st, g1),
                n1 = __builtin_amdgcn_readlane(xg_n, g1);
      const int per = cps >= 8 ? 1 : 8 / cps, g0 = j * per;  // r < 64: segments g0 .. g0 + per - 1
      // segment (adapter, first row, rows; 0 rows: none) and rank chunk of
      // logical chunk ch of the stage
      auto chunk = [&](int ch, int& l, int& a, int& n, int& rc) {
        if (cps >= 8) {
          rc = rc0 + ch;
          l = l1;
          a = a1;
          n = rc < cps ? n1 : 0;
          if (rc >= cps) rc = 0;
          return;
        }
        int u = 0;
#pragma unroll
        for (int v = 1; v < 8; ++v) u += ch >= v * cps;
        rc = ch - u * cps;
        const bool ok = u < per && g0 + u < nseg;
        const int g = ok ? g0 + u : g0;  // a chunk without ranks reads the stage's first segment's B
        // the exchanges run in every lane (a lane that skips one does not
        // supply its value to the others)
        l = __shfl(xg_l, g, 64);
        a = __shfl(xg_st, g, 64);
        const int ng = __shfl(xg_n, g, 64);
        n = ok ? ng : 0;
      };
      auto ldZ = [&](int r, char* dst) {
        int l, a, n, rc;
        chunk(C::swz(r, lslot), l, a, n, rc);
        const int grow = row0 + r;
        const uint32_t off = (uint32_t)(grow - a) < (uint32_t)n ? (uint32_t)(grow * p.r + rc * 8) * 2u : kBufNone;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(z_rs, (lds_char*)dst, 16, (int)off, 0, 0, 0);
      };
      if (THIN) {
#pragma unroll
        for (int i = 0; i < TNCA; ++i) ldZ((wave * TNCA + i) * RPC + lrow, A + (wave * TNCA + i) * RPC * PROW);
      } else {
#pragma unroll
        for (int i = 0; i < NCA; ++i) ldZ(wave * AROWS + i * RPC + lrow, A + (wave * AROWS + i * RPC) * PROW);
      }
      if (cps >= 8) {  // one segment: its B rows through a buffer resource, like W
        const uint16_t* b_base = p.B + ((size_t)l1 * p.E + e) * p.N * p.r;
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
          const int r = wave * WROWS + i * RPC + lrow;
          int l, a, n, rc;
          chunk(C::swz(r, lslot), l, a, n, rc);  // a chunk without ranks: its z side is zero, any finite B will do
          buf_copy_lds(b_base, (uint32_t)(p.N * p.r * 2), (lds_char*)(B + (wave * WROWS + i * RPC) * PROW),
                       (tile_col(r) * p.r + rc * 8) * 2);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
          const int r = wave * WROWS + i * RPC + lrow;
          int l, a, n, rc;
          chunk(C::swz(r, lslot), l, a, n, rc);
          const uint16_t* Bs = p.B + ((size_t)l * p.E + e) * p.N * p.r;
          __builtin_amdgcn_global_load_lds((const void*)(Bs + (size_t)tile_col(r) * p.r + rc * 8),
                                           (lds_char*)(B + (wave * WROWS + i * RPC) * PROW), 16, 0, 0);
        }
      }
      return;  // as many copies as a K stage (the waits count them)
    }
    const int k0 = s * BK;
    // With K a multiple of the stage depth the stage's K offset is the same
    // for every lane and goes into the scalar offset operand, so a lane's
    // offsets stay fixed over the loop (DeepSeek-like layer 7.96-8.05 ->
    // 7.89-7.91 ms, two alternating runs on one box).  A padding row's
    // offset is past the end of the buffer with or without it.
    auto ldA = [&](int i) {
      const int roff = (wave * AROWS + i * RPC) * PROW;
      if constexpr (EVENK) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lds_char*)(A + roff), 16, (int)a_off[i], k0 * 2, 0, 0);
      } else {
        int koff = k0;
        if (k0 + alchunk[i] * 8 >= p.K) koff = p.K - 8 - alchunk[i] * 8;  // clamped: a valid address
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lds_char*)(A + roff), 16, (int)(a_off[i] + (uint32_t)koff * 2u),
                                                 0, 0, 0);
      }
    };
    auto ldW = [&](int i) {
      const int roff = (wave * WROWS + i * RPC) * PROW;
      // cache policy operand 2: non-temporal
      if constexpr (EVENK) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rs, (lds_char*)(B + roff), 16, (int)w_off[i], k0 * 2, 0, NTL ? 2 : 0);
      } else {
        int koff = k0;
        if (k0 + wlchunk[i] * 8 >= p.K) koff = p.K - 8 - wlchunk[i] * 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rs, (lds_char*)(B + roff), 16, (int)(w_off[i] + (uint32_t)koff * 2u),
                                                 0, 0, NTL ? 2 : 0);
      }
    };
    // all A copies of the stage, then all W copies: at 256 x 256 this order
    // ran the Qwen3-MoE-like gate_up in 273 us against 283 us with each A
    // copy followed by its W copy (three alternating runs on one box)
    if (THIN) {
#pragma unroll
      for (int i = 0; i < TNCA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lds_char*)(A + (wave * TNCA + i) * RPC * PROW), 16,
                                                 (int)a_off_t[i], k0 * 2, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < NCA; ++i) ldA(i);
    }
#pragma unroll
    for (int i = 0; i < NCW; ++i) ldW(i);
  };
  // zero this lane's chunks of stage s that lie beyond K (after they landed)
  auto zero_tail = [&](int s) {
    if constexpr (!EVENK) {
      char* A = smem + (s % NS) * C::STAGE;
      char* B = A + C::ATILE;
#pragma unroll
      for (int i = 0; i < NCA; ++i)
        if (s * BK + alchunk[i] * 8 >= p.K)
          *reinterpret_cast<u32x4_t*>(A + (wave * AROWS + i * RPC + lrow) * PROW + lslot * 16) = zero4();
#pragma unroll
      for (int i = 0; i < NCW; ++i)
        if (s * BK + wlchunk[i] * 8 >= p.K)
          *reinterpret_cast<u32x4_t*>(B + (wave * WROWS + i * RPC + lrow) * PROW + lslot * 16) = zero4();
    }
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  const int wrow = wm * (BM / 2);                    // first tile row of this wavefront
  const bool live = p.sorted[row0 + wrow] < p.P;     // any real row in this wavefront's rows
  // 32-row blocks of this wavefront that hold a real row: padding rows close
  // an expert's run, so a block holds one exactly when its first row is real
  // (block 0 does whenever the wavefront is live); the others skip their MFMAs
  bool blk_live[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    blk_live[mi] = __builtin_amdgcn_readfirstlane(p.sorted[row0 + wrow + 32 * mi] < p.P);
  u32x4_t af[2][MI], bf[2][NI];
  // THIN: the ring holds tile rows [0, TR) only; the row blocks past TR are
  // padding (their MFMAs are skipped) and at most TMI blocks are read
  constexpr int TMI = C::TR / 32 < MI ? C::TR / 32 : MI;
  auto frag = [&](int s, int kk, int set, auto thin_c) {
    constexpr bool THIN = decltype(thin_c)::value;
    const char* A = THIN ? smem + (s % C::TNS) * C::TSTAGE : smem + (s % NS) * C::STAGE;
    const char* B = A + (THIN ? C::TATILE : C::ATILE);
    const int ch = 2 * kk + khalf;
#pragma unroll
    for (int mi = 0; mi < (THIN ? TMI : MI); ++mi)
      af[set][mi] = *reinterpret_cast<const u32x4_t*>(A + C::off(wrow + mi * 32 + l32, ch));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      bf[set][ni] = *reinterpret_cast<const u32x4_t*>(B + C::off(wn * 64 + ni * 32 + l32, ch));
  };
  // The MFMAs of fragment set `set`, with the reads of the next slice's
  // fragments (stage qn, slice kkn, into the other set) issued after the
  // first of them: at that first MFMA every older read is complete, so a
  // conservative wait there costs nothing, and the reads overlap the rest.
  // The scheduling barriers keep this order (the scheduler would otherwise
  // sink the reads next to their use).
  auto step = [&](int set, bool next, int qn, int kkn, auto thin_c, auto all_c) {
    constexpr bool THIN = decltype(thin_c)::value;
    constexpr bool ALL = decltype(all_c)::value;  // every row block holds real rows
    acc[0][0] = mfma_32x32x16(bf[set][0], af[set][0], acc[0][0]);
    __builtin_amdgcn_sched_barrier(0);
    if (next) frag(qn, kkn, set ^ 1, thin_c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mi = 0; mi < (THIN ? TMI : MI); ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        if ((mi | ni) && (mi == 0 || ALL || blk_live[mi]))
          acc[mi][ni] = mfma_32x32x16(bf[set][ni], af[set][mi], acc[mi][ni]);
  };

  // The K loop, specialised on whether this wavefront multiplies (live) and
  // on the weight cache policy, so that it has no data-dependent branches
  // around LDS reads: the compiler counts outstanding LDS reads in order, and
  // a read issued on one path only makes it wait for all of them at the
  // join.  In particular the MFMAs of a stage's last K slice, issued after
  // the barrier together with the first fragment reads of the next stage,
  // must not wait for those reads.
  constexpr int KK = BK / 16;  // MFMA K slices per stage (even)
  constexpr int VM_AHEAD = (NCA + NCW) * (NS - 2) < 63 ? (NCA + NCW) * (NS - 2) : 63;
  // weight rows of the wavefront's columns (the expand's B rows)
  int ncol[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) ncol[ni] = tile_col(wn * 64 + ni * 32 + l32);
  // The expand of adapters 0..63 runs inside the K loop, one item per stage
  // (gemm_expand.h): an item loaded during stage q is multiplied after the
  // barrier of stage q + 1, by when the stage's wait has seen its loads land.
  // Only where a wavefront holds two or more row blocks (with one, the
  // 64 x 128 tile, the expand is short and the loop's extra work cost more:
  // GPT-OSS-like gate_up 240 -> 249 us), not for a K with a remainder at
  // 256 x 256 (the clamped copies need the registers), and only when the
  // items fit in the stages give or take a few; otherwise the batched expand
  // runs after the loop (the Qwen3-MoE-like down GEMM, 12 stages for ~20
  // segments per wavefront: 183 us batched against 219 us with the leftover
  // items after the loop one round trip each).
  constexpr bool XPIPE = !XD && MI >= 2 && (EVENK || MI < 4);
  constexpr int kLeftover = 4;
  ExpandItems<MI, NI> xi;
  xi.nitems = 0;
  xi.next = 0;
  xi.lrest = 64;
  bool xpend = false;  // an item is loaded and not yet multiplied
  auto kloop = [&](auto live_c, auto nt_c, auto thin_c, auto all_c) {
    constexpr bool LIVE = decltype(live_c)::value;
    constexpr bool THIN = decltype(thin_c)::value;
    constexpr int RNS = THIN ? C::TNS : NS;  // stages in the ring
    constexpr int VMA = THIN ? (TNCA + NCW) * (C::TNS - 2) : VM_AHEAD;
    // prologue: every ring slot gets a stage; wait for stage 0
#pragma unroll
    for (int s = 0; s < RNS; ++s)
      if (s < nst) issue(s, nt_c, thin_c);
    if (LIVE && XPIPE) {
      expand_items_init(xi, p, e, row0 + wrow, 0);
      // up to kLeftover items beyond the stages run one by one after the loop;
      // past that, the whole segments that fit the stages run in the loop
      // and the rest batched after it (Qwen3-MoE-like gate_up, 32 stages for
      // ~32 items per wavefront: 247 -> 238 us)
      if (xi.nitems > ntile - 1 + kLeftover) expand_items_cap(xi, p, 0, ntile - 1);
      if (xi.nitems > 0) {
        expand_item_load(xi, p, e, row0 + wrow, 0, ncol);
        xpend = true;
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    if (tid < BM) {
      row_ok[tid] = my_ok;
      row_w[tid] = my_w;
    }
    if (partial && ntile == 1) zero_tail(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    stage_barrier();
    if (LIVE) frag(0, 0, 0, thin_c);
    for (int q = 0; q + 1 < nst; ++q) {
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk)
        if (LIVE) step(kk & 1, true, q, kk + 1, thin_c, all_c);
      // own copies of stage q + 1 have landed (later stages may still fly);
      // the wait stays behind this stage's MFMAs
      __builtin_amdgcn_sched_barrier(0);
      if (q + RNS - 1 < nst)
        __builtin_amdgcn_s_waitcnt(wait_vm(VMA));
      else
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
      if (partial && q + 1 == ntile - 1) zero_tail(q + 1);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // fragment reads of stage q and zero writes done
      stage_barrier();
      auto xitem = [&]() __attribute__((always_inline)) {
        if (LIVE && xpend) {
          expand_item_mfma(xi, acc, row0 + wrow);
          xpend = xi.next < xi.nitems;
          if (xpend) expand_item_load(xi, p, e, row0 + wrow, 0, ncol);
        }
      };
      if constexpr (THIN) {
        // the item's loads go before the copies, so that the wait above
        // (which lets the youngest stage's copies fly) counts only copies
        xitem();
        if (q + RNS < nst) issue(q + RNS, nt_c, thin_c);  // into the slot stage q just released
      } else {
        // the second row half's wavefronts (the other wavefront on each
        // SIMD) issue their copies after the slice, so that one wavefront
        // of every SIMD multiplies while the other issues
        if (!wm && q + RNS < nst) issue(q + RNS, nt_c, thin_c);
        xitem();
      }
      // last slice of stage q (its fragments are in registers), with the
      // first reads of stage q + 1
      if (LIVE) step((KK - 1) & 1, true, q + 1, 0, thin_c, all_c);
      if constexpr (!THIN) {
        if (wm && q + RNS < nst) issue(q + RNS, nt_c, thin_c);
      }
    }
    if (LIVE) {  // the last stage
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) step(kk & 1, true, nst - 1, kk + 1, thin_c, all_c);
      step((KK - 1) & 1, false, 0, 0, thin_c, all_c);
    }
  };
  typedef std::integral_constant<bool, true> yes;
  typedef std::integral_constant<bool, false> no;
  // Thin row tiles (at most TR real rows, the rest padding: an expert's
  // last tile) fetch little besides the weight tile, so the per-CU fetch
  // latency bounds them; their ring holds TR A rows per stage, which makes
  // room for three stages (two in flight).  At the DeepSeek-like shape (89
  // of 359 row tiles are thin at TR = 64) the layer went 8.50 -> 8.26 ms
  // (three alternating runs on one box, same outputs).  K without a
  // remainder only (no zero_tail).
  // Wavefronts whose row blocks all hold real rows (every wavefront of a
  // full tile) run a copy of the loop without the per-block MFMA skip: its
  // tests sat between the MFMAs of every K slice as scalar branches.
  bool all_live = true;
#pragma unroll
  for (int mi = 1; mi < MI; ++mi) all_live = all_live && blk_live[mi];
  auto run = [&](auto thin_c) {
    constexpr bool THIN = decltype(thin_c)::value;
    if (live) {
      if (!THIN && all_live) {
        if (w_once) kloop(yes(), yes(), thin_c, yes());
        else kloop(yes(), no(), thin_c, yes());
      } else {
        if (w_once) kloop(yes(), yes(), thin_c, no());
        else kloop(yes(), no(), thin_c, no());
      }
    } else {
      if (w_once) kloop(no(), yes(), thin_c, no());
      else kloop(no(), no(), thin_c, no());
    }
  };
  if constexpr (C::TR > 0) {
    if (EVENK && p.sorted[row0 + C::TR] >= p.P) run(yes());
    else run(no());
  } else {
    run(no());
  }
  if (!live) return;

  // LoRA expand: acc += s * z[rows of segment] * B[l][e][cols]^T per
  // segment -- the items the K loop had no stage left for, then adapters 64
  // and up
  while (xpend) {
    expand_item_mfma(xi, acc, row0 + wrow);
    xpend = xi.next < xi.nitems;
    if (xpend) expand_item_load(xi, p, e, row0 + wrow, 0, ncol);
  }
  const int lstart = XD ? p.L : XPIPE ? xi.lrest : 0;  // adapters the loop has not expanded
  if (lstart < p.L) lora_expand<MI, NI, true, (MI <= 3 ? 8 : 4)>(acc, p, e, row0 + wrow, ncol, lstart);

  // epilogue: the products were formed as W x A^T, so element v of
  // acc[mi][ni] is row l32 of the 32-row block and column
  // 8*(v/4) + 4*khalf + v%4 of the 32-column block: each group of 4
  // consecutive elements is 4 adjacent outputs of one row, stored at once
  // (N, I and H are multiples of 8, so a group is in range when its first
  // column is)
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int lr = wrow + mi * 32 + l32;
    if (!row_ok[lr]) continue;  // padding row
    const int row = row0 + lr;
    if (MODE == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = ntc * (BN / 2) + wn * 32 + 8 * g + 4 * khalf;
        if (j < p.I) {
          uint32_t hv[4], lv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = silu_f32(acc[mi][0][4 * g + i]) * acc[mi][1][4 * g + i];
            hv[i] = f32_to_bf16(v);
            lv[i] = f32_to_bf16(v - bf16_to_f32((uint16_t)hv[i]));
          }
          uint2 pk;
          pk.x = hv[0] | (hv[1] << 16);
          pk.y = hv[2] | (hv[3] << 16);
          *reinterpret_cast<uint2*>(p.h_out + (size_t)row * p.I + j) = pk;
          if (p.hlo_out) {  // deep down GEMM: h's bf16 remainder too
            pk.x = lv[0] | (lv[1] << 16);
            pk.y = lv[2] | (lv[3] << 16);
            *reinterpret_cast<uint2*>(p.hlo_out + (size_t)row * p.I + j) = pk;
          }
        }
      }
    } else {
      const float w = row_w[lr];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = ntc * BN + wn * 64 + ni * 32 + 8 * g + 4 * khalf;
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

template <class C, int WAVES_PER_SIMD>
int launch_dma(const GemmParams& gp_in, int mode, int64_t cap_rows, hipStream_t st) {
  static std::atomic<uint64_t> attr_done[6];  // per kernel: mode x (K with a remainder, even K, expand stages)
  GemmParams gp = gp_in;
  gp.ncol = mode == 0 ? (gp.I + C::BN / 2 - 1) / (C::BN / 2) : (gp.N + C::BN - 1) / C::BN;
  gp.nrowt = (int)((cap_rows + C::BM - 1) / C::BM);
  const unsigned grid = (unsigned)gp.ncol * (unsigned)(gp.order == 2 ? (gp.nrowt + 7) / 8 * 8 : gp.nrowt);
  const bool even = gp.K % C::BK == 0;
  const int kind = !even ? 0 : gp.xstages ? 2 : 1;
  const void* fn;
  if (mode == 0)
    fn = kind == 2 ? reinterpret_cast<const void*>(&grouped_gemm_dma_kernel<0, C, WAVES_PER_SIMD, true, true>)
         : kind == 1 ? reinterpret_cast<const void*>(&grouped_gemm_dma_kernel<0, C, WAVES_PER_SIMD, true, false>)
                     : reinterpret_cast<const void*>(&grouped_gemm_dma_kernel<0, C, WAVES_PER_SIMD, false, false>);
  else
    fn = kind == 2 ? reinterpret_cast<const void*>(&grouped_gemm_dma_kernel<1, C, WAVES_PER_SIMD, true, true>)
         : kind == 1 ? reinterpret_cast<const void*>(&grouped_gemm_dma_kernel<1, C, WAVES_PER_SIMD, true, false>)
                     : reinterpret_cast<const void*>(&grouped_gemm_dma_kernel<1, C, WAVES_PER_SIMD, false, false>);
  if (C::LDS > 64 * 1024) {  // more than the default 64 KB of dynamic LDS
    const int rc = ensure_dynamic_lds(fn, C::LDS, attr_done[3 * mode + kind]);
    if (rc) return rc;
  }
  if (mode == 0) {
    if (kind == 2) grouped_gemm_dma_kernel<0, C, WAVES_PER_SIMD, true, true><<<grid, C::NT, C::LDS, st>>>(gp);
    else if (kind == 1) grouped_gemm_dma_kernel<0, C, WAVES_PER_SIMD, true, false><<<grid, C::NT, C::LDS, st>>>(gp);
    else grouped_gemm_dma_kernel<0, C, WAVES_PER_SIMD, false, false><<<grid, C::NT, C::LDS, st>>>(gp);
  } else {
    if (kind == 2) grouped_gemm_dma_kernel<1, C, WAVES_PER_SIMD, true, true><<<grid, C::NT, C::LDS, st>>>(gp);
    else if (kind == 1) grouped_gemm_dma_kernel<1, C, WAVES_PER_SIMD, true, false><<<grid, C::NT, C::LDS, st>>>(gp);
    else grouped_gemm_dma_kernel<1, C, WAVES_PER_SIMD, false, false><<<grid, C::NT, C::LDS, st>>>(gp);
  }
  return MOE_LORA_OK;
}

}  // namespace

// 256 x 256 tiles, 8 wavefronts, two 64-deep stages (128 KB of LDS)
int launch_gemm_prefill(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st) {
  return launch_dma<DmaCfg<256, 256, 64, 2, 64>, 2>(gp, mode, cap_rows, st);
}

// 128 x 128 tiles, 4 wavefronts, two 64-deep stages (64 KB of LDS, two
// workgroups per CU).  Measured against 32-deep stages in a 3-stage ring with
// three workgroups per CU and a 4-stage ring with two: the 64-deep stages win
// (16-byte chunks of 128-byte row pieces instead of 64-byte ones).
int launch_gemm_dma128(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st) {
  return launch_dma<DmaCfg<128, 128, 64, 2>, 2>(gp, mode, cap_rows, st);
}

// 192 x 256 tiles, 8 wavefronts of 96 x 64 outputs, two 64-deep stages (113
// KB of LDS, one workgroup per CU).  At ~128 rows per expert (Qwen3-MoE-like
// shape: 101-160) every expert fits one tile and no wavefront is all
// padding; the layer ran 0.572-0.573 ms against 0.596 ms with 256 x 256
// tiles (two alternating runs on one box).  At the DeepSeek-like shape it was
// slower (9.24 against 9.01 ms).
int launch_gemm_dma192(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st) {
  return launch_dma<DmaCfg<192, 256, 64, 2, 128>, 2>(gp, mode, cap_rows, st);
}

// 64 x 128 tiles, 4 wavefronts of 32 x 64 outputs, two 64-deep stages (48 KB
// of LDS, three workgroups per CU).  At ~32 rows per expert (GPT-OSS-like
// shape) this ran gate_up in 208-211 us and down in 105-106 us against
// 234-239 and 140-142 us for the 128 x 128 tiles, whose second half of rows
// is padding; a 3-stage ring (two workgroups per CU) ran down in 129-130 us.
int launch_gemm_dma64(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st) {
  return launch_dma<DmaCfg<64, 128, 64, 2>, 3>(gp, mode, cap_rows, st);
}

}  // namespace moelora
