// Internal declarations shared by the HIP sources of the MoE-LoRA library.
// Not part of the public ABI (see include/moe_lora.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <atomic>
#include <stdint.h>

#include "moe_lora.h"

namespace moelora {

// ------------------------------------------------------------------ sizes

constexpr int kAlignChunk = 512;       // pairs per workgroup in the align count pass
constexpr int kAlignMaxBuckets = 14336;  // E*(L+1) limit: one int per bucket in LDS
constexpr int kHdrInts = 64;
// From this intermediate size on, h reaches the down GEMM as a bf16 pair
// hi + lo (hi = rne(h), lo = rne(h - hi)) instead of hi alone: the rounding
// of h is the largest error of the layer and grows with the down GEMM's
// depth I (in an fp64 emulation of the rounding points: 0.885 of the
// tolerance at I = 11008 and 2.41 at I = 25600 with bf16 h, 0.31 and 0.35
// with the pair; 0.29 at I = 2880)
constexpr int kHsplitMinI = 4096;

// header slots (int32) at the start of the workspace
enum { HDR_NUM_PADDED = 0, HDR_ERR = 1, HDR_NTILES = 2 };

// Workspace layout for one shape.  Every region starts on a 256-byte boundary.
struct Layout {
  int T, H, I, E, k, L, r, bm;
  float s;
  int64_t P, cap_rows, cap_blocks, NB, C, TS, max_tiles;
  int dsplit;  // K splits of the down GEMM (d holds one partial slab per split)
  int hsplit;  // h also stored as its bf16 remainder lo (I >= kHsplitMinI)
  int shrink_splits, shrink_zblocks;  // requested by the shape (0: chosen by plan_shrink)
  int tile_order;                     // requested order of the tiled GEMMs (0: per mode)
  int expand_mode;                    // requested form of the tiled GEMMs' expand (0: chosen)
  size_t off_hdr, off_sorted, off_eoff, off_segstart, off_segcnt, off_bexp, off_pos;
  size_t off_chunk, off_chunkerr, off_rank, off_tiles, off_zgu, off_zd, off_zbgu, off_zbd, off_h, off_hlo,
      off_d, total;
};

// Fills `L` from the shape; returns MOE_LORA_OK or an error code.
int make_layout(const moe_lora_shape* s, Layout* L);

// Shrink tile record: rows [row0, row0 + n) of the sorted order, all in the
// segment of (expert e, adapter l).
struct LoraTile {
  int e, l, row0, n;
};

// Device pointers derived from a workspace base and a layout.
struct WsPtrs {
  int32_t* hdr;
  int32_t* sorted;
  int32_t* eoff;
  int32_t* segstart;
  int32_t* segcnt;
  int32_t* bexp;
  int32_t* pos;
  int32_t* chunk;
  int32_t* chunkerr;
  int32_t* rank;
  LoraTile* tiles;
  float* zgu;
  float* zd;
  uint16_t* zbgu;  // bf16(s * z_gu), read by the LDS-tiled GEMMs' expand
  uint16_t* zbd;   // bf16(s * z_d)
  uint16_t* h;
  uint16_t* hlo;  // nullptr unless hsplit
  float* d;
};

inline WsPtrs ws_ptrs(void* base, const Layout& L) {
  char* b = static_cast<char*>(base);
  WsPtrs w;
  w.hdr = reinterpret_cast<int32_t*>(b + L.off_hdr);
  w.sorted = reinterpret_cast<int32_t*>(b + L.off_sorted);
  w.eoff = reinterpret_cast<int32_t*>(b + L.off_eoff);
  w.segstart = reinterpret_cast<int32_t*>(b + L.off_segstart);
  w.segcnt = reinterpret_cast<int32_t*>(b + L.off_segcnt);
  w.bexp = reinterpret_cast<int32_t*>(b + L.off_bexp);
  w.pos = reinterpret_cast<int32_t*>(b + L.off_pos);
  w.chunk = reinterpret_cast<int32_t*>(b + L.off_chunk);
  w.chunkerr = reinterpret_cast<int32_t*>(b + L.off_chunkerr);
  w.rank = reinterpret_cast<int32_t*>(b + L.off_rank);
  w.tiles = reinterpret_cast<LoraTile*>(b + L.off_tiles);
  w.zgu = reinterpret_cast<float*>(b + L.off_zgu);
  w.zd = reinterpret_cast<float*>(b + L.off_zd);
  w.zbgu = reinterpret_cast<uint16_t*>(b + L.off_zbgu);
  w.zbd = reinterpret_cast<uint16_t*>(b + L.off_zbd);
  w.h = reinterpret_cast<uint16_t*>(b + L.off_h);
  w.hlo = L.hsplit ? reinterpret_cast<uint16_t*>(b + L.off_hlo) : nullptr;
  w.d = reinterpret_cast<float*>(b + L.off_d);
  return w;
}

// Arguments of the grouped GEMM kernels (both families).
struct GemmParams {
  const uint16_t* in;      // mode 0: x [T][K]; mode 1: h [cap_rows][K]
  const uint16_t* in_lo;   // mode 1 with hsplit: h's bf16 remainder [cap_rows][K]
  uint32_t in_bytes;       // size of that buffer (< 2^31, checked by the ABI)
  const uint16_t* W;       // [E][N][K]
  const uint16_t* B;       // [L][E][N][r]
  const float* z;          // [cap_rows][r]
  const uint16_t* zb;      // [cap_rows][r] bf16(s * z) (LDS-tiled family)
  const int32_t* sorted;
  const int32_t* bexp;
  const int32_t* segstart;  // [E][L+1] first row of each (expert, slot) segment
  const int32_t* segcnt;    // [E][L+1] rows in it
  const int32_t* hdr;
  const int32_t* lora_ids;
  const float* topk_w;
  uint16_t* h_out;         // mode 0: [cap_rows][I]
  uint16_t* hlo_out;       // mode 0 with hsplit: h - rne(h), bf16 [cap_rows][I]; else nullptr
  float* d_out;            // mode 1: [cap_rows][H]
  int K, N, I, H, E, L, r, topk, P, bm, nsteps;
  int ncol, nrowt;  // tiled family: column tiles and row tiles of the launch
  int ksplit;       // streaming family, mode 1: K splits (d_out slab per split)
  int order;        // tiled family: 1 row tile-major, 2 row tiles interleaved over XCDs
  int64_t d_slab;   // elements between the d_out slabs of consecutive splits
  float s;
  int xstages;        // tiled family: the expand as extra K stages through the LDS ring
  uint32_t zb_bytes;  // size of zb in bytes (below 2^31 whenever xstages is set)
  int gbal;           // streaming family, mode 0: column groups spread evenly over gridDim.x
                      // workgroups (some wavefronts idle) instead of NWV per workgroup
};

// ------------------------------------------------------------------ stage timing

enum Stage {
  ST_ALIGN_COUNT = 0,
  ST_ALIGN_PLACE,
  ST_SHRINK_GU,
  ST_GEMM_GU,
  ST_SHRINK_DOWN,
  ST_GEMM_DOWN,
  ST_COMBINE,
  ST_ROUTE,
  ST_COUNT
};

// Stage start/stop events recorded into a caller-owned profiler (nullptr:
// nothing is recorded); a call counts once its forward is enqueued.
void prof_stage_begin(moe_lora_profiler* pr, int stage, hipStream_t st);
void prof_stage_end(moe_lora_profiler* pr, int stage, hipStream_t st);
void prof_call_done(moe_lora_profiler* pr);

// ------------------------------------------------------------------ launchers

// Raises kernel fn's dynamic-LDS limit to `bytes` on the current device (the
// attribute belongs to the device; above 64 KB it must be set before the
// launch).  `done` remembers the devices (ids < 64) already set; safe to call
// from several host threads.
inline int ensure_dynamic_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_LORA_EHIP;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return MOE_LORA_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return MOE_LORA_EHIP;
  if (bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return MOE_LORA_OK;
}


// logits != nullptr: route first (top-k and weights from logits [T][E]) into
// ids_out / w_out, then align on those ids; topk_ids is then unused.
int launch_align(const Layout& L, const int32_t* topk_ids, const int32_t* lora_ids, void* ws,
                 hipStream_t st, moe_lora_profiler* pr, const float* logits = nullptr,
                 int32_t* ids_out = nullptr, float* w_out = nullptr);
int launch_router(const Layout& L, const float* logits, int32_t* ids, float* w, hipStream_t st);

struct ShrinkPlan {
  int splits;       // K split count (1 = plain stores)
  int grid;         // workgroups (grid-stride over tiles x splits)
};
ShrinkPlan plan_shrink(const Layout& L, int K);

// The LDS-tiled GEMM of this mode (0 gate_up, 1 down) runs, and its expand
// reads z as bf16(s * z)
// An expert's weights of the GEMM of `mode` fit a buffer resource (below 2 GB),
// as the LDS-tiled GEMMs address them; larger ones run on the streaming kernel.
inline bool tiled_w_fits(const Layout& L, int mode) {
  return (mode == 0 ? 2 * (int64_t)L.I * L.H : (int64_t)L.H * L.I) * 2 < (1LL << 31);
}
inline bool tiled_expand(const Layout& L, int mode) {
  return L.bm >= 64 && !(mode == 1 && L.hsplit) && tiled_w_fits(L, mode);
}

// mode 0: gate_up shrink from x rows gathered by token; mode 1: down shrink
// from h rows.  z receives the fp32 sums; when tiled_expand(L, mode) also zb
// receives bf16(s * z).
int launch_shrink(const Layout& L, int mode, const uint16_t* in, const uint16_t* A, float* z, uint16_t* zb,
                  void* ws, hipStream_t st);

// mode 0: gate_up GEMM + expand + SiLU gate -> h; mode 1: down GEMM + expand + weight -> d
int launch_gemm(const Layout& L, int mode, const uint16_t* x, const int32_t* lora_ids,
                const float* topk_weights, const uint16_t* W, const uint16_t* B, void* ws,
                hipStream_t st);

// The LDS-DMA family (gemm_dma.hip): 256 x 256 tiles when block_m == 256,
// 128 x 128 tiles when block_m == 128.
int launch_gemm_prefill(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st);
int launch_gemm_dma128(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st);
int launch_gemm_dma64(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st);
int launch_gemm_dma192(const GemmParams& gp, int mode, int64_t cap_rows, hipStream_t st);

int launch_combine(const Layout& L, void* ws, uint16_t* y, hipStream_t st);

}  // namespace moelora
