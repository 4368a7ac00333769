// C ABI of the MoE-LoRA library: argument checks, workspace layout, stage
// dispatch and stage timing.  Declarations and contracts: include/moe_lora.h.
#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "internal.h"

namespace moelora {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static int check_shape(const moe_lora_shape* s) {
  if (!s) return MOE_LORA_EINVAL;
  if (s->T < 0 || s->H <= 0 || s->I <= 0 || s->E <= 0 || s->topk <= 0 || s->topk > s->E ||
      s->L <= 0 || s->r <= 0)
    return MOE_LORA_EINVAL;
  const int bm = s->block_m;
  if (!(bm == 0 || bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 192 || bm == 256)) return MOE_LORA_EINVAL;
  if (s->H % 8 || s->I % 8) return MOE_LORA_EALIGN;
  if (s->r % 8 || s->r > 128) return MOE_LORA_EUNSUPPORTED;
  if ((int64_t)s->E * (s->L + 1) > kAlignMaxBuckets) return MOE_LORA_EUNSUPPORTED;
  // every index into the row-major buffers must fit the kernels' int arithmetic
  const int64_t P = (int64_t)s->T * s->topk;
  const int64_t cap = P + (int64_t)s->E * 255;
  if (P > (1LL << 30) || cap > (1LL << 30)) return MOE_LORA_EUNSUPPORTED;
  // the streaming GEMM addresses one expert's weights with 32-bit element
  // offsets; the tiled GEMMs read x and the intermediate rows through buffer
  // resources, which take byte offsets below 2^31
  const int64_t lim = 1LL << 32, blim = 1LL << 31;
  if ((int64_t)2 * s->I * s->H >= lim || (int64_t)s->T * s->H * 2 >= blim || cap * s->I * 2 >= blim)
    return MOE_LORA_EUNSUPPORTED;
  // kernel configuration (0 = chosen from the shape)
  if (s->shrink_splits < 0 || s->shrink_splits > 64) return MOE_LORA_EINVAL;
  const int zb = s->shrink_zblocks;
  if (zb < 0 || (zb > 1 && (s->r % zb || (s->r / zb) % 8))) return MOE_LORA_EINVAL;
  if (s->down_splits < 0 || s->down_splits > 64) return MOE_LORA_EINVAL;
  if (s->tile_order < 0 || s->tile_order > 2) return MOE_LORA_EINVAL;
  if (s->expand_mode < 0 || s->expand_mode > 2) return MOE_LORA_EINVAL;
  return MOE_LORA_OK;
}

static int resolve_bm(const moe_lora_shape* s) {
  if (s->block_m) return s->block_m;
  // rows per touched expert, if routing were even
  const int64_t P = (int64_t)s->T * s->topk;
  const int64_t touched = std::max<int64_t>(1, std::min<int64_t>(s->E, P));
  const int64_t rows = (P + touched - 1) / touched;
  // up to ~24 rows per expert the weight stream dominates (streaming GEMM
  // family); beyond that an LDS-tiled GEMM whose row tile holds an expert's
  // rows with about a third to spare for uneven routing (64 rows up to 48,
  // 192 rows up to 144), so that each expert's weights are read once and no
  // wavefront holds only padding rows; 128 rows in between; from ~150 rows
  // the 256 x 256 tiles, which read the gathered x rows half as often per
  // column (padding rows cost no traffic) and each expert's weights once per
  // 256 rows
  if (rows <= 16) return 16;
  if (rows <= 24) return 32;
  // few experts with wide weights (dense layers): the tiled grids would be
  // too small to fill the GPU (the down projection has one 128-column tile
  // per expert and 128 output columns), so stream instead
  if (touched * ((s->H + 127) / 128) < 512) return 32;
  if (rows <= 48) return 64;
  if (rows < 96) return 128;
  if (rows <= 144) return 192;
  return 256;
}

int make_layout(const moe_lora_shape* s, Layout* L) {
  int rc = check_shape(s);
  if (rc) return rc;
  L->T = s->T;
  L->H = s->H;
  L->I = s->I;
  L->E = s->E;
  L->k = s->topk;
  L->L = s->L;
  L->r = s->r;
  L->bm = resolve_bm(s);
  L->s = s->lora_scale;
  L->P = (int64_t)s->T * s->topk;
  L->cap_rows = L->P + (int64_t)L->E * (L->bm - 1);
  L->cap_blocks = (L->cap_rows + L->bm - 1) / L->bm;
  L->NB = (int64_t)L->E * (L->L + 1);
  L->C = std::max<int64_t>(1, (L->P + kAlignChunk - 1) / kAlignChunk);
  // shrink tile rows: 16 when (expert, adapter) segments would hold at most
  // 16 rows under even routing and adapters, else 64, so that each adapter
  // slab is read once per 64 rows (16 above rank 64: LDS budget)
  {
    const int64_t seg = (L->P + (int64_t)L->E * L->L - 1) / ((int64_t)L->E * L->L);
    L->TS = (L->r > 64 || seg <= 16) ? 16 : 64;
  }
  L->max_tiles = (L->P + L->TS - 1) / L->TS + std::min<int64_t>((int64_t)L->E * L->L, L->P);
  // The streaming down GEMM splits K when its (row tile x 64-column) grid is
  // small (few experts with wide weights, e.g. dense layers): each split
  // writes its own partial slab of d and the combine adds the slabs in order.
  L->hsplit = L->I >= kHsplitMinI;
  L->shrink_splits = s->shrink_splits;
  L->shrink_zblocks = s->shrink_zblocks;
  L->tile_order = s->tile_order;
  L->expand_mode = s->expand_mode;
  L->dsplit = 1;
  if ((L->bm <= 32 || L->hsplit) && s->down_splits > 0) {
    // the streaming down GEMM splits K in 128-wide chunks
    L->dsplit = (int)std::min<int64_t>(s->down_splits, std::max<int64_t>(1, L->I / 128));
  } else if (L->bm <= 32) {
    const int64_t tile_rows = L->bm >= 32 ? 32 : 16;
    // the split count is sized for ~1024 workgroups of an estimated tile
    // grid; at 16-row tiles it counts 64-column tiles (the measured best
    // split at the decode shape), at 32-row tiles the kernel's 128 columns
    const int64_t tile_cols = L->bm >= 32 ? 128 : 64;
    const int64_t tiles = ((L->H + tile_cols - 1) / tile_cols) * ((L->cap_rows + tile_rows - 1) / tile_rows);
    const int64_t chunks = std::max<int64_t>(1, L->I / 128);
    L->dsplit = (int)std::min<int64_t>(std::min<int64_t>(8, chunks), std::max<int64_t>(1, (1024 + tiles - 1) / tiles));
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + std::max<size_t>(bytes, 1), 256);
    return at;
  };
  L->off_hdr = take(sizeof(int32_t) * kHdrInts);
  L->off_sorted = take(sizeof(int32_t) * L->cap_rows);
  L->off_eoff = take(sizeof(int32_t) * (L->E + 1));
  L->off_segstart = take(sizeof(int32_t) * L->NB);
  L->off_segcnt = take(sizeof(int32_t) * L->NB);
  L->off_bexp = take(sizeof(int32_t) * L->cap_blocks);
  L->off_pos = take(sizeof(int32_t) * L->P);
  L->off_chunk = take(sizeof(int32_t) * L->NB * L->C);
  L->off_chunkerr = take(sizeof(int32_t) * L->C);
  L->off_rank = take(sizeof(int32_t) * L->P);
  L->off_tiles = take(sizeof(LoraTile) * L->max_tiles);
  L->off_zgu = take(sizeof(float) * L->cap_rows * L->r);
  L->off_zd = take(sizeof(float) * L->cap_rows * L->r);
  L->off_zbgu = take(sizeof(uint16_t) * L->cap_rows * L->r);
  L->off_zbd = take(sizeof(uint16_t) * L->cap_rows * L->r);
  L->off_h = take(sizeof(uint16_t) * L->cap_rows * L->I);
  L->off_hlo = L->hsplit ? take(sizeof(uint16_t) * L->cap_rows * L->I) : 0;
  L->off_d = take(sizeof(float) * L->dsplit * L->cap_rows * L->H);
  L->total = o;
  return MOE_LORA_OK;
}

}  // namespace moelora

// ------------------------------------------------------------------ stage timing

// A caller-owned recorder: events [call][stage][start, stop] and the stages
// recorded per call.
struct moe_lora_profiler {
  int max_calls = 0;
  int call = 0;
  uint32_t mask = 0;
  std::vector<hipEvent_t> ev;
  std::vector<uint32_t> recorded;
};

namespace moelora {

void prof_stage_begin(moe_lora_profiler* pr, int stage, hipStream_t st) {
  if (!pr || pr->call >= pr->max_calls || !(pr->mask & (1u << stage))) return;
  hipEventRecord(pr->ev[((size_t)pr->call * ST_COUNT + stage) * 2], st);
}

void prof_stage_end(moe_lora_profiler* pr, int stage, hipStream_t st) {
  if (!pr || pr->call >= pr->max_calls || !(pr->mask & (1u << stage))) return;
  hipEventRecord(pr->ev[((size_t)pr->call * ST_COUNT + stage) * 2 + 1], st);
  pr->recorded[pr->call] |= 1u << stage;
}

void prof_call_done(moe_lora_profiler* pr) {
  if (pr && pr->call < pr->max_calls) pr->call++;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace moelora

using namespace moelora;

extern "C" {

int moe_lora_resolve_block_m(const moe_lora_shape* shape) {
  int rc = check_shape(shape);
  return rc ? rc : resolve_bm(shape);
}

int moe_lora_tune_apply(const moe_lora_shape* shape, const moe_lora_tune_entry* table, int32_t n,
                        float max_dist, moe_lora_shape* out) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!out) return MOE_LORA_EINVAL;
  *out = *shape;
  const int64_t P = (int64_t)shape->T * shape->topk;
  const int64_t touched = std::max<int64_t>(1, std::min<int64_t>(shape->E, P));
  const double key[6] = {(double)((P + touched - 1) / touched), (double)shape->H, (double)shape->I,
                         (double)shape->E, (double)shape->r, (double)shape->L};
  const double weight[6] = {4.0, 1.0, 1.0, 1.0, 1.0, 1.0};
  int best = -1;
  double best_d = 0.0;
  for (int32_t i = 0; table && i < n; ++i) {
    const moe_lora_tune_entry& t = table[i];
    const int bm = t.block_m;
    if (bm != 16 && bm != 32 && bm != 64 && bm != 128 && bm != 192 && bm != 256) continue;
    const int32_t ek[6] = {t.rows_per_expert, t.H, t.I, t.E, t.r, t.L};
    double d = 0.0;
    bool ok = true;
    for (int j = 0; j < 6; ++j) {
      if (ek[j] <= 0) {
        ok = false;
        break;
      }
      d += weight[j] * std::fabs(std::log2(std::max(key[j], 1.0) / (double)ek[j]));
    }
    if (!ok || (max_dist > 0.f && d > (double)max_dist)) continue;
    if (best < 0 || d < best_d) {
      best = i;
      best_d = d;
    }
  }
  if (best >= 0) {
    const moe_lora_tune_entry& t = table[best];
    moe_lora_shape s2 = *shape;
    if (!s2.block_m) s2.block_m = t.block_m;
    if (!s2.shrink_splits) s2.shrink_splits = t.shrink_splits;
    if (!s2.shrink_zblocks) s2.shrink_zblocks = t.shrink_zblocks;
    if (!s2.down_splits) s2.down_splits = t.down_splits;
    if (!s2.tile_order) s2.tile_order = t.tile_order;
    if (!s2.expand_mode) s2.expand_mode = t.expand_mode;
    Layout L;
    if (make_layout(&s2, &L) == MOE_LORA_OK) *out = s2;  // else: the entry does not fit this shape
  }
  return resolve_bm(out);
}

int moe_lora_tune_block_m(const moe_lora_shape* shape, const moe_lora_tune_entry* table, int32_t n,
                          float max_dist) {
  moe_lora_shape out;
  return moe_lora_tune_apply(shape, table, n, max_dist, &out);
}

size_t moe_lora_workspace_bytes(const moe_lora_shape* shape) {
  Layout L;
  if (make_layout(shape, &L)) return 0;
  return L.total;
}

int moe_lora_workspace_view(const moe_lora_shape* shape, void* workspace, moe_lora_views* out) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (!workspace || !out) return MOE_LORA_EINVAL;
  WsPtrs w = ws_ptrs(workspace, L);
  out->sorted_ids = w.sorted;
  out->expert_off = w.eoff;
  out->seg_start = w.segstart;
  out->seg_cnt = w.segcnt;
  out->block_expert = w.bexp;
  out->pos_of_pair = w.pos;
  out->num_padded = w.hdr + HDR_NUM_PADDED;
  out->err_count = w.hdr + HDR_ERR;
  out->z_gu = w.zgu;
  out->z_down = w.zd;
  out->h = w.h;
  out->d = w.d;
  out->d_splits = L.dsplit;
  out->cap_rows = L.cap_rows;
  out->cap_blocks = L.cap_blocks;
  out->block_m = L.bm;
  out->h_lo = w.hlo;
  return MOE_LORA_OK;
}

int moe_lora_align_view(const moe_lora_shape* shape, const void* workspace, moe_lora_align_ptrs* out) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (!workspace || !out) return MOE_LORA_EINVAL;
  WsPtrs w = ws_ptrs(const_cast<void*>(workspace), L);
  out->sorted_ids = w.sorted;
  out->expert_off = w.eoff;
  out->seg_start = w.segstart;
  out->seg_cnt = w.segcnt;
  out->block_expert = w.bexp;
  out->pos_of_pair = w.pos;
  out->num_padded = w.hdr + HDR_NUM_PADDED;
  out->err_count = w.hdr + HDR_ERR;
  return MOE_LORA_OK;
}

int moe_lora_align_timed(const moe_lora_shape* shape, const int32_t* topk_ids, const int32_t* lora_ids,
                         void* workspace, size_t ws_bytes, void* stream, moe_lora_profiler* prof) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (L.T == 0) return MOE_LORA_OK;
  if (!topk_ids || !lora_ids) return MOE_LORA_EINVAL;
  if (!workspace || ws_bytes < L.total) return MOE_LORA_EWORKSPACE;
  if (!aligned16(workspace)) return MOE_LORA_EALIGN;
  return launch_align(L, topk_ids, lora_ids, workspace, (hipStream_t)stream, prof);
}

int moe_lora_align(const moe_lora_shape* shape, const int32_t* topk_ids, const int32_t* lora_ids,
                   void* workspace, size_t ws_bytes, void* stream) {
  return moe_lora_align_timed(shape, topk_ids, lora_ids, workspace, ws_bytes, stream, nullptr);
}

int moe_lora_route(const moe_lora_shape* shape, const float* logits, int32_t* topk_ids,
                   float* topk_weights, void* stream) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (L.T == 0) return MOE_LORA_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_LORA_EINVAL;
  if (L.k > 64) return MOE_LORA_EUNSUPPORTED;
  return launch_router(L, logits, topk_ids, topk_weights, (hipStream_t)stream);
}

int moe_lora_route_align_timed(const moe_lora_shape* shape, const float* logits, const int32_t* lora_ids,
                               int32_t* topk_ids, float* topk_weights, void* workspace, size_t ws_bytes,
                               void* stream, moe_lora_profiler* prof) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (L.T == 0) return MOE_LORA_OK;
  if (!logits || !lora_ids || !topk_ids || !topk_weights) return MOE_LORA_EINVAL;
  if (L.k > 64) return MOE_LORA_EUNSUPPORTED;
  if (!workspace || ws_bytes < L.total) return MOE_LORA_EWORKSPACE;
  if (!aligned16(workspace)) return MOE_LORA_EALIGN;
  return launch_align(L, topk_ids, lora_ids, workspace, (hipStream_t)stream, prof, logits, topk_ids,
                      topk_weights);
}

int moe_lora_route_align(const moe_lora_shape* shape, const float* logits, const int32_t* lora_ids,
                         int32_t* topk_ids, float* topk_weights, void* workspace, size_t ws_bytes,
                         void* stream) {
  return moe_lora_route_align_timed(shape, logits, lora_ids, topk_ids, topk_weights, workspace, ws_bytes,
                                    stream, nullptr);
}

int moe_lora_forward_timed(const moe_lora_shape* shape, const uint16_t* x, const int32_t* topk_ids,
                           const float* topk_weights, const int32_t* lora_ids, const uint16_t* W_gu,
                           const uint16_t* W_down, const uint16_t* A_gu, const uint16_t* B_gu,
                           const uint16_t* A_down, const uint16_t* B_down, void* workspace,
                           size_t ws_bytes, uint16_t* y, void* stream, moe_lora_profiler* prof) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (L.T == 0) {
    prof_call_done(prof);
    return MOE_LORA_OK;
  }
  const void* ptrs[] = {x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu, A_down, B_down, y};
  for (const void* p : ptrs)
    if (!p) return MOE_LORA_EINVAL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_LORA_EALIGN;
  if (!workspace || ws_bytes < L.total) return MOE_LORA_EWORKSPACE;
  if (!aligned16(workspace)) return MOE_LORA_EALIGN;
  hipStream_t st = (hipStream_t)stream;
  WsPtrs w = ws_ptrs(workspace, L);

  prof_stage_begin(prof, ST_SHRINK_GU, st);
  rc = launch_shrink(L, 0, x, A_gu, w.zgu, w.zbgu, workspace, st);
  prof_stage_end(prof, ST_SHRINK_GU, st);
  if (rc) return rc;
  prof_stage_begin(prof, ST_GEMM_GU, st);
  rc = launch_gemm(L, 0, x, lora_ids, topk_weights, W_gu, B_gu, workspace, st);
  prof_stage_end(prof, ST_GEMM_GU, st);
  if (rc) return rc;
  prof_stage_begin(prof, ST_SHRINK_DOWN, st);
  rc = launch_shrink(L, 1, w.h, A_down, w.zd, w.zbd, workspace, st);
  prof_stage_end(prof, ST_SHRINK_DOWN, st);
  if (rc) return rc;
  prof_stage_begin(prof, ST_GEMM_DOWN, st);
  rc = launch_gemm(L, 1, nullptr, lora_ids, topk_weights, W_down, B_down, workspace, st);
  prof_stage_end(prof, ST_GEMM_DOWN, st);
  if (rc) return rc;
  prof_stage_begin(prof, ST_COMBINE, st);
  rc = launch_combine(L, workspace, y, st);
  prof_stage_end(prof, ST_COMBINE, st);
  prof_call_done(prof);
  return rc;
}

int moe_lora_forward(const moe_lora_shape* shape, const uint16_t* x, const int32_t* topk_ids,
                     const float* topk_weights, const int32_t* lora_ids, const uint16_t* W_gu,
                     const uint16_t* W_down, const uint16_t* A_gu, const uint16_t* B_gu,
                     const uint16_t* A_down, const uint16_t* B_down, void* workspace,
                     size_t ws_bytes, uint16_t* y, void* stream) {
  return moe_lora_forward_timed(shape, x, topk_ids, topk_weights, lora_ids, W_gu, W_down, A_gu, B_gu,
                                A_down, B_down, workspace, ws_bytes, y, stream, nullptr);
}

int moe_lora_device_errors(const moe_lora_shape* shape, const void* workspace, int32_t* host_count,
                           void* stream) {
  Layout L;
  int rc = make_layout(shape, &L);
  if (rc) return rc;
  if (!workspace || !host_count) return MOE_LORA_EINVAL;
  if (L.T == 0) {
    *host_count = 0;
    return MOE_LORA_OK;
  }
  WsPtrs w = ws_ptrs(const_cast<void*>(workspace), L);
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(host_count, w.hdr + HDR_ERR, sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return MOE_LORA_EHIP;
  return hipStreamSynchronize(st) == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

const char* moe_lora_status_str(int status) {
  switch (status) {
    case MOE_LORA_OK: return "ok";
    case MOE_LORA_EINVAL: return "invalid argument";
    case MOE_LORA_EALIGN: return "misaligned pointer or size";
    case MOE_LORA_EWORKSPACE: return "workspace too small";
    case MOE_LORA_EUNSUPPORTED: return "unsupported shape";
    case MOE_LORA_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_lora_stage_count(void) { return ST_COUNT; }

const char* moe_lora_stage_name(int stage) {
  static const char* names[ST_COUNT] = {"align_count", "align_place", "shrink_gate_up",
                                        "gemm_gate_up", "shrink_down", "gemm_down", "combine",
                                        "route"};
  return (stage >= 0 && stage < ST_COUNT) ? names[stage] : "unknown";
}

int moe_lora_profiler_create(int max_calls, uint32_t stage_mask, moe_lora_profiler** out) {
  if (max_calls <= 0 || !out) return MOE_LORA_EINVAL;
  *out = nullptr;
  moe_lora_profiler* pr = new (std::nothrow) moe_lora_profiler;
  if (!pr) return MOE_LORA_EHIP;
  pr->ev.assign((size_t)max_calls * ST_COUNT * 2, nullptr);
  for (auto& e : pr->ev)
    // no system-scope fence: a plain event between two kernels adds a
    // ~10 us bubble, which would distort the stages it brackets
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      e = nullptr;
      moe_lora_profiler_destroy(pr);
      return MOE_LORA_EHIP;
    }
  pr->recorded.assign(max_calls, 0u);
  pr->max_calls = max_calls;
  pr->mask = stage_mask;
  *out = pr;
  return MOE_LORA_OK;
}

int moe_lora_profiler_read(moe_lora_profiler* pr, float* stage_ms, int n, int* calls) {
  if (!pr || !stage_ms || n < 0 || n > ST_COUNT) return MOE_LORA_EINVAL;
  for (int s = 0; s < n; ++s) stage_ms[s] = 0.f;
  const int ncalls = std::min(pr->call, pr->max_calls);
  for (int c = 0; c < ncalls; ++c)
    for (int s = 0; s < n; ++s) {
      if (!(pr->recorded[c] & (1u << s))) continue;
      hipEvent_t a = pr->ev[((size_t)c * ST_COUNT + s) * 2];
      hipEvent_t b = pr->ev[((size_t)c * ST_COUNT + s) * 2 + 1];
      float ms = 0.f;
      if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess)
        return MOE_LORA_EHIP;
      stage_ms[s] += ms;
    }
  if (calls) *calls = ncalls;
  return MOE_LORA_OK;
}

void moe_lora_profiler_destroy(moe_lora_profiler* pr) {
  if (!pr) return;
  for (hipEvent_t e : pr->ev)
    if (e) (void)hipEventDestroy(e);
  delete pr;
}

}  // extern "C"
