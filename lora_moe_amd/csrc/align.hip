// (expert, adapter) align: a stable counting sort of the (token, slot) pairs.
//
// The pages' kernel adds a grid dimension over the active adapters and shares
// one BLOCK_SIZE_M across the four LoRA ops (vLLM blog "Multi-LoRA for MoE
// models", sections "Implementing multi-LoRA inference for MoE models in vLLM"
// and "Tuning kernel configurations ...").  Here that becomes one sort by key
// (expert, slot), slot = adapter id or L for "no adapter": every expert's pairs
// form one run padded to block_m rows, and inside it each adapter's pairs are
// one contiguous segment, so the base GEMM tiles by expert and the LoRA ops
// tile by (expert, adapter) segment over the same rows.
//
// Four short kernels, all deterministic (no atomic placement).  No thread
// reads back global data written by another thread of its workgroup, so the
// workgroup barriers order LDS only and the global stores drain in the
// background:
//   1. count: per chunk of 512 pairs, an LDS histogram over the E*(L+1) keys
//      and each pair's rank among earlier same-key pairs of its chunk;
//   2. bucket scan: per key, exclusive prefix of the chunk counts (one
//      wavefront per key) and the key total;
//   3. offsets: one workgroup scans expert sizes (padded to block_m), writes
//      segment starts, the block -> expert map of the runs and the list of
//      shrink tiles (<= TS rows of one segment each);
//   4. place: row of pair p = segment start + chunk prefix + rank.
// The count pass also fills every row with the pad sentinel and every block
// with -1 (a share per workgroup), so that the offsets pass, a single
// workgroup, writes only what depends on the scan.
// Small batches (at most 1024 pairs, decode) run all of it in one
// single-workgroup kernel instead, with the counts and offsets in LDS.
#include <algorithm>

#include "device_util.h"
#include "internal.h"
#include "router_device.h"

namespace moelora {

namespace {

__device__ __forceinline__ int pair_key(const int32_t* __restrict__ topk_ids,
                                        const int32_t* __restrict__ lora_ids, int p, int k, int E,
                                        int L, int* lora_out, int* err) {
  const int t = p / k;
  int l = lora_ids[t];
  if (!(l >= -1 && l < L)) {
    l = -1;
    if (err && p - t * k == 0) (*err)++;  // count a bad adapter id once per token
  }
  *lora_out = l;
  const int e = topk_ids[p];
  if (e < 0 || e >= E) {
    if (err) (*err)++;
    return -1;
  }
  return e * (L + 1) + (l >= 0 ? l : L);
}

// Lanes of a wavefront with the same key >= 0 form a group: *rin = number of
// lower lanes in the group, *gsize = group size, *leader = lowest lane.  The
// wavefront's keys go through its 64 slots of wkeys (LDS, 16-byte aligned)
// and every lane compares against all of them: a fixed cost, independent of
// how many distinct keys the wavefront holds.
__device__ __forceinline__ void wave_key_groups(int key, int* wkeys, int* rin, int* gsize,
                                                bool* leader) {
  const int lane = threadIdx.x & 63;
  wkeys[lane] = key;  // LDS operations of one wavefront complete in order
  int before = 0, total = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const int4 k4 = *reinterpret_cast<const int4*>(wkeys + j);
    const int m0 = k4.x == key, m1 = k4.y == key, m2 = k4.z == key, m3 = k4.w == key;
    total += m0 + m1 + m2 + m3;
    before += (m0 & (j < lane)) + (m1 & (j + 1 < lane)) + (m2 & (j + 2 < lane)) + (m3 & (j + 3 < lane));
  }
  *rin = before;
  *gsize = total;
  *leader = key >= 0 && before == 0;
}

// Stable rank of each pair among the earlier pairs of the workgroup with the
// same key: the wavefronts take turns (in order) reading and advancing the
// per-key running count run[key] (LDS, zero on entry), so the result is
// deterministic; run[] ends holding the workgroup's count per key.  All
// threads must call it; nw = wavefronts that hold pairs; wkeys = blockDim.x
// ints of LDS scratch.
__device__ __forceinline__ int ordered_rank(int key, int* run, int nw, int* wkeys) {
  const int wave = threadIdx.x >> 6;
  int rin, gsize;
  bool leader;
  wave_key_groups(key, wkeys + wave * 64, &rin, &gsize, &leader);
  int rnk = 0;
  for (int w = 0; w < nw; ++w) {
    if (wave == w && key >= 0) {
      const int base = run[key];  // every lane reads before the leaders write (in-order LDS)
      rnk = base + rin;
      if (leader) run[key] = base + gsize;
    }
    lds_barrier();
  }
  return rnk;
}

// Sentinels for the padding rows of every expert run and for the rows past
// the last run, and the row-block -> expert map: eoff[E+1] run starts and
// n[E] real rows per expert (LDS).  One wavefront per expert in turn, its
// lanes over the expert's rows and blocks.
__device__ __forceinline__ void write_pads_and_blocks(int32_t* __restrict__ sorted,
                                                      int32_t* __restrict__ bexp, const int* eoff,
                                                      const int* n, int E, int P, int bm,
                                                      int64_t cap_rows, int64_t cap_blocks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (nw == 1) {
    // one wavefront: a lane per expert, so the experts' LDS reads overlap
    // instead of following one another (decode align 8.2 -> 7.1 us)
    for (int e = lane; e < E; e += 64) {
      const int a = eoff[e], b = eoff[e + 1];
      for (int row = a + n[e]; row < b; ++row) sorted[row] = P;
      for (int blk = a / bm; blk < b / bm; ++blk) bexp[blk] = e;
    }
  } else {
    for (int e = wave; e < E; e += nw) {
      const int a = eoff[e], b = eoff[e + 1];
      for (int row = a + n[e] + lane; row < b; row += 64) sorted[row] = P;
      for (int blk = a / bm + lane; blk < b / bm; blk += 64) bexp[blk] = e;
    }
  }
  const int num_padded = eoff[E];
  for (int64_t row = num_padded + threadIdx.x; row < cap_rows; row += blockDim.x) sorted[row] = P;
  for (int64_t blk = num_padded / bm + threadIdx.x; blk < cap_blocks; blk += blockDim.x) bexp[blk] = -1;
}

// Clears the split-K accumulators (z, r floats per row) of the rows in
// `row` (one per lane, -1 = none) of a whole wavefront: the lanes take the
// rows in turn, 64 / (r/4) rows per store instruction with consecutive
// lanes on consecutive 16-byte pieces of a row, so each store writes whole
// rows (a lane-per-row store writes 64 scattered pieces).  All lanes of the
// wavefront must call it; r % 8 == 0 and r <= 128.
__device__ __forceinline__ void clear_z_rows(int row, int r, int zero_gu, int zero_d,
                                             float* __restrict__ zgu, float* __restrict__ zd) {
  const int lane = threadIdx.x & 63;
  const int cpr = r >> 2;        // 16-byte pieces per row (2..32)
  const int rpi = 64 / cpr;      // rows per instruction
  const int sub = lane / cpr, piece = lane - sub * cpr;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < 64; j0 += rpi) {
    const int j = j0 + sub;
    const int src = j < 64 ? j : 63;
    const int rj = __shfl(row, src, 64);
    if (sub < rpi && j < 64 && rj >= 0) {
      if (zero_gu) *reinterpret_cast<float4*>(zgu + (size_t)rj * r + piece * 4) = z;
      if (zero_d) *reinterpret_cast<float4*>(zd + (size_t)rj * r + piece * 4) = z;
    }
  }
}

__global__ __launch_bounds__(kAlignChunk) void align_count_kernel(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ lora_ids, int P, int k, int E,
    int L, int NB, int C, int32_t* __restrict__ chunk_cnt, int32_t* __restrict__ chunk_err,
    int32_t* __restrict__ rank, int32_t* __restrict__ sorted, int32_t* __restrict__ bexp,
    int64_t cap_rows, int64_t cap_blocks) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  int* wkeys = lds;                // [kAlignChunk]
  int* errs = wkeys + kAlignChunk; // [1]
  int* hist = errs + 1;            // [NB]
  const int tid = threadIdx.x, c = blockIdx.x;
  // this workgroup's share of the sentinel fill (the place pass overwrites
  // the real rows, the offsets pass the blocks of the runs)
  {
    const int64_t rs = (cap_rows + C - 1) / C, r0 = c * rs, r1 = min(cap_rows, r0 + rs);
    for (int64_t row = r0 + tid; row < r1; row += blockDim.x) sorted[row] = P;
    const int64_t bs = (cap_blocks + C - 1) / C, b0 = c * bs, b1 = min(cap_blocks, b0 + bs);
    for (int64_t blk = b0 + tid; blk < b1; blk += blockDim.x) bexp[blk] = -1;
  }
  for (int b = tid; b < NB; b += blockDim.x) hist[b] = 0;
  if (tid == 0) errs[0] = 0;
  const int p = c * kAlignChunk + tid;
  int key = -1, err = 0, l;
  if (p < P) key = pair_key(topk_ids, lora_ids, p, k, E, L, &l, &err);
  lds_barrier();  // hist and errs cleared
  if (err) atomicAdd(&errs[0], err);
  // rank among earlier pairs of this chunk with the same key (stable order);
  // hist ends as the chunk's count per key
  const int rnk = ordered_rank(key, hist, (min(P - c * kAlignChunk, kAlignChunk) + 63) >> 6, wkeys);
  for (int b = tid; b < NB; b += blockDim.x) chunk_cnt[(size_t)b * C + c] = hist[b];
  if (p < P) rank[p] = rnk;
  if (tid == 0) chunk_err[c] = errs[0];
}

// One wavefront per key: chunk counts -> exclusive prefixes (in place), total.
__global__ __launch_bounds__(256) void align_bucket_scan_kernel(int NB, int C,
                                                                int32_t* __restrict__ chunk_cnt,
                                                                int32_t* __restrict__ segcnt) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= NB) return;
  int32_t* row = chunk_cnt + (size_t)b * C;
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < C ? row[c] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (c < C) row[c] = carry + x - v;
    carry += __shfl(x, 63, 64);
  }
  if (lane == 0) segcnt[b] = carry;
}

__global__ __launch_bounds__(1024) void align_offsets_kernel(
    int E, int L, int C, int bm, int TS, const int32_t* __restrict__ chunk_err,
    const int32_t* __restrict__ segcnt, int32_t* __restrict__ hdr, int32_t* __restrict__ eoff,
    int32_t* __restrict__ segstart, int32_t* __restrict__ bexp, LoraTile* __restrict__ tiles) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x, nt = blockDim.x, S = L + 1, NB = E * S;
  int* scan = lds;              // [16]
  int* s_eoff = scan + 16;      // [E+1] run starts
  int* s_cnt = s_eoff + E + 1;  // [NB] rows per (expert, slot); then the segment starts
  for (int b = tid; b < NB; b += nt) s_cnt[b] = segcnt[b];
  int errs = 0;
  for (int c = tid; c < C; c += nt) errs += chunk_err[c];
  lds_barrier();

  // padded expert sizes, scanned over experts (each thread owns a range)
  const int per = (E + nt - 1) / nt;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) {
    int n = 0;
    for (int sl = 0; sl < S; ++sl) n += s_cnt[e * S + sl];
    local += (n + bm - 1) / bm * bm;
  }
  int total;
  int at = block_exclusive_scan<true>(local, scan, &total);
  for (int e = e0; e < e1; ++e) {
    s_eoff[e] = at;
    eoff[e] = at;
    int n = 0;
    for (int sl = 0; sl < S; ++sl) {
      const int cnt = s_cnt[e * S + sl];
      segstart[e * S + sl] = at + n;
      s_cnt[e * S + sl] = at + n;  // start in place of the count (slot L ends the slots before it)
      n += cnt;
    }
    at += (n + bm - 1) / bm * bm;
  }
  if (tid == 0) {
    s_eoff[E] = total;
    eoff[E] = total;
  }
  int nerr;
  block_exclusive_scan<true>(errs, scan, &nerr);  // also orders the s_eoff writes before the reads below
  const int num_padded = total;
  // block -> expert map of the runs, a thread per expert (the count pass
  // wrote -1 everywhere, the place pass writes the real rows; the padding
  // rows keep the count pass's sentinel)
  for (int e = tid; e < E; e += nt) {
    const int a = s_eoff[e], b = s_eoff[e + 1];
    for (int blk = a / bm; blk < b / bm; ++blk) bexp[blk] = e;
  }

  // shrink tiles: segments (e, l < L) cut into pieces of <= TS rows; a
  // thread owns consecutive segments; segment (e, l) spans the starts of
  // slots l and l + 1
  const int NS = E * L;
  const int perS = (NS + nt - 1) / nt;
  const int s0 = min(NS, tid * perS), s1 = min(NS, s0 + perS);
  int lt = 0;
  for (int i = s0; i < s1; ++i) {
    const int b = (i / L) * S + i % L;
    lt += (s_cnt[b + 1] - s_cnt[b] + TS - 1) / TS;
  }
  int ntiles;
  int tb = block_exclusive_scan<true>(lt, scan, &ntiles);
  for (int i = s0; i < s1; ++i) {
    const int e = i / L, l = i % L, b = e * S + l;
    const int st = s_cnt[b], cnt = s_cnt[b + 1] - st;
    for (int o = 0; o < cnt; o += TS) {
      LoraTile tl;
      tl.e = e;
      tl.l = l;
      tl.row0 = st + o;
      tl.n = min(TS, cnt - o);
      tiles[tb++] = tl;
    }
  }
  if (tid == 0) {
    hdr[HDR_NUM_PADDED] = num_padded;
    hdr[HDR_ERR] = nerr;
    hdr[HDR_NTILES] = ntiles;
  }
}

__global__ __launch_bounds__(256) void align_place_kernel(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ lora_ids, int P, int k, int E,
    int L, int C, int r, int zero_gu, int zero_d, const int32_t* __restrict__ chunk_cnt,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ segstart,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos, float* __restrict__ zgu,
    float* __restrict__ zd) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  int zrow = -1;  // adapter row whose split-K accumulators this lane's pair owns
  if (p < P) {
    int l;
    const int key = pair_key(topk_ids, lora_ids, p, k, E, L, &l, nullptr);
    if (key < 0) {
      pos[p] = -1;
    } else {
      const int c = p / kAlignChunk;
      const int row = segstart[key] + chunk_cnt[(size_t)key * C + c] + rank[p];
      sorted[row] = p;
      pos[p] = row;
      if (l >= 0) zrow = row;
    }
  }
  if (zero_gu || zero_d) clear_z_rows(zrow, r, zero_gu, zero_d, zgu, zd);  // whole wavefronts
}

constexpr int kSmallMaxPairs = 1024;
constexpr size_t kSmallMaxLds = 64 * 1024;  // the single-workgroup path keeps its tables in LDS
constexpr int kFusedRouteMaxPairs = 256;  // router fused into the single-workgroup align up to here

// The whole align (and, when given logits, the router: one thread per
// token) for P <= 1024 in one workgroup of ceil(P/64) wavefronts (thread =
// pair), same outputs as the four-kernel path.
__global__ __launch_bounds__(1024) void align_small_kernel(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ lora_ids, int P, int k, int E,
    int L, int bm, int64_t cap_rows, int64_t cap_blocks, int TS, int r, int zero_gu, int zero_d,
    int32_t* __restrict__ hdr, int32_t* __restrict__ sorted, int32_t* __restrict__ eoff,
    int32_t* __restrict__ segstart, int32_t* __restrict__ segcnt, int32_t* __restrict__ bexp,
    int32_t* __restrict__ pos, LoraTile* __restrict__ tiles, float* __restrict__ zgu,
    float* __restrict__ zd, const float* __restrict__ logits, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  const int S = L + 1, NB = E * S;
  int* wkeys = lds;                  // [kSmallMaxPairs]
  int* rids = wkeys + kSmallMaxPairs; // [kSmallMaxPairs] routed expert per pair (router fused)
  int* cnt = rids + kSmallMaxPairs;  // [NB]
  int* sst = cnt + NB;               // [NB] segment starts
  int* s_eoff = sst + NB;            // [E+1]
  int* s_n = s_eoff + E + 1;         // [E] real rows per expert
  int* scan = s_n + E;               // [16]
  int* errs = scan + 16;             // [1]
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int b = tid; b < NB; b += nt) cnt[b] = 0;
  if (tid == 0) errs[0] = 0;
  const int32_t* ids_src = topk_ids;
  if (logits) {  // router fused in: thread t routes token t
    if (tid < P / k) {
      route_token_thread(logits + (size_t)tid * E, E, k, rids + tid * k, w_out + (size_t)tid * k);
      for (int j = 0; j < k; ++j) ids_out[(size_t)tid * k + j] = rids[tid * k + j];
    }
    lds_barrier();
    ids_src = rids;
  }
  int key = -1, err = 0, l = -1;
  if (tid < P) key = pair_key(ids_src, lora_ids, tid, k, E, L, &l, &err);
  lds_barrier();  // cnt and errs cleared
  if (err) atomicAdd(&errs[0], err);
  // stable rank = earlier pairs with the same key; cnt ends as the key counts
  const int rnk = ordered_rank(key, cnt, (min(P, nt) + 63) >> 6, wkeys);

  // padded expert sizes, scanned over experts (each thread owns a range)
  const int per = (E + nt - 1) / nt;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) {
    int n = 0;
    for (int s = 0; s < S; ++s) n += cnt[e * S + s];
    s_n[e] = n;
    local += (n + bm - 1) / bm * bm;
  }
  int total;
  int at = block_exclusive_scan<true>(local, scan, &total);
  for (int e = e0; e < e1; ++e) {
    s_eoff[e] = at;
    eoff[e] = at;
    int n = 0;
    for (int s = 0; s < S; ++s) {
      sst[e * S + s] = at + n;
      segstart[e * S + s] = at + n;
      segcnt[e * S + s] = cnt[e * S + s];
      n += cnt[e * S + s];
    }
    at += (n + bm - 1) / bm * bm;
  }
  if (tid == 0) {
    s_eoff[E] = total;
    eoff[E] = total;
  }
  lds_barrier();
  const int num_padded = total;
  write_pads_and_blocks(sorted, bexp, s_eoff, s_n, E, P, bm, cap_rows, cap_blocks);
  int zrow = -1;  // adapter row whose split-K accumulators this pair owns
  if (tid < P) {
    if (key < 0) {
      pos[tid] = -1;
    } else {
      const int row = sst[key] + rnk;
      sorted[row] = tid;
      pos[tid] = row;
      if (l >= 0) zrow = row;
    }
  }
  if (zero_gu || zero_d) clear_z_rows(zrow, r, zero_gu, zero_d, zgu, zd);  // whole wavefronts

  // shrink tiles: segments (e, l < L) cut into pieces of <= TS rows
  const int NS = E * L;
  const int perS = (NS + nt - 1) / nt;
  const int s0 = min(NS, tid * perS), s1 = min(NS, s0 + perS);
  int lt = 0;
  for (int i = s0; i < s1; ++i) lt += (cnt[(i / L) * S + i % L] + TS - 1) / TS;
  int ntiles;
  int tb = block_exclusive_scan<true>(lt, scan, &ntiles);
  for (int i = s0; i < s1; ++i) {
    const int e = i / L, ll = i % L;
    const int c = cnt[e * S + ll], st = sst[e * S + ll];
    for (int o = 0; o < c; o += TS) {
      LoraTile tl;
      tl.e = e;
      tl.l = ll;
      tl.row0 = st + o;
      tl.n = min(TS, c - o);
      tiles[tb++] = tl;
    }
  }
  if (tid == 0) {
    hdr[HDR_NUM_PADDED] = num_padded;
    hdr[HDR_ERR] = errs[0];
    hdr[HDR_NTILES] = ntiles;
  }
}

}  // namespace

int launch_align(const Layout& L, const int32_t* topk_ids, const int32_t* lora_ids, void* ws,
                 hipStream_t st, moe_lora_profiler* pr, const float* logits, int32_t* ids_out,
                 float* w_out) {
  WsPtrs w = ws_ptrs(ws, L);
  const int P = (int)L.P, NB = (int)L.NB, C = (int)L.C;
  if (P <= 0) return MOE_LORA_OK;  // no pairs: nothing to sort
  const int zero_gu = plan_shrink(L, L.H).splits > 1;
  const int zero_d = plan_shrink(L, L.I).splits > 1;
  const size_t small_lds = sizeof(int) * (2 * kSmallMaxPairs + 2 * (size_t)NB + 2 * L.E + 1 + 16 + 1);
  const bool small = P <= kSmallMaxPairs && small_lds <= kSmallMaxLds;
  // The router runs inside the single-workgroup align (one thread per token)
  // only for decode-sized batches; beyond that its own kernel (a wavefront per
  // token, all tokens at once) runs first and the align reads its output.
  if (logits && !(small && P <= kFusedRouteMaxPairs)) {
    prof_stage_begin(pr, ST_ROUTE, st);
    const int rc = launch_router(L, logits, ids_out, w_out, st);
    prof_stage_end(pr, ST_ROUTE, st);
    if (rc) return rc;
    topk_ids = ids_out;
    logits = nullptr;
  }
  if (small) {
    prof_stage_begin(pr, ST_ALIGN_PLACE, st);
    const size_t lds = small_lds;
    // one thread per pair (whole wavefronts): fewer wavefronts, cheaper barriers
    const int nthreads = std::min(kSmallMaxPairs, (P + 63) / 64 * 64);
    align_small_kernel<<<1, nthreads, lds, st>>>(
        logits ? nullptr : topk_ids, lora_ids, P, L.k, L.E, L.L, L.bm, L.cap_rows, L.cap_blocks, (int)L.TS, L.r, zero_gu,
        zero_d, w.hdr, w.sorted, w.eoff, w.segstart, w.segcnt, w.bexp, w.pos, w.tiles, w.zgu, w.zd,
        logits, ids_out, w_out);
    prof_stage_end(pr, ST_ALIGN_PLACE, st);
    return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
  }
  prof_stage_begin(pr, ST_ALIGN_COUNT, st);
  align_count_kernel<<<C, kAlignChunk, (kAlignChunk + 1 + NB) * sizeof(int), st>>>(
      topk_ids, lora_ids, P, L.k, L.E, L.L, NB, C, w.chunk, w.chunkerr, w.rank, w.sorted, w.bexp, L.cap_rows,
      L.cap_blocks);
  align_bucket_scan_kernel<<<(NB + 3) / 4, 256, 0, st>>>(NB, C, w.chunk, w.segcnt);
  prof_stage_end(pr, ST_ALIGN_COUNT, st);
  prof_stage_begin(pr, ST_ALIGN_PLACE, st);
  const size_t off_lds = sizeof(int) * (16 + (size_t)L.E + 1 + NB);
  if (off_lds > 64 * 1024) {  // above the default dynamic LDS limit (at most 86 KB here)
    static std::atomic<uint64_t> attr_done{0};
    const int rc = ensure_dynamic_lds(reinterpret_cast<const void*>(&align_offsets_kernel), 160 * 1024,
                                      attr_done);
    if (rc) return rc;
  }
  align_offsets_kernel<<<1, 1024, off_lds, st>>>(L.E, L.L, C, L.bm, (int)L.TS, w.chunkerr, w.segcnt, w.hdr,
                                                  w.eoff, w.segstart, w.bexp, w.tiles);
  align_place_kernel<<<(P + 255) / 256, 256, 0, st>>>(topk_ids, lora_ids, P, L.k, L.E, L.L, C, L.r,
                                                      zero_gu, zero_d, w.chunk, w.rank, w.segstart,
                                                      w.sorted, w.pos, w.zgu, w.zd);
  prof_stage_end(pr, ST_ALIGN_PLACE, st);
  return hipGetLastError() == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

}  // namespace moelora
