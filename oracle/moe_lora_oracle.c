/* Plain fp64 CPU reference ("oracle") of the fused MoE-LoRA layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP product path
 * never calls it, and it shares no code, header or table with that path.
 *
 * What it computes (sources are the pages on vLLM multi-LoRA serving for MoE
 * models; "vLLM blog" is the page "vllm.com.cn/blog/2026-02-26-multi-lora"):
 *   - each expert is a two-stage feed-forward network: a gate_up projection
 *     widens the hidden state, a down projection narrows it back
 *     (vLLM blog, section on implementing multi-LoRA for MoE, Figure 1);
 *   - every projection with weight W (h_in x h_out) carries an adapter A
 *     (h_in x r) and B (r x h_out), and the output is y = xW + xAB; the shrink
 *     computes z = xA, the expand computes zB (same section, Eq. y = xW + xAB);
 *   - the router sends each token to experts and the layer then sums their
 *     outputs (same section); the weighted top-k sum is the plain reading;
 *   - the activation between the projections is not named on the pages; the
 *     plain reading used here is SiLU-gating: h = silu(gate) * up with
 *     silu(v) = v / (1 + exp(-v)), gate = first half of the gate_up output;
 *   - the (expert, adapter) align: a stable counting sort of the pairs with
 *     per-expert padding (orc_align), and the router that picks the top-k
 *     experts and their weights from logits (orc_route); the readings are in
 *     their comments.
 *
 * Parity status: every function here is pinned by the CPU tests (closed-form
 * worked examples, reductions to a dense SwiGLU MLP computed with library
 * matmuls, the merged-weight identity W + s*A*B, invariances, brute-force
 * sorting of the align keys).  None is "parity unpinned".
 *
 * Storage (all row-major, weights with the reduction index contiguous, i.e.
 * the transposes of the pages' h_in x h_out matrices):
 *   x        [T][H]        bf16 bits        W_gu   [E][2I][H]   bf16 bits
 *   topk_ids [T][k]        int32            W_down [E][H][I]    bf16 bits
 *   topk_w   [T][k]        float            A_gu   [L][E][r][H] bf16 bits
 *   lora_ids [T]           int32 (-1=none)  B_gu   [L][E][2I][r] bf16 bits
 *                                           A_down [L][E][r][I] bf16 bits
 *                                           B_down [L][E][H][r] bf16 bits
 * All bf16 values are decoded exactly into fp64; nothing is rounded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf(uint16_t u) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)u << 16;
  return (double)v.f;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

typedef struct {
  int T, H, I, E, k, L, r;
  double s;
  const uint16_t *x, *W_gu, *W_down, *A_gu, *B_gu, *A_down, *B_down;
  const int32_t *topk_ids, *lora_ids;
  const float* topk_w;
} layer_t;

/* Expert id of pair (t, j), or -1 when it is outside [0, E) (pair dropped). */
static int pair_expert(const layer_t* P, int t, int j) {
  int e = P->topk_ids[(size_t)t * P->k + j];
  return (e >= 0 && e < P->E) ? e : -1;
}

/* Adapter of token t, or -1 for "no adapter" (ids outside [-1, L) count as none). */
static int token_adapter(const layer_t* P, int t) {
  int l = P->lora_ids[t];
  return (l >= 0 && l < P->L) ? l : -1;
}

/* One (token, expert) pair through the expert with its adapter l (-1: none).
 * Outputs: g[2I] gate_up result, zg[r] gate_up shrink, h[I] activation,
 * zd[r] down shrink, d[H] down result.  zg/zd are left 0 when l < 0. */
static void pair_forward(const layer_t* P, int t, int e, int l,
                         double* g, double* zg, double* h, double* zd, double* d) {
  const int H = P->H, I = P->I, E = P->E, r = P->r;
  const uint16_t* xr = P->x + (size_t)t * H;

  /* base gate_up: g = x W_gu[e]  (W stored [2I][H]) */
  const uint16_t* Wg = P->W_gu + (size_t)e * 2 * I * H;
  for (int n = 0; n < 2 * I; ++n) {
    double acc = 0.0;
    for (int i = 0; i < H; ++i) acc += bf(xr[i]) * bf(Wg[(size_t)n * H + i]);
    g[n] = acc;
  }
  for (int q = 0; q < r; ++q) zg[q] = 0.0;
  if (l >= 0) {
    /* gate_up shrink: zg = x A_gu[l][e]  (A stored [r][H]) */
    const uint16_t* A = P->A_gu + ((size_t)l * E + e) * r * H;
    for (int q = 0; q < r; ++q) {
      double acc = 0.0;
      for (int i = 0; i < H; ++i) acc += bf(xr[i]) * bf(A[(size_t)q * H + i]);
      zg[q] = acc;
    }
    /* gate_up expand, added to the base output: g += s * zg B_gu[l][e]  (B stored [2I][r]) */
    const uint16_t* B = P->B_gu + ((size_t)l * E + e) * 2 * I * r;
    for (int n = 0; n < 2 * I; ++n) {
      double acc = 0.0;
      for (int q = 0; q < r; ++q) acc += zg[q] * bf(B[(size_t)n * r + q]);
      g[n] += P->s * acc;
    }
  }
  /* activation: h = silu(gate) * up, gate = g[0, I), up = g[I, 2I) */
  for (int i = 0; i < I; ++i) h[i] = silu(g[i]) * g[I + i];

  /* base down: d = h W_down[e]  (W stored [H][I]) */
  const uint16_t* Wd = P->W_down + (size_t)e * H * I;
  for (int m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += h[i] * bf(Wd[(size_t)m * I + i]);
    d[m] = acc;
  }
  for (int q = 0; q < r; ++q) zd[q] = 0.0;
  if (l >= 0) {
    /* down shrink: zd = h A_down[l][e]  (A stored [r][I]) */
    const uint16_t* A = P->A_down + ((size_t)l * E + e) * r * I;
    for (int q = 0; q < r; ++q) {
      double acc = 0.0;
      for (int i = 0; i < I; ++i) acc += h[i] * bf(A[(size_t)q * I + i]);
      zd[q] = acc;
    }
    /* down expand, added to the base output: d += s * zd B_down[l][e]  (B stored [H][r]) */
    const uint16_t* B = P->B_down + ((size_t)l * E + e) * H * r;
    for (int m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int q = 0; q < r; ++q) acc += zd[q] * bf(B[(size_t)m * r + q]);
      d[m] += P->s * acc;
    }
  }
}

/* Layer output for the tokens listed in `tokens` (all T tokens when tokens is
 * NULL): y[i][:] = sum_j topk_w[t][j] * d(t, j) for t = tokens[i].  Pairs with
 * an out-of-range expert id contribute nothing.  Returns 0, or -1 when the
 * scratch allocation fails. */
int orc_layer(int T, int H, int I, int E, int k, int L, int r, double scale,
              const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
              const int32_t* lora_ids, const uint16_t* W_gu, const uint16_t* W_down,
              const uint16_t* A_gu, const uint16_t* B_gu, const uint16_t* A_down,
              const uint16_t* B_down, const int32_t* tokens, int n_tokens, double* y,
              int nthreads) {
  layer_t P = {T, H, I, E, k, L, r, scale, x, W_gu, W_down, A_gu, B_gu, A_down, B_down,
               topk_ids, lora_ids, topk_w};
  int n = tokens ? n_tokens : T;
  int failed = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    size_t rr = r > 0 ? (size_t)r : 1;
    double* g = (double*)malloc(sizeof(double) * (2 * (size_t)I + I + H + 2 * rr));
    if (!g) {
#pragma omp atomic write
      failed = 1;
    } else {
      double *h = g + 2 * (size_t)I, *d = h + I, *zg = d + H, *zd = zg + rr;
#pragma omp for schedule(dynamic, 1)
      for (int i = 0; i < n; ++i) {
        int t = tokens ? tokens[i] : i;
        double* yr = y + (size_t)i * H;
        for (int m = 0; m < H; ++m) yr[m] = 0.0;
        int l = token_adapter(&P, t);
        for (int j = 0; j < k; ++j) {
          int e = pair_expert(&P, t, j);
          if (e < 0) continue;
          pair_forward(&P, t, e, l, g, zg, h, zd, d);
          double w = (double)topk_w[(size_t)t * k + j];
          for (int m = 0; m < H; ++m) yr[m] += w * d[m];
        }
      }
      free(g);
    }
  }
  return failed ? -1 : 0;
}

/* Intermediate values of one pair (t, j) for stage checks: g[2I], zg[r],
 * h[I], zd[r], d[H] (d before the top-k weight).  Returns -1 when the pair's
 * expert id is out of range (nothing written). */
int orc_pair(int T, int H, int I, int E, int k, int L, int r, double scale,
             const uint16_t* x, const int32_t* topk_ids, const int32_t* lora_ids,
             const uint16_t* W_gu, const uint16_t* W_down, const uint16_t* A_gu,
             const uint16_t* B_gu, const uint16_t* A_down, const uint16_t* B_down, int t, int j,
             double* g, double* zg, double* h, double* zd, double* d) {
  layer_t P = {T, H, I, E, k, L, r, scale, x, W_gu, W_down, A_gu, B_gu, A_down, B_down,
               topk_ids, lora_ids, NULL};
  int e = pair_expert(&P, t, j);
  if (e < 0) return -1;
  pair_forward(&P, t, e, token_adapter(&P, t), g, zg, h, zd, d);
  return 0;
}

/* (expert, adapter) align: a stable counting sort of the P = T*k pairs
 * p = t*k + j by key (e, slot), slot = adapter of token t, or L for "no
 * adapter", so that each expert's pairs are contiguous, its adapter groups
 * form contiguous segments in adapter order with the no-adapter group last,
 * and pairs keep ascending p inside a segment.  Each expert's run is padded
 * to a multiple of block_m (one block size shared by every op of the layer,
 * vLLM blog, section on tuning kernel configurations) with the sentinel P.
 *
 *   sorted_ids[cap_rows]      pair ids, sentinel P in pad slots and beyond
 *   expert_off[E+1]           start of each expert's padded run
 *   seg_start/seg_cnt[E*(L+1)] segment of (expert e, slot s) at [e*(L+1)+s]
 *   block_expert[cap_blocks]  expert of each block_m-row block, -1 if unused
 *   pos_of_pair[P]            row of pair p in sorted_ids, -1 if dropped
 *   num_padded                expert_off[E]
 *   err_count                 pairs with expert id outside [0,E) plus tokens
 *                             with adapter id outside [-1,L)
 * Returns 0, or -1 when cap_rows / cap_blocks are too small. */
int orc_align(int T, int k, int E, int L, int block_m, const int32_t* topk_ids,
              const int32_t* lora_ids, int cap_rows, int cap_blocks, int32_t* sorted_ids,
              int32_t* expert_off, int32_t* seg_start, int32_t* seg_cnt, int32_t* block_expert,
              int32_t* pos_of_pair, int32_t* num_padded, int32_t* err_count) {
  const int P = T * k, S = L + 1;
  int32_t* cnt = (int32_t*)calloc((size_t)E * S + 1, sizeof(int32_t));
  int32_t* cur = (int32_t*)calloc((size_t)E * S + 1, sizeof(int32_t));
  if (!cnt || !cur) { free(cnt); free(cur); return -1; }
  int errs = 0;
  for (int t = 0; t < T; ++t) {
    int l = lora_ids[t];
    if (!(l >= -1 && l < L)) errs++;
  }
  for (int p = 0; p < P; ++p) {
    int e = topk_ids[p];
    if (e < 0 || e >= E) { errs++; continue; }
    int l = lora_ids[p / k];
    int s = (l >= 0 && l < L) ? l : L;
    cnt[(size_t)e * S + s]++;
  }
  expert_off[0] = 0;
  for (int e = 0; e < E; ++e) {
    int n_e = 0;
    for (int s = 0; s < S; ++s) n_e += cnt[(size_t)e * S + s];
    int pad = (n_e + block_m - 1) / block_m * block_m;
    expert_off[e + 1] = expert_off[e] + pad;
  }
  int total = expert_off[E];
  if (total > cap_rows || (total + block_m - 1) / block_m > cap_blocks) {
    free(cnt); free(cur); return -1;
  }
  for (int e = 0; e < E; ++e) {
    int at = expert_off[e];
    for (int s = 0; s < S; ++s) {
      seg_start[(size_t)e * S + s] = at;
      seg_cnt[(size_t)e * S + s] = cnt[(size_t)e * S + s];
      cur[(size_t)e * S + s] = at;
      at += cnt[(size_t)e * S + s];
    }
  }
  for (int i = 0; i < cap_rows; ++i) sorted_ids[i] = P;
  for (int p = 0; p < P; ++p) {
    int e = topk_ids[p];
    if (e < 0 || e >= E) { pos_of_pair[p] = -1; continue; }
    int l = lora_ids[p / k];
    int s = (l >= 0 && l < L) ? l : L;
    int pos = cur[(size_t)e * S + s]++;
    sorted_ids[pos] = p;
    pos_of_pair[p] = pos;
  }
  for (int b = 0; b < cap_blocks; ++b) {
    long row = (long)b * block_m;
    block_expert[b] = -1;
    for (int e = 0; e < E && row < total; ++e)
      if (row >= expert_off[e] && row < expert_off[e + 1]) { block_expert[b] = e; break; }
  }
  *num_padded = total;
  *err_count = errs;
  free(cnt);
  free(cur);
  return 0;
}

/* Router: each token goes to the k experts with the largest logits, and the
 * layer sums their outputs with weights (vLLM blog, section on implementing
 * multi-LoRA for MoE: the router picks top-k experts per token and the
 * outputs are aggregated).  The pages fix neither the order of equal logits
 * nor the weight formula; the plain reading used here:
 *   - experts in descending logit order, equal logits by ascending index
 *     (slot j holds the j-th choice);
 *   - weights = softmax over the k chosen logits, which equals the full
 *     softmax's top-k probabilities renormalised to sum to one;
 *   - a logit that is not a finite number (NaN, +inf, -inf) is never chosen:
 *     it has no place in a descending order that a softmax can weight.  When
 *     fewer than k finite logits remain, the slots left over get expert -1
 *     and weight 0, and the chosen ones share the weight.
 * logits [T][E] float, ids [T][k] int32, w [T][k] double.
 * Returns 0, or -1 for k outside [1, E]. */
int orc_route(int T, int E, int k, const float* logits, int32_t* ids, double* w) {
  if (k < 1 || k > E) return -1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  if (!taken) return -1;
  for (int t = 0; t < T; ++t) {
    const float* lg = logits + (size_t)t * E;
    int32_t* id = ids + (size_t)t * k;
    double* wt = w + (size_t)t * k;
    memset(taken, 0, (size_t)E);
    int nch = 0;  /* slots that received an expert */
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e] || !isfinite(lg[e])) continue;
        if (best < 0 || (double)lg[e] > (double)lg[best]) best = e;  /* strict: ties keep the lower index */
      }
      id[j] = best;
      if (best < 0) continue;
      taken[best] = 1;
      ++nch;
    }
    if (nch == 0) {
      for (int j = 0; j < k; ++j) wt[j] = 0.0;
      continue;
    }
    const double m = (double)lg[id[0]];  /* the largest chosen logit */
    double sum = 0.0;
    for (int j = 0; j < nch; ++j) sum += exp((double)lg[id[j]] - m);
    for (int j = 0; j < k; ++j) wt[j] = j < nch ? exp((double)lg[id[j]] - m) / sum : 0.0;
  }
  free(taken);
  return 0;
}
