// Router: the per-token top-k choice and its weights, shared by the router
// kernel and the fused router + align kernel.
//
// The router sends each token to its top-k experts and the layer aggregates
// their outputs (vLLM blog "Multi-LoRA for MoE models", section
// "Implementing multi-LoRA inference for MoE models in vLLM").  The pages fix
// neither the order of equal logits nor the weight formula; this library
// takes experts by descending logit with equal logits by ascending expert
// index (slot j holds the j-th choice), and weights = softmax over the k
// chosen logits (the full softmax's top-k probabilities renormalised).
//
// One wavefront per token.  Choice j is the largest element, in the order
// (logit descending, index ascending), among those that come after choice
// j-1 in that order, so no list of taken experts is kept: each lane scans
// its experts (lane, lane + 64, ...) for the best eligible one and a
// butterfly of lane exchanges picks the wavefront's best.  Lane j keeps
// choice j; the softmax runs across lanes 0..k-1 (k <= 64).  Comparisons are
// exact fp32 comparisons, so the chosen ids are bit-exact.  A non-finite
// logit (NaN, +inf, -inf) is never chosen: slots left without a finite
// logit get expert -1 and weight 0 (the align counts and drops such pairs),
// and the chosen ones share the weight.
#pragma once

#include "device_util.h"

namespace moelora {

// a before b in the choice order: larger logit, or equal logit and lower index
__device__ __forceinline__ bool before(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// x (logit of expert e) may be chosen after the previous choice (pv, pe):
// it is finite and comes after that choice in the order
__device__ __forceinline__ bool eligible(float pv, int pe, float x, int e) {
  return __builtin_isfinite(x) && before(pv, pe, x, e);
}

// Routes token t with one wavefront (all 64 lanes call it); on return lane j
// < k holds (expert, weight) of slot j.  R = experts cached per lane in
// registers (E <= 64 * R), 0 to read them from memory every round.
template <int R>
__device__ __forceinline__ void route_token(const float* __restrict__ lg, int E, int k, int* my_e,
                                            float* my_w) {
  const int lane = threadIdx.x & 63;
  float v[R > 0 ? R : 1];
#pragma unroll
  for (int i = 0; i < (R > 0 ? R : 1); ++i) {
    const int e = lane + 64 * i;
    v[i] = (R > 0 && e < E) ? lg[e] : 0.f;
  }
  float pv = __builtin_inff();  // previous choice: everything comes after (+inf, -1)
  int pe = -1;
  int ce = -1;
  float cv = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int be = -1;
    if (R > 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int e = lane + 64 * i;
        if (e < E && eligible(pv, pe, v[i], e) && (be < 0 || before(v[i], e, bv, be))) {
          bv = v[i];
          be = e;
        }
      }
    } else {
      for (int e = lane; e < E; e += 64) {
        const float x = lg[e];
        if (eligible(pv, pe, x, e) && (be < 0 || before(x, e, bv, be))) {
          bv = x;
          be = e;
        }
      }
    }
    // wavefront-wide best; lanes without a candidate carry be = -1
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (oe >= 0 && (be < 0 || before(ov, oe, bv, be))) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == j) {
      ce = be;
      cv = bv;
    }
    if (be < 0) break;  // uniform: nothing eligible is left (non-finite logits)
    pv = bv;
    pe = be;
  }
  // softmax over the chosen logits (lane 0 holds the largest)
  const float m = __shfl(cv, 0, 64);
  const float ex = (lane < k && ce >= 0) ? expf(cv - m) : 0.f;
  float sum = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  *my_e = ce;
  *my_w = ce >= 0 ? ex / sum : 0.f;
}

// The same choice and weights by one thread for one token (no lane
// exchanges): k scans over the token's E logits.  For small batches, where a
// thread per token keeps every token in flight at once.  Writes ids[0..k) and
// w[0..k) (ids may be LDS: it is read back for the weights).
__device__ __forceinline__ void route_token_thread(const float* __restrict__ lg, int E, int k,
                                                   int32_t* ids, float* __restrict__ w) {
  float pv = __builtin_inff();
  int pe = -1;
  float m = 0.f;
  int nch = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int be = -1;
    for (int e = 0; e < E; ++e) {
      const float x = lg[e];
      if (eligible(pv, pe, x, e) && (be < 0 || before(x, e, bv, be))) {
        bv = x;
        be = e;
      }
    }
    ids[j] = be;
    if (be < 0) continue;  // nothing eligible is left (non-finite logits)
    if (j == 0) m = bv;
    ++nch;
    pv = bv;
    pe = be;
  }
  float sum = 0.f;
  for (int j = 0; j < nch; ++j) sum += expf(lg[ids[j]] - m);
  for (int j = 0; j < k; ++j) w[j] = j < nch ? expf(lg[ids[j]] - m) / sum : 0.f;
}

}  // namespace moelora
