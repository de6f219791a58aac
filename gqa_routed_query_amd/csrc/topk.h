// Top-k selection for the GQE router, shared by the router kernels.
//
// gist.science explainer of "Grouped Query Experts: Mixture-of-Experts on GQA
// Self-Attention", section "Architecture et Routage": per token the router
// keeps k experts inside each GQA group, and the kept experts are weighted by
// the router probabilities renormalised over the k kept. Renormalising over
// the kept set cancels the softmax denominator, so
// gate_j = exp(l_j - l_max) / sum over kept of exp(l - l_max).
//
// Rank order: higher logit first; equal logits keep the lower head index
// first. The raw fp32 logits are compared with '>' only, so the selection is
// exact and +0.0 / -0.0 count as equal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// ell(e) returns logit e (< r <= 64) of one group whose first head is `base`;
// writes the k kept heads (global ids, rank order) to idx and their gates to
// gate (gate doubles as scratch for the unnormalised weights).
template <typename Logit>
__device__ inline void topk_select(Logit ell, int r, int k, int base, int32_t* idx, float* gate) {
  uint64_t taken = 0;
  float top = 0.0f, wsum = 0.0f;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float vb = 0.0f;
    for (int e = 0; e < r; ++e) {
      if ((taken >> e) & 1ull) continue;
      const float v = ell(e);
      if (best < 0 || v > vb) {
        best = e;
        vb = v;
      }
    }
    taken |= 1ull << best;
    if (j == 0) top = vb;
    const float w = expf(vb - top);
    gate[j] = w;
    wsum += w;
    idx[j] = base + best;
  }
  for (int j = 0; j < k; ++j) gate[j] = gate[j] / wsum;
}

// topk_rank for groups of at most N heads whose logits sit in registers (v[e],
// e < r <= N): the loops are unrolled over N, so every logit is read by a
// static index and the loads that fill v can all be in flight together.
template <int N>
__device__ inline uint64_t topk_rank_reg(const float (&v)[N], int r, int k, int slot, int* e_slot,
                                         float* gate_slot) {
  uint64_t taken = 0;
  float top = 0.0f, wsum = 0.0f, w_slot = 0.0f;
  int e_s = 0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float vb = 0.0f;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      if (e >= r || ((taken >> e) & 1ull)) continue;
      if (best < 0 || v[e] > vb) {
        best = e;
        vb = v[e];
      }
    }
    taken |= 1ull << best;
    if (j == 0) top = vb;
    const float w = expf(vb - top);
    wsum += w;
    if (j == slot) {
      e_s = best;
      w_slot = w;
    }
  }
  *e_slot = e_s;
  *gate_slot = w_slot / wsum;
  return taken;
}

// The same selection with the same arithmetic, for one rank: returns the mask
// of the kept heads (bit e: head base + e) and sets *e_slot to the group
// position of the slot-th kept head and *gate_slot to its gate. For kernels
// that route inside their own rows instead of reading a router's output.
template <typename Logit>
__device__ inline uint64_t topk_rank(Logit ell, int r, int k, int slot, int* e_slot, float* gate_slot) {
  uint64_t taken = 0;
  float top = 0.0f, wsum = 0.0f, w_slot = 0.0f;
  int e_s = 0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float vb = 0.0f;
    for (int e = 0; e < r; ++e) {
      if ((taken >> e) & 1ull) continue;
      const float v = ell(e);
      if (best < 0 || v > vb) {
        best = e;
        vb = v;
      }
    }
    taken |= 1ull << best;
    if (j == 0) top = vb;
    const float w = expf(vb - top);
    wsum += w;
    if (j == slot) {
      e_s = best;
      w_slot = w;
    }
  }
  *e_slot = e_s;
  *gate_slot = w_slot / wsum;
  return taken;
}

}  // namespace gqa
