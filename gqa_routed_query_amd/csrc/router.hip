// GQE router selection: for every (batch, token, KV group) keep the top-k of
// the group's h/g query-head experts and compute their gates.
//
// gist.science explainer of "Grouped Query Experts: Mixture-of-Experts on GQA
// Self-Attention", section "Architecture et Routage": per token the router
// keeps k experts inside each GQA group (the K/V heads stay dense), and the
// kept experts are weighted by the router probabilities renormalised over the
// k kept. Renormalising over the kept set cancels the softmax denominator, so
// gate_j = exp(l_j - l_max) / sum over kept of exp(l - l_max).
//
// Rank order: higher logit first; equal logits keep the lower head index
// first. The raw fp32 logits are compared with '>' only, so the selection is
// exact and +0.0 / -0.0 count as equal.
//
// One lane per (batch, token, group): the group's h/g logits are contiguous,
// so a lane reads them with vector loads and selects in registers; there is
// nothing to share across lanes for the group sizes GQA uses (h/g <= 64).
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kMaxR = 64;

__global__ __launch_bounds__(256) void router_topk_kernel(RouterParams p) {
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n_items = (long long)p.B * p.T * p.g;
  if (item >= n_items) return;
  const int r = p.h / p.g;
  const int gam = (int)(item % p.g);
  const long long bt = item / p.g;
  const float* lg = p.logits + bt * p.h + (long long)gam * r;
  float ell[kMaxR];
  for (int e = 0; e < r; ++e) ell[e] = lg[e];
  uint64_t taken = 0;
  float top = 0.0f, wsum = 0.0f;
  float w[kMaxR];
  int32_t* idx = p.idx + item * p.k;
  for (int j = 0; j < p.k; ++j) {
    int best = -1;
    for (int e = 0; e < r; ++e) {
      if ((taken >> e) & 1ull) continue;
      if (best < 0 || ell[e] > ell[best]) best = e;
    }
    taken |= 1ull << best;
    if (j == 0) top = ell[best];
    w[j] = expf(ell[best] - top);
    wsum += w[j];
    idx[j] = gam * r + best;
  }
  float* gate = p.gate + item * p.k;
  for (int j = 0; j < p.k; ++j) gate[j] = w[j] / wsum;
}

}  // namespace

hipError_t launch_router(const RouterParams& p, hipStream_t stream) {
  const long long n_items = (long long)p.B * p.T * p.g;
  if (n_items == 0) return hipSuccess;
  const int threads = 256;
  const dim3 grid((unsigned)((n_items + threads - 1) / threads));
  hipLaunchKernelGGL(router_topk_kernel, grid, dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
