// The renormalised weighted-sum slot of the GQE output build.
//
// gist.science explainer of "Grouped Query Experts", section "Architecture et
// Routage", output construction: besides the hard concatenation of the k
// experts kept in a group, the layer forms a weighted sum of their outputs
// with the router probabilities renormalised over the k kept (the gates).
// For every (batch, token, group): wsum = sum_j gate_j * concat_j.
//
// HBM-bound elementwise pass: one thread per 8 consecutive output elements,
// reading the k kept rows' matching 8 elements (16 or 32 bytes each).
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

__global__ __launch_bounds__(256) void wsum_kernel(WsumParams p) {
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = p.d / 8;
  if (item >= p.n * per_row) return;
  const long long n = item / per_row;
  const int c = (int)(item - n * per_row) * 8;
  float acc[8] = {};
  for (int j = 0; j < p.k; ++j) {
    const float gj = p.gate[n * p.k + j];
    const size_t off = ((size_t)n * p.k + j) * p.d + c;
    if (p.bf16) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(p.concat) + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += gj * (float)x[e];
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.concat) + off);
      const float4 x0 = src[0], x1 = src[1];
      acc[0] += gj * x0.x; acc[1] += gj * x0.y; acc[2] += gj * x0.z; acc[3] += gj * x0.w;
      acc[4] += gj * x1.x; acc[5] += gj * x1.y; acc[6] += gj * x1.z; acc[7] += gj * x1.w;
    }
  }
  const size_t o = (size_t)n * p.d + c;
  if (p.bf16) {
    *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(p.wsum) + o) = pack_bf16x8(acc);
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.wsum) + o);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

hipError_t launch_wsum(const WsumParams& p, hipStream_t stream) {
  const long long items = p.n * (p.d / 8);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(wsum_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
