// Peak microbenchmarks (measurement support): the rates the path's kernels
// are compared with besides the datasheet peaks of MI355X.
//  * An HBM read stream: every 16-byte word of a buffer read once, two
//    4-wave workgroups per CU (the decode kernel's grid), each streaming a
//    contiguous chunk with eight 16-byte loads in flight per lane. The XOR of
//    all words comes back (one atomic per workgroup), so a test can check that
//    every word was read exactly once. The workgroups finish together, so
//    their atomics on the one result word queue up at the end of the launch:
//    with eight workgroups per CU that queue cost about 10% of a 4 GiB read,
//    with two it is a few microseconds.
//  * An MFMA-only loop: v_mfma_f32_32x32x16_bf16 on register operands, four
//    independent accumulators per wave and two waves per SIMD on every SIMD
//    of the chip. The sum of all accumulators comes back (one atomic per
//    workgroup), so a test can check the work that was counted.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kPeakThreads = 256;
constexpr int kMfmaChains = 4;

// Each workgroup streams one contiguous chunk of the buffer, as a decode
// workgroup streams its share of the KV cache: a step reads 8 x 4 KiB
// (every load instruction of a wave reads 1 KiB), eight loads in flight per lane.
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kPeakThreads) void hbm_read_kernel(const u32x4* buf, size_t n16, unsigned* x_out) {
  __shared__ unsigned red[kPeakThreads / 64];
  constexpr size_t kStep = (size_t)kReadUnroll * kPeakThreads;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = min((size_t)blockIdx.x * per, n16), hi = min(lo + per, n16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  const u32x4* const chunk = buf + lo;
  const size_t n = hi - lo;
  size_t i = threadIdx.x;
  for (; i + (kReadUnroll - 1) * kPeakThreads < n; i += kStep) {
    u32x4 w[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) w[k] = __builtin_nontemporal_load(chunk + i + k * kPeakThreads);
    // Keep the scheduler from pulling the first XOR (and its wait) in between
    // the loads, which would leave two of them in flight instead of eight.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= w[k];
  }
  for (; i < n; i += kPeakThreads) acc ^= chunk[i];
  unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned w = 0u;
#pragma unroll
    for (int k = 0; k < kPeakThreads / 64; ++k) w ^= red[k];
    atomicXor(x_out, w);
  }
}

// operands: 128 bf16x8 (2 KiB): A fragments of the 64 lanes, then B fragments.
__global__ __launch_bounds__(kPeakThreads) void mfma_loop_kernel(const bf16x8* operands, int iters, float* sum_out) {
  __shared__ float red[kPeakThreads / 64];
  const int lane = threadIdx.x & 63;
  const bf16x8 a = operands[lane], b = operands[64 + lane];
  f32x16 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) c[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) c[k] = mfma32x32x16(a, b, c[k]);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[k][e];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float w = 0.0f;
#pragma unroll
    for (int k = 0; k < kPeakThreads / 64; ++k) w += red[k];
    atomicAdd(sum_out, w);
  }
}

int device_cu_count() {
  int n_cu = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  (void)hipGetLastError();
  return n_cu;
}

}  // namespace

hipError_t launch_peak_hbm_read(const void* buf, size_t bytes, unsigned* x_out, hipStream_t stream) {
  const dim3 grid(device_cu_count() * 2), block(kPeakThreads);
  hipLaunchKernelGGL(hbm_read_kernel, grid, block, 0, stream, static_cast<const u32x4*>(buf), bytes / 16, x_out);
  return hipGetLastError();
}

hipError_t launch_peak_mfma_bf16(const void* operands, int iters, float* sum_out, double* flops, hipStream_t stream) {
  // Two 4-wave workgroups per CU: two waves on every SIMD.
  const int n_wg = device_cu_count() * 2;
  *flops = (double)n_wg * (kPeakThreads / 64) * kMfmaChains * (double)iters * (2.0 * 32 * 32 * 16);
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_wg), dim3(kPeakThreads), 0, stream,
                     static_cast<const bf16x8*>(operands), iters, sum_out);
  return hipGetLastError();
}

}  // namespace gqa
