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
//  * The attention tile loop: the work a prefill wave does per 32-key tile of
//    its 32 query rows -- the K and V fragment reads from LDS, S^T = K Q^T
//    (8 MFMAs), the online softmax as the prefill kernel takes it, O^T +=
//    V^T P^T (8 MFMAs) -- on one tile staged in LDS once, every iteration,
//    twelve waves per CU (three per SIMD, the prefill kernel's occupancy),
//    with no global memory traffic and no barrier. Its rate bounds any kernel that does this work per tile on the
//    chip. The tile repeats, so a wave's normalised output is the attention
//    of its 32 queries over the 32 keys, which a test checks.
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

constexpr int kTileWaves = 12;

// qkv: q, k, v of one tile, each [32][128] bf16 row-major. out: [32][128]
// fp32, the normalised output of wave 0 of workgroup 0 (every wave computes
// the same). c = scale * log2(e).
__global__ __launch_bounds__(kTileWaves * 64) __attribute__((amdgpu_waves_per_eu(3))) void attn_tile_kernel(
    const uint16_t* qkv, int iters, float c, float* out) {
  constexpr int D = 128, kPitch = D + 8, vPitch = D + 32;  // the prefill kernel's padded LDS rows
  __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * kPitch], Vs[32 * vPitch];
  const int lane = threadIdx.x & 63, l32 = lane & 31, hq = lane >> 5;
  const uint16_t* const q = qkv;
  const uint16_t* const k = qkv + 32 * D;
  const uint16_t* const v = qkv + 2 * 32 * D;
  for (int x = threadIdx.x; x < 32 * D / 8; x += kTileWaves * 64) {
    const int row = x / (D / 8), col = (x % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(Ks + row * kPitch + col) = *reinterpret_cast<const uint4*>(k + row * D + col);
    *reinterpret_cast<uint4*>(Vs + row * vPitch + col) = *reinterpret_cast<const uint4*>(v + row * D + col);
  }
  __syncthreads();
  // Q^T fragments in registers (lane half hq holds d in [64 hq, 64 hq + 64));
  // K fragments read from LDS as A operands and V^T fragments by transposing
  // reads, per iteration, as the prefill kernel reads them per tile.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(q + l32 * D + hq * (D / 2) + 8 * st);
  const int grp = lane >> 4, i16 = lane & 15;
  const int tr_row = 4 * hq + (i16 >> 2), tr_col = 16 * (grp & 1) + 4 * (i16 & 3);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.0f;
  for (int it = 0; it < iters; ++it) {
    f32x16 s = f32x16{};
    {
      // The row offset is made opaque to the compiler each iteration, so that
      // the fragment reads stay in the loop as they do per tile in the prefill.
      int koff = l32 * kPitch + hq * (D / 2);
      asm volatile("" : "+v"(koff));
      const uint16_t* krow = Ks + koff;
      bf16x8 kf[D / 16];
#pragma unroll
      for (int st = 0; st < D / 16; ++st) kf[st] = *reinterpret_cast<const bf16x8*>(krow + 8 * st);
#pragma unroll
      for (int st = 0; st < D / 16; ++st) s = mfma32x32x16(kf[st], qf[st], s);
    }
    bf16x8 pf[2];
    float lt[2];
    auto probs = [&]() {
      lt[0] = lt[1] = 0.0f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(fmaf(s[8 * u + j], c, -m_ref));
        pf[u] = pack_bf16x8(pv);
        const bf16x2* pp = reinterpret_cast<const bf16x2*>(&pf[u]);
#pragma unroll
        for (int j = 0; j < 4; ++j) lt[u] = __builtin_amdgcn_fdot2_f32_bf16(pp[j], ones, lt[u], false);
      }
    };
    probs();
    if (__any(!(lt[0] + lt[1] <= 256.0f))) {
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; i += 2) mloc = fmaxf(fmaxf(mloc, s[i]), s[i + 1]);
      const float mloc_s = mloc * c;
      const float m_new = fmaxf(m_ref, fmaxf(mloc_s, __shfl_xor(mloc_s, 32)));
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      probs();
    }
    l_run += lt[0] + lt[1];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int voff = (16 * u + tr_row) * vPitch + tr_col;
      asm volatile("" : "+v"(voff));
      const uint16_t* p0 = Vs + voff;
      bf16x8 vf[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[db] = lds_read_tr_pair(p0 + 32 * db, p0 + 8 * vPitch + 32 * db);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = mfma32x32x16(vf[db], pf[u], o[db]);
    }
  }
  const float inv = 1.0f / (l_run + __shfl_xor(l_run, 32));
  if (blockIdx.x == 0 && threadIdx.x < 64) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) out[l32 * D + 32 * db + 8 * (i >> 2) + 4 * hq + (i & 3)] = o[db][i] * inv;
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

hipError_t launch_peak_attn_tile(const void* qkv, int iters, float scale, float* out, double* flops,
                                 hipStream_t stream) {
  const int n_wg = device_cu_count();
  *flops = (double)n_wg * kTileWaves * (double)iters * 16.0 * (2.0 * 32 * 32 * 16);
  hipLaunchKernelGGL(attn_tile_kernel, dim3(n_wg), dim3(kTileWaves * 64), 0, stream, static_cast<const uint16_t*>(qkv),
                     iters, scale * kLog2e, out);
  return hipGetLastError();
}

}  // namespace gqa
