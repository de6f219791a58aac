// GQE router kernels: the top-k selection of query-head experts per (token,
// KV group) from given logits, and the router projection fused with it.
//
// gist.science explainer of "Grouped Query Experts: Mixture-of-Experts on GQA
// Self-Attention", section "Architecture et Routage": per token the router
// keeps k experts inside each GQA group (the K/V heads stay dense), weighted by
// the router probabilities renormalised over the k kept (topk.h).
//
// router_topk_kernel: one lane per (batch, token, group); the group's h/g
// logits are contiguous, so a lane reads them and selects in registers.
//
// router_proj_kernel: logits = x W_r^T for a tile of 32 tokens, then the same
// selection. The contraction is skinny (h <= 64 outputs per token over d_model
// inputs) and HBM-bound on x, so it runs on v_mfma_f32_32x32x16_bf16 with the
// heads as the 32 A rows and the tokens as the 32 B columns. x and W_r move
// to LDS by DMA (global_load_lds_dwordx4) in 256-column chunks, with three
// chunks in flight behind the one in use (two for h > 32), no registers
// staging them. Workgroups start at different chunks, so that the whole chip
// does not read the same column window (rows d_model apart) at once. The 8
// waves split each chunk's columns for the MFMAs and reduce through LDS. The
// selection then reads the summed logits from LDS, one thread per (token,
// group).
#include "common.h"
#include "launch.h"
#include "topk.h"

#include <type_traits>

namespace gqa {
namespace {

__global__ __launch_bounds__(256) void router_topk_kernel(RouterParams p) {
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n_items = (long long)p.B * p.T * p.g;
  if (item >= n_items) return;
  const int r = p.h / p.g;
  const int gam = (int)(item % p.g);
  const long long bt = item / p.g;
  const float* lg = p.logits + bt * p.h + (long long)gam * r;
  topk_select([&](int e) { return lg[e]; }, r, p.k, gam * r, p.idx + item * p.k, p.gate + item * p.k);
}


constexpr int kPW = 8;      // waves per workgroup
constexpr int kPTok = 32;   // tokens per workgroup
constexpr int kKC = 256;    // d_model columns per chunk (512 bytes of a bf16 row)
constexpr int kRowEl = kKC;               // LDS row pitch in elements: 512 B, XOR-swizzled granules
constexpr int kTileEl = 32 * kRowEl;      // one 32-row tile (x rows or a block of 32 W_r rows)
constexpr int kSteps = kKC / kPW / 16;    // 16-wide MFMA k-steps per wave and chunk (2)

struct ProjArgs {
  const uint16_t* x;  // [n_tok, dm] bf16
  const uint16_t* w;  // [h, dm] bf16
  float* logits;      // [n_tok, h] or null
  int32_t* idx;       // [n_tok, g, k]
  float* gate;        // [n_tok, g, k]
  int n_tok, dm, h, g, k;
};

// LDS granule (16 bytes) of row r, logical granule q of a 512-byte row: the
// granule index is XORed with r mod 8, so the 16-byte reads of one granule
// column by rows 0..7 (one MFMA operand step) fall in eight different banks.
__device__ __forceinline__ int swz(int r, int q) { return r * (kRowEl / 8) + (q ^ (r & 7)); }

// Byte address of an LDS location, for ds_read operands.
__device__ __forceinline__ unsigned lds_addr(const uint16_t* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

template <int HB>  // head blocks of 32 (h <= 32 * HB)
__global__ __launch_bounds__(kPW * 64) void router_proj_kernel(ProjArgs a) {
  // Buffers: the chunk in use and NB-1 in flight. Each holds the chunk's 32
  // token rows and its HB blocks of 32 W_r rows. One array per buffer, so that
  // with the buffer fixed at compile time the compiler can tell the DMA into
  // one buffer from the reads of another.
  constexpr int NB = HB == 1 ? 4 : 3;
  constexpr int kBufEl = (1 + HB) * kTileEl;
  __shared__ __attribute__((aligned(16))) uint16_t B0[kBufEl], B1[kBufEl], B2[kBufEl];
  __shared__ __attribute__((aligned(16))) uint16_t B3[NB == 4 ? kBufEl : 8];
  constexpr int kDmaPerWave = (1 + HB) * 16 / kPW;  // 1 KiB DMA instructions (two rows each) per wave and chunk

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hq = lane >> 5;
  const int tok0 = blockIdx.x * kPTok;
  const int n_chunks = div_up(a.dm, kKC);
  // Workgroups start at different chunks, so that the chip does not read the
  // same column window of every row at once.
  const int c_first = blockIdx.x % n_chunks;
  auto chunk_col = [&](int c) { return ((c + c_first) % n_chunks) * kKC; };
  auto buf = [&](auto nb) -> uint16_t* {
    return nb.value == 0 ? B0 : nb.value == 1 ? B1 : nb.value == 2 ? B2 : B3;
  };

  // Chunk c into buffer nb by DMA. Instruction i of the chunk moves rows
  // 2i, 2i+1 of the chunk's (1 + HB) 32-row tiles (token rows, then W_r rows):
  // lane l moves granule l % 32 of row 2i + l / 32, written at its swizzled
  // place, i.e. loaded from the granule that belongs there. Rows past n_tok or
  // h and columns past the row end load valid memory that is never used, so
  // every chunk costs kDmaPerWave instructions per wave, which `step` counts on.
  auto issue = [&](int c, auto nb) {
    uint16_t* const Xb = buf(nb);
    const int c0 = chunk_col(c);
    const int width = min(kKC, a.dm - c0);
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const int i = wave * kDmaPerWave + j;  // 0 .. (1+HB)*16-1, uniform
      const int tl = i / 16;                 // tile: 0 = tokens, 1.. = W_r head blocks
      const int r = 2 * (i % 16) + lane / 32;
      const int q = (lane & 31) ^ (r & 7);   // logical granule stored at physical granule lane % 32
      const int col = q * 8 < width ? q * 8 : 0;
      const uint16_t* src = tl == 0 ? a.x + (size_t)min(tok0 + r, a.n_tok - 1) * a.dm
                                    : a.w + (size_t)min((tl - 1) * 32 + r, a.h - 1) * a.dm;
      auto* const dst = (__attribute__((address_space(3))) void*)(Xb + tl * kTileEl + (i % 16) * 2 * kRowEl);
      if (tl == 0)  // x is read once: nontemporal
        __builtin_amdgcn_global_load_lds(src + c0 + col, dst, 16, 0, 2);
      else          // W_r is read by every workgroup
        __builtin_amdgcn_global_load_lds(src + c0 + col, dst, 16, 0, 0);
    }
  };

  f32x16 acc[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16{};
  using N0 = std::integral_constant<int, 0>;
  using N1 = std::integral_constant<int, 1>;
  using N2 = std::integral_constant<int, 2>;
  using N3 = std::integral_constant<int, 3>;
  issue(0, N0{});
  if (n_chunks > 1) issue(1, N1{});
  if (NB == 4 && n_chunks > 2) issue(2, N2{});

  // Chunk c in buffer nb. Before the barrier each wave waits for its own DMA
  // of chunk c; the NB-2 chunks issued after it stay in flight.
  constexpr int kAhead = (NB - 2) * kDmaPerWave;
  auto step = [&](int c, auto nb) {
    if (c + NB - 2 < n_chunks) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kAhead) : "memory");
    } else if (NB == 4 && c + 1 < n_chunks) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kDmaPerWave) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // The buffer NB-1 steps ahead held chunk c-1, which every wave has finished.
    if (c + NB - 1 < n_chunks) issue(c + NB - 1, std::integral_constant<int, (nb.value + NB - 1) % NB>{});
    const uint16_t* const Xb = buf(nb);
    const int per = min(kKC, a.dm - chunk_col(c)) / kPW;  // a multiple of 16
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (16 * st >= per) break;
      const int q = (wave * per + 16 * st + 8 * hq) / 8;  // logical granule of this step
      const unsigned ax = lds_addr(Xb + swz(l32, q) * 8);
      // The step's operand reads, written out with their own wait: the
      // compiler's tracking of the DMAs into the other buffers would otherwise
      // put a full vmcnt(0) wait before the first read after the loop's back
      // edge, draining the chunks in flight.
      bf16x8 xb, wa[HB];
      if (HB == 1) {
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(xb), "=v"(wa[0])
                     : "v"(ax), "n"(kTileEl * 2));
      } else {
        asm volatile(
            "ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:%4\n\tds_read_b128 %2, %3 offset:%5\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(xb), "=v"(wa[0]), "=v"(wa[HB - 1])
            : "v"(ax), "n"(kTileEl * 2), "n"(kTileEl * 4));
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x16(wa[hb], xb, acc[hb]);
    }
  };
  for (int c = 0; c < n_chunks; c += NB) {
    step(c, N0{});
    if (c + 1 < n_chunks) step(c + 1, N1{});
    if (c + 2 < n_chunks) step(c + 2, N2{});
    if (NB == 4 && c + 3 < n_chunks) step(c + 3, N3{});
  }
  __syncthreads();

  // acc[hb][i] = partial logit of head hb*32 + 8(i/4) + 4hq + i%4, token l%32.
  // Reduce over the waves through LDS, one block of 32 heads at a time.
  constexpr int kPitch = kPTok;  // writes and reads both run along consecutive tokens
  static_assert(kPW * 32 * kPitch * 4 <= kBufEl * 2, "a reduction round fits in one buffer");
  float* const red = reinterpret_cast<float*>(B0);
  float* const lg = reinterpret_cast<float*>(B1);  // summed logits [HB*32][kPitch]
  const int r = a.h / a.g;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wave * 32 + 8 * (i >> 2) + 4 * hq + (i & 3)) * kPitch + l32] = acc[hb][i];
    __syncthreads();
    for (int item = tid; item < 32 * kPTok; item += kPW * 64) {
      const int hh = item / kPTok, t = item % kPTok;
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kPW; ++wv) v += red[(wv * 32 + hh) * kPitch + t];
      const int head = hb * 32 + hh;
      lg[head * kPitch + t] = v;
      if (a.logits && head < a.h && tok0 + t < a.n_tok) a.logits[(size_t)(tok0 + t) * a.h + head] = v;
    }
    __syncthreads();
  }
  for (int item = tid; item < kPTok * a.g; item += kPW * 64) {
    const int t = item % kPTok;
    const int gam = item / kPTok;
    if (tok0 + t >= a.n_tok) continue;
    const size_t row = (size_t)(tok0 + t);
    topk_select([&](int e) { return lg[(gam * r + e) * kPitch + t]; }, r, a.k, gam * r,
                a.idx + (row * a.g + gam) * a.k, a.gate + (row * a.g + gam) * a.k);
  }
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

bool router_proj_supports(int d_model, int h) {
  return d_model >= kPW * 16 && d_model % (kPW * 16) == 0 && h >= 1 && h <= 64;
}

hipError_t launch_router_proj(const RouterProjParams& p, hipStream_t stream) {
  if (p.n_tok == 0) return hipSuccess;
  ProjArgs a{static_cast<const uint16_t*>(p.x), static_cast<const uint16_t*>(p.w), p.logits, p.idx,
             p.gate, p.n_tok, p.d_model, p.h, p.g, p.k};
  const dim3 grid((unsigned)div_up(p.n_tok, kPTok)), block(kPW * 64);
  if (p.h <= 32)
    hipLaunchKernelGGL(router_proj_kernel<1>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(router_proj_kernel<2>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace gqa
