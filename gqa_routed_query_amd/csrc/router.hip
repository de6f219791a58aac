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
// heads as the 32 A rows and the tokens as the 32 B columns. x is staged
// through LDS in 1024-column chunks (2 KiB of each of the 32 token rows), each
// wave instruction loading 1 KiB of one row, double-buffered in registers;
// workgroups start at different chunks so that the whole chip does not read
// the same column window (rows d_model apart) at once. The 8 waves split each
// chunk's columns for the MFMAs, read W_r from L2 (256 KiB at h=32,
// d_model=4096) one chunk ahead, and reduce through LDS. The selection then
// reads the summed logits from LDS, one thread per (token, group).
#include "common.h"
#include "launch.h"
#include "topk.h"

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
constexpr int kKC = 1024;   // d_model columns per LDS chunk (2 KiB of a bf16 row)
constexpr int kXPitch = kKC + 8;  // 16-byte pad: B-operand reads of 16 rows hit distinct banks

struct ProjArgs {
  const uint16_t* x;  // [n_tok, dm] bf16
  const uint16_t* w;  // [h, dm] bf16
  float* logits;      // [n_tok, h] or null
  int32_t* idx;       // [n_tok, g, k]
  float* gate;        // [n_tok, g, k]
  int n_tok, dm, h, g, k;
};

template <int HB>  // head blocks of 32 (h <= 32 * HB)
__global__ __launch_bounds__(kPW * 64) void router_proj_kernel(ProjArgs a) {
  constexpr int kPitch = kPTok + 1;
  constexpr int kXElems = kPTok * kXPitch;
  constexpr int kRedFloats = kPW * HB * 32 * kPitch;
  constexpr int kSmem = (2 * kXElems * 2 > kRedFloats * 4) ? 2 * kXElems * 2 : kRedFloats * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);  // two chunk buffers [kPTok][kXPitch]
  float* red = reinterpret_cast<float*>(smem);       // reused after the last chunk

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hq = lane >> 5;
  const int tok0 = blockIdx.x * kPTok;

  // Chunk loads: wave w fetches rows 4w .. 4w+3 of the tile, one instruction
  // per row, lane l taking the row's 16-byte piece l (1 KiB contiguous).
  constexpr int kRowsPerWave = kPTok / kPW;
  constexpr int kPieces = kKC / 512;
  u32x4 xr[kRowsPerWave * kPieces];
  auto load_chunk = [&](int c0, int width) {
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
      for (int q = 0; q < kPieces; ++q) {
        const int t = tok0 + wave * kRowsPerWave + j;
        const int col = q * 512 + lane * 8;
        const bool ok = t < a.n_tok && col < width;
        xr[j * kPieces + q] = ok ? *reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.dm + c0 + col)
                                 : u32x4{0u, 0u, 0u, 0u};
      }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
      for (int q = 0; q < kPieces; ++q)
        *reinterpret_cast<u32x4*>(xs + buf * kXElems + (wave * kRowsPerWave + j) * kXPitch + q * 512 + lane * 8) =
            xr[j * kPieces + q];
  };

  bool w_ok[HB];
  const uint16_t* wr[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = hb * 32 + l32;
    w_ok[hb] = head < a.h;
    wr[hb] = a.w + (size_t)(w_ok[hb] ? head : 0) * a.dm + 8 * hq;
  }
  f32x16 acc[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16{};

  // A chunk's columns are split over the waves: wave w takes
  // [w * width/8, (w+1) * width/8), at most kSteps 16-wide MFMA steps (lane
  // half hq holds 8 of each step's 16). W_r fragments of the next chunk are
  // fetched from L2 together with its x rows.
  constexpr int kSteps = kKC / kPW / 16;
  bf16x8 wn[HB][kSteps];
  auto load_w = [&](int c0, int width) {
    const int per = width / kPW;
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        wn[hb][st] = (16 * st < per && w_ok[hb])
                         ? *reinterpret_cast<const bf16x8*>(wr[hb] + c0 + wave * per + 16 * st)
                         : bf16x8{};
  };

  const int n_chunks = div_up(a.dm, kKC);
  const int c_first = blockIdx.x % n_chunks;
  auto chunk_col = [&](int c) { return ((c + c_first) % n_chunks) * kKC; };
  load_chunk(chunk_col(0), min(kKC, a.dm - chunk_col(0)));
  load_w(chunk_col(0), min(kKC, a.dm - chunk_col(0)));
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    const int c0 = chunk_col(c);
    const int per = min(kKC, a.dm - c0) / kPW;  // a multiple of 16
    bf16x8 wc[HB][kSteps];
#pragma unroll
    for (int st = 0; st < kSteps; ++st)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) wc[hb][st] = wn[hb][st];
    if (c + 1 < n_chunks) {
      const int n0 = chunk_col(c + 1);
      load_chunk(n0, min(kKC, a.dm - n0));
      load_w(n0, min(kKC, a.dm - n0));
    }
    const uint16_t* xb_row = xs + (c & 1) * kXElems + l32 * kXPitch + wave * per + 8 * hq;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (16 * st >= per) break;
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(xb_row + 16 * st);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x16(wc[hb][st], xb, acc[hb]);
    }
    if (c + 1 < n_chunks) store_chunk((c + 1) & 1);
    __syncthreads();
  }

  // acc[hb][i] = partial logit of head hb*32 + 8(i/4) + 4hq + i%4, token l%32
  // (the LDS chunks are no longer read: the last barrier above).
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int head = hb * 32 + 8 * (i >> 2) + 4 * hq + (i & 3);
      red[(wave * HB * 32 + head) * kPitch + l32] = acc[hb][i];
    }
  __syncthreads();

  const int r = a.h / a.g;
  for (int item = tid; item < kPTok * a.g; item += kPW * 64) {
    const int t = item % kPTok;
    const int gam = item / kPTok;
    if (tok0 + t >= a.n_tok) continue;
    const size_t row = (size_t)(tok0 + t);
    // Sum the waves' partials in place (this item owns column t of its heads).
    for (int e = 0; e < r; ++e) {
      const int head = gam * r + e;
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kPW; ++wv) v += red[(wv * HB * 32 + head) * kPitch + t];
      red[head * kPitch + t] = v;
      if (a.logits) a.logits[row * a.h + head] = v;
    }
    topk_select([&](int e) { return red[(gam * r + e) * kPitch + t]; }, r, a.k, gam * r,
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
