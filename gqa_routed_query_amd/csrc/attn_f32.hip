// Grouped-query attention prefill in fp32 arithmetic throughout, for dense
// GQA and routed GQE rows: fp32 inputs (no bf16 anywhere), and bf16 inputs at
// the head dims below the bf16 MFMA kernel's tiles (16 and 32), upcast exactly
// to fp32 as they are loaded.
//
// Same definition as the bf16 kernel (ml-canon "56 GQA / MQA", PyTorch GQA
// function; IBM Think GQA page, scaled dot-product attention; causal mask
// key j <= t; routed rows per the gist.science GQE explainer, "Architecture et
// Routage"), on the vector ALUs: fp32 inputs leave no dense contraction that
// the bf16 matrix cores could take without rounding the operands.
//
// A workgroup owns a run of token-major rows of one (batch, KV group) and
// stages 32-key K/V tiles in LDS, shared by every query head of the group.
// Each row is handled by LPR lanes, each holding D/LPR of the query and of
// the accumulator; dot products are reduced across those lanes with shuffles.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kBNF = 32;  // keys per tile

struct KArgs {
  const void* q;  // fp32, or bf16 when the kernel's IN_BF16 is set
  const void* k;
  const void* v;
  void* out;
  const int32_t* idx;
  const float* gate;
  int h, g, T, R, r;
  int rows_per_block;
  int n_row_tiles;
  int BG;
  float c;  // scale * log2(e)
  int causal, out_bf16, zero_unselected;
};

template <int D>
__device__ void zero_unselected_rows_f32(const KArgs& a, int b, int gam, int row0, int n_rows) {
  const int R = a.R, r = a.r;
  const int t_lo = div_up(row0, R);
  const int t_hi = (min(row0 + a.rows_per_block, n_rows) - 1) / R;
  if (t_hi < t_lo) return;
  const int n_items = (t_hi - t_lo + 1) * r * D;
  for (int c = threadIdx.x; c < n_items; c += kThreads) {
    const int tt = c / (r * D);
    const int rem = c - tt * r * D;
    const int e = rem / D;
    const int col = rem - e * D;
    const int t = t_lo + tt;
    const int head = gam * r + e;
    const int32_t* sel = a.idx + ((size_t)(b * a.T + t) * a.g + gam) * R;
    bool kept = false;
    for (int j = 0; j < R; ++j) kept |= (sel[j] == head);
    if (kept) continue;
    const size_t off = ((size_t)(b * a.h + head) * a.T + t) * D + col;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[off] = 0;
    else
      static_cast<float*>(a.out)[off] = 0.0f;
  }
}

// Element i of an fp32 or bf16 array, as fp32 (bf16 widens exactly).
template <bool IN_BF16>
__device__ __forceinline__ float load_elt(const void* base, size_t i) {
  if constexpr (IN_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

// Four consecutive elements starting at i (a multiple of 4), as fp32.
template <bool IN_BF16>
__device__ __forceinline__ float4 load_4(const void* base, size_t i) {
  if constexpr (IN_BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
  }
}

template <int D, bool ROUTED, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(KArgs a) {
  constexpr int EPL = D < 32 ? D : 32;  // elements per lane
  constexpr int LPR = D / EPL;          // lanes per row (1, 2 or 4)
  constexpr int RPB = kThreads / LPR;   // rows per block
  __shared__ __attribute__((aligned(16))) float Ks[kBNF * D];
  __shared__ __attribute__((aligned(16))) float Vs[kBNF * D];

  const int bid = blockIdx.x;
  const int bg = bid % a.BG;
  const int tile = a.causal ? (a.n_row_tiles - 1 - bid / a.BG) : (bid / a.BG);
  const int b = bg / a.g;
  const int gam = bg - b * a.g;
  const int tid = threadIdx.x;
  const int part = tid % LPR;
  const int n_rows = a.T * a.R;
  const int row0 = tile * RPB;

  if (ROUTED && a.zero_unselected) zero_unselected_rows_f32<D>(a, b, gam, row0, n_rows);

  const int rho = row0 + tid / LPR;
  const bool row_valid = rho < n_rows;
  const int rho_c = row_valid ? rho : n_rows - 1;
  const int t_row = rho_c / a.R;
  const int slot = rho_c - t_row * a.R;
  int head;
  float gate = 1.0f;
  if (ROUTED) {
    const size_t o = ((size_t)(b * a.T + t_row) * a.g + gam) * a.R + slot;
    head = a.idx[o];
    gate = a.gate[o];
  } else {
    head = gam * a.r + slot;
  }
  const int t_last = (min(row0 + RPB, n_rows) - 1) / a.R;
  const int n_keys = a.causal ? t_last + 1 : a.T;
  const int lim = a.causal ? t_row : a.T - 1;

  float qv[EPL], acc[EPL];
  {
    const size_t q0 = ((size_t)(b * a.h + head) * a.T + t_row) * D + part * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      qv[e] = load_elt<IN_BF16>(a.q, q0 + e);
      acc[e] = 0.0f;
    }
  }
  float m_run = -INFINITY, l_run = 0.0f;
  const size_t kv0 = (size_t)bg * a.T * D;

  for (int key0 = 0; key0 < n_keys; key0 += kBNF) {
    __syncthreads();
    for (int c = tid; c < kBNF * D / 4; c += kThreads) {
      const int row = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      const int key = key0 + row;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (key < a.T) {
        kk = load_4<IN_BF16>(a.k, kv0 + (size_t)key * D + col);
        vv = load_4<IN_BF16>(a.v, kv0 + (size_t)key * D + col);
      }
      *reinterpret_cast<float4*>(Ks + row * D + col) = kk;
      *reinterpret_cast<float4*>(Vs + row * D + col) = vv;
    }
    __syncthreads();

    float s[kBNF];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBNF; ++j) {
      const float* kr = Ks + j * D + part * EPL;
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], kr[e], dot);
#pragma unroll
      for (int w = 1; w < LPR; w <<= 1) dot += __shfl_xor(dot, w);
      s[j] = (key0 + j <= lim) ? dot : -INFINITY;
      mloc = fmaxf(mloc, s[j]);
    }
    const float m_new = fmaxf(m_run, mloc * a.c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kBNF; ++j) {
      const float p = fast_exp2(fmaf(s[j], a.c, -m_new));
      l_run += p;
      const float* vr = Vs + j * D + part * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vr[e], acc[e]);
    }
  }

  if (row_valid) {
    const float inv = gate / l_run;
    const size_t off = ((size_t)(b * a.h + head) * a.T + t_row) * D + part * EPL;
    if (a.out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + off;
#pragma unroll
      for (int e = 0; e < EPL; e += 2) {
        const uint32_t w = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
        o[e] = static_cast<uint16_t>(w & 0xffffu);
        o[e + 1] = static_cast<uint16_t>(w >> 16);
      }
    } else {
      float* o = static_cast<float*>(a.out) + off;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
    }
  }
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  constexpr int EPL = D < 32 ? D : 32;
  constexpr int RPB = kThreads / (D / EPL);
  KArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.idx = p.idx;
  a.gate = p.gate;
  a.h = p.h;
  a.g = p.g;
  a.T = p.T;
  a.R = p.R;
  a.r = p.h / p.g;
  a.rows_per_block = RPB;
  a.n_row_tiles = div_up(p.T * p.R, RPB);
  a.BG = p.B * p.g;
  a.c = p.scale * kLog2e;
  a.causal = p.causal;
  a.out_bf16 = p.out_bf16;
  a.zero_unselected = p.zero_unselected;
  const dim3 grid(a.n_row_tiles * a.BG), block(kThreads);
  if (p.in_bf16) {
    if (p.idx)
      hipLaunchKernelGGL((attn_f32_kernel<D, true, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_f32_kernel<D, false, true>), grid, block, 0, stream, a);
  } else {
    if (p.idx)
      hipLaunchKernelGGL((attn_f32_kernel<D, true, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_f32_kernel<D, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

bool attn_f32_supports(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) {
  if (p.out_slots || p.q_b || p.kv_b || p.o_b || p.o_h || p.o_t || p.q_shared)
    return hipErrorInvalidValue;  // default layout only
  if (p.in_bf16 && p.d > 32) return hipErrorInvalidValue;  // bf16 at d >= 64 runs on the MFMA kernel
  switch (p.d) {
    case 16: return launch_d<16>(p, stream);
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
