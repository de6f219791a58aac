// Grouped-query attention decode over a KV cache: one new query token per
// sequence, bf16 cache, fp32 accumulation, split-K with a log-sum-exp merge.
//
// What is computed (aiunderstanding.org "Attention aux requetes groupees",
// section "Plongee profonde"; ml-canon "56 GQA / MQA", section on where the
// KV-cache saving comes from): the query of each of the h heads attends to the
// cached keys 0 .. lens[b]-1 of its KV group and mixes the matching cached
// values. Decode reads the whole cache once per step, so its cost is the
// cache bytes, 2 * g * d * lens[b] * sizeof(bf16) per sequence -- the reason
// GQA shrinks it by h/g.
//
// Design for CDNA4 (HBM-bound):
//  * A workgroup of 4 waves owns one (batch, KV group, key chunk). Every cached
//    K/V row of the chunk is read once, with coalesced 16-byte loads, and
//    serves all h/g query heads of the group from registers.
//  * Per 32-key sub-block a wave computes S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16 (heads are the 16-wide B columns; groups with
//    fewer than 16 heads leave columns idle -- the matrix cores have far more
//    headroom than HBM), runs the online softmax on its lanes, and accumulates
//    O^T += V^T P^T with V transposed by ds_read_b64_tr_b16 from a wave-private
//    LDS buffer.
//  * The 4 waves combine their (max, sum, accumulator) in LDS and the block
//    writes one partial per (head, chunk); a second kernel merges the chunks
//    by log-sum-exp. A problem with a single chunk skips the merge and writes
//    the normalised output directly.
//  * Cache rows at or beyond lens[b] are never loaded: padding may hold
//    anything, NaN included.
#include <cstdlib>

#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSub = 32;  // keys per wave sub-block

template <int D>
struct DTile {
  static constexpr int kPitch = D + 8;   // 16-byte pad: A-operand reads of 16 rows hit distinct banks
  static constexpr int vPitch = D + 16;  // 32-byte pad: 8 rows of a transposing read hit distinct banks
  static constexpr int kElems = kSub * kPitch;
  static constexpr int vElems = kSub * vPitch;
  static constexpr int wElems = kElems + vElems;    // one wave's LDS staging area
  static constexpr int kCPR = D / 8;
  static constexpr int kLoads = kSub * kCPR / 64;   // 16-byte loads per lane per sub-block (K or V)
  static constexpr int kDS = D / 32;                // 32-wide reduction steps for S^T
};

struct KArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* lens;
  void* out;
  float* part_acc;
  float* part_ml;
  int h, g, r, T_max;
  int chunk, n_split;
  float c;
  int out_bf16;
};

template <int D, int HB>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(KArgs a) {
  using L = DTile<D>;
  constexpr int kComb = kWaves * 16 * (D + 2);  // floats per head block of the combine
  constexpr int kSmemBytes =
      (kWaves * L::wElems * 2 > kComb * 4) ? kWaves * L::wElems * 2 : kComb * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];

  const int split = blockIdx.x % a.n_split;
  const int bg = blockIdx.x / a.n_split;
  const int b = bg / a.g;
  const int gam = bg - b * a.g;
  const int len = min(max(a.lens[b], 0), a.T_max);
  const int s0 = split * a.chunk;
  const int tid = threadIdx.x;
  if (s0 >= len) {
    // The merge never reads chunks past lens[b]; with a single chunk there is
    // no merge, so an empty sequence writes its zero rows here.
    if (a.n_split == 1) {
      for (int x = tid; x < a.r * D; x += kThreads) {
        const size_t off = ((size_t)b * a.h + gam * a.r) * D + x;
        if (a.out_bf16)
          static_cast<uint16_t*>(a.out)[off] = 0;
        else
          static_cast<float*>(a.out)[off] = 0.0f;
      }
    }
    return;
  }
  const int s1 = min(s0 + a.chunk, len);

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int i16 = lane & 15;
  uint16_t* Kw = reinterpret_cast<uint16_t*>(smem) + wave * L::wElems;
  uint16_t* Vw = Kw + L::kElems;

  // Q^T fragments: column = head hb*16 + l%16 of this group; lane group grp
  // holds d in [grp*D/4, grp*D/4 + D/4), 8 per reduction step.
  bf16x8 qf[HB][L::kDS];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int e = hb * 16 + i16;
    const uint16_t* qrow = a.q + ((size_t)b * a.h + gam * a.r + min(e, a.r - 1)) * D + grp * (D / 4);
#pragma unroll
    for (int ds = 0; ds < L::kDS; ++ds) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 8 * ds);
      if (e >= a.r) x = bf16x8{};
      qf[hb][ds] = x;
    }
  }

  f32x4 o[HB][D / 16];
  float m_run[HB], l_run[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m_run[hb] = -INFINITY;
    l_run[hb] = 0.0f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[hb][db] = f32x4{};
  }

  const size_t cache_base = (size_t)bg * a.T_max * D;
  const uint16_t* kbase = a.kc + cache_base;
  const uint16_t* vbase = a.vc + cache_base;
  const int tr_row = 4 * grp + (i16 >> 2);
  const int tr_col = 4 * (i16 & 3);

  // Coalesced 16-byte loads of one 32-key sub-block of K and V into
  // registers: chunk c = lane + 64i is row c / (D/8), column (c % (D/8)) * 8.
  // Rows at or past s1 are not loaded (they may hold anything) and stage as 0.
  uint4 kr[L::kLoads], vr[L::kLoads];
  auto load_sub = [&](int sb0) {
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) {
      const int cidx = lane + 64 * i;
      const int key = sb0 + cidx / L::kCPR;
      const size_t off = (size_t)key * D + (cidx % L::kCPR) * 8;
      const bool ok = key < s1;
      kr[i] = ok ? *reinterpret_cast<const uint4*>(kbase + off) : make_uint4(0u, 0u, 0u, 0u);
      vr[i] = ok ? *reinterpret_cast<const uint4*>(vbase + off) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  const int sb_first = s0 + wave * kSub;
  if (sb_first < s1) load_sub(sb_first);
  for (int sb0 = sb_first; sb0 < s1; sb0 += kWaves * kSub) {
    // Stage this sub-block in the wave's LDS area, then start loading the
    // next one so that its HBM reads overlap the math below.
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) {
      const int cidx = lane + 64 * i;
      const int row = cidx / L::kCPR, col = (cidx % L::kCPR) * 8;
      *reinterpret_cast<uint4*>(Kw + row * L::kPitch + col) = kr[i];
      *reinterpret_cast<uint4*>(Vw + row * L::vPitch + col) = vr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (sb0 + kWaves * kSub < s1) load_sub(sb0 + kWaves * kSub);
    // K in the A-operand layout: lane holds key sb0 + 16kb + l%16 and d in
    // [grp*D/4, grp*D/4 + D/4), 8 per reduction step.
    bf16x8 kf[2][L::kDS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < L::kDS; ++ds)
        kf[kb][ds] = *reinterpret_cast<const bf16x8*>(Kw + (16 * kb + i16) * L::kPitch + grp * (D / 4) + 8 * ds);

#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      // S^T[key][head]: lane holds keys sb0 + 16kb + 4grp + i for its head column.
      f32x4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4{};
#pragma unroll
        for (int ds = 0; ds < L::kDS; ++ds) s[kb] = mfma16x16x32(kf[kb][ds], qf[hb][ds], s[kb]);
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (sb0 + 16 * kb + 4 * grp + i >= s1) s[kb][i] = -INFINITY;
          mloc = fmaxf(mloc, s[kb][i]);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run[hb], mloc * a.c);
      const float alpha = fast_exp2(m_run[hb] - m_new);
      m_run[hb] = m_new;
      float pv[8];
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = fast_exp2(fmaf(s[j >> 2][j & 3], a.c, -m_new));
        psum += pv[j];
      }
      l_run[hb] = l_run[hb] * alpha + psum;
      const bf16x8 pf = pack_bf16x8(pv);
      // O^T += V^T P^T: element j is key 4grp + j (j < 4) or 16 + 4grp + j-4.
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const uint16_t* p0 = Vw + tr_row * L::vPitch + 16 * db + tr_col;
        const bf16x8 vf = lds_read_tr_pair(p0, p0 + 16 * L::vPitch);
        o[hb][db] = mfma16x16x32(vf, pf, o[hb][db] * alpha);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Combine the 4 waves, one head block at a time, through LDS.
  float* comb = reinterpret_cast<float*>(smem);
  const bool single = (a.n_split == 1);
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float lsum = l_run[hb];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    __syncthreads();  // LDS is free (V buffers or the previous head block)
    float* w = comb + (wave * 16 + i16) * (D + 2);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[16 * db + 4 * grp + i] = o[hb][db][i];
    if (grp == 0) {
      w[D] = m_run[hb];
      w[D + 1] = lsum;
    }
    __syncthreads();
    // 16 heads x D values over 256 threads.
    for (int x = tid; x < 16 * D; x += kThreads) {
      const int hh = x / D;
      const int d = x - hh * D;
      const int e = hb * 16 + hh;
      float M = -INFINITY;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, comb[(wv * 16 + hh) * (D + 2) + D]);
      float acc = 0.0f, den = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        const float* src = comb + (wv * 16 + hh) * (D + 2);
        const float mw = src[D];
        const float sc = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
        acc += sc * src[d];
        den += sc * src[D + 1];
      }
      if (e < a.r) {
        const size_t row = (size_t)b * a.h + gam * a.r + e;
        if (single) {
          const float y = acc / den;
          if (a.out_bf16)
            static_cast<uint16_t*>(a.out)[row * D + d] = static_cast<uint16_t>(pack_bf16x2(y, 0.0f) & 0xffffu);
          else
            static_cast<float*>(a.out)[row * D + d] = y;
        } else {
          const size_t pidx = row * a.n_split + split;
          a.part_acc[pidx * D + d] = acc;
          if (d == 0) {
            a.part_ml[pidx * 2 + 0] = M;
            a.part_ml[pidx * 2 + 1] = den;
          }
        }
      }
    }
  }
}

// One wave per (batch, head): merge the chunk partials by log-sum-exp.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(KArgs a) {
  const int row = blockIdx.x;  // b*h + head
  const int b = row / a.h;
  const int len = min(max(a.lens[b], 0), a.T_max);
  const int n_valid = div_up(len, a.chunk);
  const int lane = threadIdx.x;
  constexpr int EPL = D / 64;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  float M = -INFINITY;
  for (int s = 0; s < n_valid; ++s) M = fmaxf(M, a.part_ml[((size_t)row * a.n_split + s) * 2]);
  float den = 0.0f;
  for (int s = 0; s < n_valid; ++s) {
    const size_t pidx = (size_t)row * a.n_split + s;
    const float sc = fast_exp2(a.part_ml[pidx * 2] - M);
    den += sc * a.part_ml[pidx * 2 + 1];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += sc * a.part_acc[pidx * D + lane + 64 * e];
  }
  const float inv = n_valid > 0 ? 1.0f / den : 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float y = acc[e] * inv;
    const size_t off = (size_t)row * D + lane + 64 * e;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[off] = static_cast<uint16_t>(pack_bf16x2(y, 0.0f) & 0xffffu);
    else
      static_cast<float*>(a.out)[off] = y;
  }
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  KArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const uint16_t*>(p.k_cache);
  a.vc = static_cast<const uint16_t*>(p.v_cache);
  a.lens = p.lens;
  a.out = p.out;
  a.part_acc = p.part_acc;
  a.part_ml = p.part_ml;
  a.h = p.h;
  a.g = p.g;
  a.r = p.h / p.g;
  a.T_max = p.T_max;
  a.chunk = p.chunk;
  a.n_split = p.n_split;
  a.c = p.scale * kLog2e;
  a.out_bf16 = p.out_bf16;
  const dim3 grid(p.B * p.g * p.n_split), block(kThreads);
  const int hb = div_up(a.r, 16);
  if (hb == 1)
    hipLaunchKernelGGL((decode_split_kernel<D, 1>), grid, block, 0, stream, a);
  else if (hb == 2)
    hipLaunchKernelGGL((decode_split_kernel<D, 2>), grid, block, 0, stream, a);
  else if (hb <= 4)
    hipLaunchKernelGGL((decode_split_kernel<D, 4>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.B * p.h), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
const void* kernel_for_hb(int hb) {
  if (hb == 1) return reinterpret_cast<const void*>(&decode_split_kernel<D, 1>);
  if (hb == 2) return reinterpret_cast<const void*>(&decode_split_kernel<D, 2>);
  if (hb <= 4) return reinterpret_cast<const void*>(&decode_split_kernel<D, 4>);
  return nullptr;
}

const void* decode_kernel_for(int d, int hb) {
  if (d == 64) return kernel_for_hb<64>(hb);
  if (d == 128) return kernel_for_hb<128>(hb);
  return nullptr;
}

}  // namespace

bool decode_supports(int d) { return d == 64 || d == 128; }

int decode_chunk(int B, int h, int g, int T_max, int d) {
  if (const char* env = std::getenv("GQA_DECODE_CHUNK")) {
    const int c = std::atoi(env);
    if (c > 0) return div_up(c, 128) * 128;
  }
  // Few, long key streams: a block streams its chunk with one 32-key
  // sub-block per wave in flight, and per-chunk costs (first-load latency,
  // the block combine, the partial write and the merge) favour long chunks.
  // Split only as far as needed to give every block slot of the chip work.
  int n_cu = 256, per_cu = 2;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) n_cu = v;
    const void* fn = decode_kernel_for(d, div_up(h / g, 16));
    int blocks = 0;
    if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kThreads, 0) == hipSuccess &&
        blocks > 0)
      per_cu = blocks;
  }
  (void)hipGetLastError();
  const long long streams = (long long)B * g;
  const long long want = (long long)per_cu * n_cu;
  const int n_split = streams >= want ? 1 : (int)((want + streams - 1) / streams);
  const int c = div_up(div_up(T_max, n_split), 128) * 128;
  return c > 0 ? c : 128;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
