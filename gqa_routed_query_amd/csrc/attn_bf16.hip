// Grouped-query attention prefill, bf16 inputs, fp32 accumulation, on the
// gfx950 matrix cores. One kernel serves dense GQA and routed GQE.
//
// What is computed (ml-canon "56 GQA / MQA", PyTorch GQA function; IBM Think
// "What is grouped query attention (GQA)?", scaled dot-product attention):
// for every query head i of KV group gamma = i / (h/g), out = softmax(q k^T *
// scale) v over the keys of that group, with the causal mask (key j visible to
// query t iff j <= t) when requested. Routed GQE (gist.science explainer of
// "Grouped Query Experts", section "Architecture et Routage") runs the same
// attention for the (token, head) pairs its router kept, on dense K/V, and
// multiplies each row by its gate.
//
// Design for CDNA4:
//  * A workgroup owns W*32 attention rows of one (batch, KV group): rows are
//    (token, slot) pairs in token-major order, so one K/V tile staged in LDS is
//    shared by every query head of the group (the GQA reuse), and a routed
//    problem is just a shorter row list with a head lookup per row.
//  * Each wave owns 32 rows. Large grids use 12 waves with 32-key tiles: the
//    kernel is latency-bound (LDS fragment reads, MFMA -> softmax -> MFMA
//    dependencies, barriers), and the small tile keeps registers within three
//    waves per SIMD, which hides more of those latencies than larger tiles at
//    two waves per SIMD. Grids too small to give every CU two such workgroups
//    (short routed problems) use 8 waves with 64-key tiles instead, halving the
//    per-tile overhead and spreading the rows over more workgroups.
//    Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 so that each lane ends up owning one query row
//    (column l%32); the probabilities are then already in the B-operand layout
//    of O^T += V^T P^T, and the online-softmax statistics of a row live in two
//    lanes (l and l^32) -- one cross-lane max per tile, sums combined once.
//  * K tiles are read from LDS with 16-byte reads in the A-operand layout; V
//    stays row-major in LDS and is transposed by ds_read_b64_tr_b16.
//  * Double-buffered LDS: the next tile's global loads are in flight while the
//    current tile is multiplied; one barrier per tile.
//  * Causal grids are issued heaviest-first; (batch, group) is the fastest
//    varying part of the block index, so with B*g a multiple of 8 all tiles of
//    one group land on one XCD and share its L2.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

// Two configurations: 12 waves with 32-key tiles (three waves per SIMD) for
// large grids, and 8 waves with 64-key tiles (two waves per SIMD, half the
// per-tile overhead) when a 12-wave grid would leave compute units without
// two workgroups' worth of work (short routed problems).
constexpr int kWavesLarge = 12, kBNLarge = 32;
constexpr int kWavesSmall = 8, kBNSmall = 64;
constexpr float kRescale = 8.0f;                      // lazy-rescale threshold, log2 units

template <int D, int W, int kBN>
struct Tile {
  static constexpr int kThreads = W * 64;
  static constexpr int kPitch = D + 8;    // 16-byte pad: A-operand reads of 16 rows hit distinct banks
  static constexpr int vPitch = D + 32;   // 64-byte pad: transposing reads of 4 rows hit distinct banks
  static constexpr int kElems = kBN * kPitch;
  static constexpr int vElems = kBN * vPitch;
  static constexpr int kCPR = D / 8;      // 16-byte chunks per row
  static constexpr int kChunks = kBN * kCPR;
  static constexpr int kLoads = (kChunks + kThreads - 1) / kThreads;
};

struct KArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  const int32_t* idx;
  const float* gate;
  int h, g, T, R, r;
  int n_row_tiles;
  int BG;
  float c;  // scale * log2(e)
  int causal, out_bf16, zero_unselected;
  int out_slots;  // 1: output row of (token, group, slot) is slot gam*R + slot, not its head; no gate
  // Element strides: q row (b, head, t) at b*q_b + head*q_h + t*D; the K/V rows
  // of (b, gam) start at b*kv_b + gam*kv_g; output row (b, o, t) at
  // b*o_b + o*o_h + t*o_t, o being the head or the slot.
  size_t q_b, q_h, kv_b, kv_g, o_b, o_h, o_t;
  // Problems bg >= BG_main (when q_sh is set): the shared head of batch
  // bg - BG_main, one query row per token (q_sh, out_sh [B, T, D]) on KV head sh_kv.
  int BG_main;
  const uint16_t* q_sh;
  void* out_sh;
  int sh_kv;
};

// Zero the output rows of heads the router did not keep, for the tokens whose
// first row lies in this block's row range.
template <int D, int W>
__device__ void zero_unselected_rows(const KArgs& a, int b, int gam, int row0, int n_rows) {
  constexpr int kThreads = W * 64, kRowsPerBlock = W * 32;
  const int R = a.R, r = a.r;
  const int t_lo = div_up(row0, R);
  const int t_hi = (min(row0 + kRowsPerBlock, n_rows) - 1) / R;
  if (t_hi < t_lo) return;
  constexpr int CPR = D / 8;
  const int n_items = (t_hi - t_lo + 1) * r * CPR;
  for (int c = threadIdx.x; c < n_items; c += kThreads) {
    const int tt = c / (r * CPR);
    const int rem = c - tt * r * CPR;
    const int e = rem / CPR;
    const int ch = rem - e * CPR;
    const int t = t_lo + tt;
    const int head = gam * r + e;
    const int32_t* sel = a.idx + ((size_t)(b * a.T + t) * a.g + gam) * R;
    bool kept = false;
    for (int j = 0; j < R; ++j) kept |= (sel[j] == head);
    if (kept) continue;
    const size_t off = b * a.o_b + head * a.o_h + t * a.o_t + ch * 8;
    const uint4 z = {0u, 0u, 0u, 0u};
    if (a.out_bf16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + off) = z;
    } else {
      uint4* p = reinterpret_cast<uint4*>(static_cast<float*>(a.out) + off);
      p[0] = z;
      p[1] = z;
    }
  }
}

template <int D, int W, int kBN, bool ROUTED>
__global__ __launch_bounds__(W * 64) void attn_bf16_kernel(KArgs a) {
  using L = Tile<D, W, kBN>;
  constexpr int kThreads = W * 64, kRowsPerBlock = W * 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (L::kElems + L::vElems)];
  uint16_t* Ks = smem;
  uint16_t* Vs = smem + 2 * L::kElems;

  const int bid = blockIdx.x;
  const int bg = bid % a.BG;
  const int tile = a.causal ? (a.n_row_tiles - 1 - bid / a.BG) : (bid / a.BG);
  // The shared head's problem (uniform per block; only routed launches carry one).
  const bool shared = ROUTED && bg >= a.BG_main;
  const int b = shared ? bg - a.BG_main : bg / a.g;
  const int gam = shared ? a.sh_kv : bg - b * a.g;
  const int R = shared ? 1 : a.R;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hq = lane >> 5;  // which half of the reduction dim / key quad this lane holds
  const int n_rows = a.T * R;
  const int row0 = tile * kRowsPerBlock;
  if (row0 >= n_rows) return;  // a shared-head problem has T rows, fewer than the routed ones when k > 1

  if (ROUTED && a.zero_unselected && !shared) zero_unselected_rows<D, W>(a, b, gam, row0, n_rows);

  // This lane's attention row.
  const int rho = row0 + wave * 32 + l32;
  const bool row_valid = rho < n_rows;
  const int rho_c = row_valid ? rho : n_rows - 1;
  const int t_row = rho_c / R;
  const int slot = rho_c - t_row * R;
  int head;
  float gate = 1.0f;
  if (shared) {
    head = 0;
  } else if (ROUTED) {
    const size_t o = ((size_t)(b * a.T + t_row) * a.g + gam) * a.R + slot;
    head = a.idx[o];
    gate = a.out_slots ? 1.0f : a.gate[o];
  } else {
    head = gam * a.r + slot;
  }

  // Token range of this wave and of the block (uniform values).
  const int wrow0 = row0 + wave * 32;
  const bool wave_has_rows = wrow0 < n_rows;
  const int wt_lo = min(wrow0, n_rows - 1) / R;
  const int wt_hi = (min(wrow0 + 31, n_rows - 1)) / R;
  const int t_last = (min(row0 + kRowsPerBlock, n_rows) - 1) / R;
  const int n_keys = a.causal ? t_last + 1 : a.T;
  const int n_tiles = div_up(n_keys, kBN);

  // Q^T fragments: B operand of S^T = K Q^T. Lane half hq holds d in
  // [hq*D/2, hq*D/2 + D/2); step st uses 8 of them.
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = (shared ? a.q_sh + (size_t)b * a.T * D : a.q + b * a.q_b + head * a.q_h) +
                           (size_t)t_row * D + hq * (D / 2);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 8 * st);
  }

  const uint16_t* kbase = a.k + b * a.kv_b + gam * a.kv_g;
  const uint16_t* vbase = a.v + b * a.kv_b + gam * a.kv_g;
  uint4 rk[L::kLoads], rv[L::kLoads];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) {
      const int c = tid + i * kThreads;
      const int key = kt * kBN + c / L::kCPR;
      const int col = (c % L::kCPR) * 8;
      if (c < L::kChunks && key < a.T) {
        rk[i] = *reinterpret_cast<const uint4*>(kbase + (size_t)key * D + col);
        rv[i] = *reinterpret_cast<const uint4*>(vbase + (size_t)key * D + col);
      } else {
        rk[i] = make_uint4(0u, 0u, 0u, 0u);  // keys past T: finite zeros, masked below
        rv[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c >= L::kChunks) continue;
      const int row = c / L::kCPR;
      const int col = (c % L::kCPR) * 8;
      *reinterpret_cast<uint4*>(Ks + buf * L::kElems + row * L::kPitch + col) = rk[i];
      *reinterpret_cast<uint4*>(Vs + buf * L::vElems + row * L::vPitch + col) = rv[i];
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  // m_ref: the row's reference max (scaled, log2 units) that probabilities are
  // taken against; identical in lanes l and l^32. It is raised only when a new
  // score exceeds it by more than kRescale, so most tiles skip the rescale of
  // the accumulators; probabilities stay below 2^kRescale and the final
  // division by the row sum is exact whatever reference was used.
  float m_ref = -INFINITY;
  float l_run = 0.0f;

  // Lane roles for the transposing V reads.
  const int grp = lane >> 4;
  const int i16 = lane & 15;
  const int tr_row = 4 * hq + (i16 >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (i16 & 3);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) load_tile(kt + 1);
    const int key0 = kt * kBN;
    const bool active = wave_has_rows && (!a.causal || key0 <= wt_hi);
    if (active) {
      // S^T[key][row] for the 64 keys of this tile, two 32-key blocks. The 8
      // A-operand fragments of a block are read from LDS before its MFMAs.
      f32x16 s[kBN / 32];
      const uint16_t* kl = Ks + buf * L::kElems;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        const uint16_t* krow = kl + (kb * 32 + l32) * L::kPitch + hq * (D / 2);
        bf16x8 kfr[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) kfr[st] = *reinterpret_cast<const bf16x8*>(krow + 8 * st);
        s[kb] = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) s[kb] = mfma32x32x16(kfr[st], qf[st], s[kb]);
      }
      // Keep several fragment reads in flight ahead of the MFMAs that use them
      // (LDS latency is several MFMA issue slots).
      constexpr int kAhead = 6, kFrags = (kBN / 32) * (D / 16);
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int i = 0; i < kFrags - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
      // Mask keys past the row's limit: (kb, i) holds key key0 + 32kb + 8(i/4) + 4hq + i%4.
      const bool need_mask = (a.causal && key0 + kBN - 1 > wt_lo) || (key0 + kBN > a.T);
      if (need_mask) {
        const int lim = a.causal ? t_row : a.T - 1;
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * hq + (i & 3);
            if (key > lim) s[kb][i] = -INFINITY;
          }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mloc = fmaxf(fmaxf(mloc, s[kb][i]), s[kb][i + 1]);
      const float mloc_s = mloc * a.c;
      if (__any(mloc_s > m_ref + kRescale)) {
        const float m_new = fmaxf(m_ref, fmaxf(mloc_s, __shfl_xor(mloc_s, 32)));
        const float alpha = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      }

      // P^T as bf16 B operands: step u covers keys 16u .. 16u+15 of the tile.
      // The row sum adds the rounded bf16 values, the ones the MFMA uses.
      bf16x8 pf[kBN / 16];
#pragma unroll
      for (int u = 0; u < kBN / 16; ++u) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(fmaf(s[u >> 1][8 * (u & 1) + j], a.c, -m_ref));
        pf[u] = pack_bf16x8(pv);
        const bf16x2* pp = reinterpret_cast<const bf16x2*>(&pf[u]);
#pragma unroll
        for (int j = 0; j < 4; ++j) l_run = __builtin_amdgcn_fdot2_f32_bf16(pp[j], ones, l_run, false);
      }

      // O^T += V^T P^T. Element j of step u is key 16u + 8(j/4) + 4hq + j%4,
      // which the two transposing reads fetch for d = 32db + l%32.
      const uint16_t* vl = Vs + buf * L::vElems;
#pragma unroll
      for (int u = 0; u < kBN / 16; ++u) {
        const uint16_t* p0 = vl + (16 * u + tr_row) * L::vPitch + tr_col;
        bf16x8 vfr[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          vfr[db] = lds_read_tr_pair(p0 + 32 * db, p0 + 8 * L::vPitch + 32 * db);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = mfma32x32x16(vfr[db], pf[u], o[db]);
      }
    }
    if (kt + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_valid) {
    const float inv = gate / l_tot;
    const int oslot = a.out_slots ? gam * a.R + slot : head;
    void* const outp = shared ? a.out_sh : a.out;
    const size_t obase = shared ? ((size_t)b * a.T + t_row) * D + 4 * hq
                                : b * a.o_b + oslot * a.o_h + t_row * a.o_t + 4 * hq;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const size_t off = obase + 32 * db + 8 * i4;
        const float x0 = o[db][4 * i4 + 0] * inv, x1 = o[db][4 * i4 + 1] * inv;
        const float x2 = o[db][4 * i4 + 2] * inv, x3 = o[db][4 * i4 + 3] * inv;
        if (a.out_bf16) {
          uint2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(outp) + off) = w;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(outp) + off) = make_float4(x0, x1, x2, x3);
        }
      }
  }
}

template <int D, int W, int BN>
hipError_t launch_dw(KArgs a, const AttnParams& p, hipStream_t stream) {
  a.n_row_tiles = div_up(p.T * p.R, W * 32);
  const dim3 grid(a.n_row_tiles * a.BG), block(W * 64);
  if (p.idx)
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  KArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = p.out;
  a.idx = p.idx;
  a.gate = p.gate;
  a.h = p.h;
  a.g = p.g;
  a.T = p.T;
  a.R = p.R;
  a.r = p.h / p.g;
  a.BG_main = p.B * p.g;
  a.q_sh = static_cast<const uint16_t*>(p.q_shared);
  a.out_sh = p.out_shared;
  a.sh_kv = p.shared_kv;
  if (p.q_shared && !p.idx) return hipErrorInvalidValue;  // a shared head rides on a routed launch
  a.BG = a.BG_main + (p.q_shared ? p.B : 0);
  a.c = p.scale * kLog2e;
  a.causal = p.causal;
  a.out_bf16 = p.out_bf16;
  a.zero_unselected = p.zero_unselected;
  a.out_slots = p.out_slots;
  const size_t TD = (size_t)p.T * D;
  a.q_b = p.q_b ? p.q_b : (size_t)p.h * TD;
  a.q_h = TD;
  a.kv_b = p.kv_b ? p.kv_b : (size_t)p.g * TD;
  a.kv_g = TD;
  a.o_b = p.o_b ? p.o_b : (size_t)p.h * TD;
  a.o_h = p.o_h ? p.o_h : TD;
  a.o_t = p.o_t ? p.o_t : D;
  int n_cu = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  const long long large_grid = (long long)a.BG * div_up(p.T * p.R, kWavesLarge * 32);
  if (large_grid >= 2ll * n_cu) return launch_dw<D, kWavesLarge, kBNLarge>(a, p, stream);
  return launch_dw<D, kWavesSmall, kBNSmall>(a, p, stream);
}

}  // namespace

bool attn_bf16_supports(int d) { return d == 64 || d == 128; }

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
