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
//  * K/V tiles reach LDS by DMA (global_load_lds_dwordx4, no registers), double
//    buffered: the next tile is in flight while the current one is multiplied;
//    one barrier per tile.
//  * Q comes in and the output goes out through a per-wave LDS region, so
//    both move whole rows per instruction; read straight from HBM in the
//    fragment layouts, each instruction would touch 16 bytes of 32 rows.
//  * (batch, group) is the fastest varying part of the block index, so with B*g
//    a multiple of 8 all tiles of one group land on one XCD and share its L2.
//    The row tiles of a causal grid differ in cost (the number of visible key
//    tiles), and their dispatch order is planned on the host (plan_order).
#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <type_traits>
#include <vector>

#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

// Two configurations: 12 waves with 32-key tiles (three waves per SIMD) for
// large grids, and 8 waves with 64-key tiles (two waves per SIMD, half the
// per-tile overhead) when a 12-wave grid would leave compute units without
// two workgroups' worth of work (short routed problems).
constexpr int kWavesLarge = 12, kBNLarge = 32, kOccLarge = 3;
constexpr int kWavesSmall = 8, kBNSmall = 64, kOccSmall = 2;
constexpr float kRescale = 8.0f;                      // lazy-rescale threshold, log2 units
constexpr int kMaxOrder = 48;                         // row-tile bands with a planned dispatch order

template <int D, int W, int kBN>
struct Tile {
  static constexpr int kThreads = W * 64;
  static constexpr int kPitch = D + 8;    // 16-byte pad: A-operand reads of 16 rows hit distinct banks
  static constexpr int vPitch = D + 32;   // 64-byte pad: transposing reads of 4 rows hit distinct banks
  static constexpr int kCPR = D / 8;      // 16-byte granules of data per row
  // Staging by DMA: one global_load_lds_dwordx4 fills 64 consecutive 16-byte
  // LDS granules, so a padded tile is filled granule by granule, pad granules
  // included (they receive a copy of an in-row granule and are never read).
  static constexpr int kGPR = kPitch / 8;  // granules per K row, pad included
  static constexpr int vGPR = vPitch / 8;  // granules per V row, pad included
  static constexpr int kDmaK = (kBN * kGPR + 63) / 64;
  static constexpr int kDmaV = (kBN * vGPR + 63) / 64;
  static constexpr int kDma = kDmaK + kDmaV;
  static constexpr int kMine = (kDma + W - 1) / W;  // DMA instructions per wave, at most
  static constexpr int kElems = kDmaK * 512;        // bf16 elements per K buffer
  static constexpr int vElems = kDmaV * 512;
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
  // Causal grids: block band i (blocks i*BG .. i*BG + BG-1, one per problem)
  // runs row tile order[i] when n_order > 0, else row tile n_row_tiles-1-i.
  int n_order;
  uint16_t order[kMaxOrder];
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

template <int D, int W, int kBN, int OCC, bool ROUTED>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(OCC))) void attn_bf16_kernel(KArgs a) {
  using L = Tile<D, W, kBN>;
  constexpr int kThreads = W * 64, kRowsPerBlock = W * 32;
  // One array per buffer: with the buffer fixed at compile time, the compiler
  // can tell that reads of one buffer do not alias the DMA into the other and
  // adds no wait for the DMA before them.
  __shared__ __attribute__((aligned(16))) uint16_t K0[L::kElems], K1[L::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t V0[L::vElems], V1[L::vElems];
  // Per-wave staging of the wave's 32 rows (padded pitch kPitch): Q on the way
  // in, the output on the way out, so that both move whole rows per
  // instruction instead of 16 bytes of 32 different rows.
  constexpr int kQDma = (32 * L::kGPR + 63) / 64;
  constexpr int kQElems = kQDma * 512;
  __shared__ __attribute__((aligned(16))) uint16_t QO[W * kQElems];
  // Per-wave table of the wave's 32 rows: token, head, slot, gate.
  __shared__ int4 rowtab[W * 32];

  const int bid = blockIdx.x;
  const int bg = bid % a.BG;
  const int band = bid / a.BG;
  const int tile = !a.causal ? band : a.n_order ? (int)a.order[band] : a.n_row_tiles - 1 - band;
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

  // Attention row rho (< n_rows): token, slot, head (a routed row's head is
  // the router's pick) and gate.
  struct RowInfo {
    int t, slot, head;
    float gate;
  };
  auto row_info = [&](int rho) {
    RowInfo ri;
    ri.t = rho / R;
    ri.slot = rho - ri.t * R;
    ri.gate = 1.0f;
    if (shared) {
      ri.head = 0;
    } else if (ROUTED) {
      const size_t o = ((size_t)(b * a.T + ri.t) * a.g + gam) * a.R + ri.slot;
      ri.head = a.idx[o];
      ri.gate = a.out_slots ? 1.0f : a.gate[o];
    } else {
      ri.head = gam * a.r + ri.slot;
    }
    return ri;
  };

  // This lane's attention row (the last row stands in for rows past the end).
  const int rho = row0 + wave * 32 + l32;
  const int t_row = min(rho, n_rows - 1) / R;

  // Token range of this wave and of the block (uniform values).
  const int wrow0 = row0 + wave * 32;
  const bool wave_has_rows = wrow0 < n_rows;
  const int wt_lo = min(wrow0, n_rows - 1) / R;
  const int wt_hi = (min(wrow0 + 31, n_rows - 1)) / R;
  const int t_last = (min(row0 + kRowsPerBlock, n_rows) - 1) / R;
  const int n_keys = a.causal ? t_last + 1 : a.T;
  const int n_tiles = div_up(n_keys, kBN);

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint16_t* const QOw = QO + wave_u * kQElems;
  int4* const tab = rowtab + wave_u * 32;
  // Each lane resolves its own row once (rows past the end stand in as the
  // last row); lanes that move other rows read them from the table.
  if (hq == 0) {
    const RowInfo ri = row_info(min(rho, n_rows - 1));
    tab[l32] = make_int4(ri.t, ri.head, ri.slot, __float_as_int(ri.gate));
  }
  __syncthreads();
  // The wave's 32 Q rows into QOw by DMA, granule by granule as for K (pad
  // granules receive a copy of granule 0).
#pragma unroll
  for (int j = 0; j < kQDma; ++j) {
    const int p = j * 64 + lane;
    int row = p / L::kGPR, gr = p - row * L::kGPR;
    if (row > 31) row = 31;
    if (gr >= L::kCPR) gr = 0;
    const int4 ri = tab[row];
    const uint16_t* src = (shared ? a.q_sh + (size_t)b * a.T * D : a.q + b * a.q_b + (size_t)ri.y * a.q_h) +
                          (size_t)ri.x * D + gr * 8;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(QOw + j * 512), 16, 0, 0);
  }

  const uint16_t* kbase = a.k + b * a.kv_b + gam * a.kv_g;
  const uint16_t* vbase = a.v + b * a.kv_b + gam * a.kv_g;
  // Byte offsets (from the tile's first key row) that this lane loads for the
  // wave's DMA instructions j = wave + W*i: K granules first, then V.
  uint32_t dma_off[L::kMine];
#pragma unroll
  for (int i = 0; i < L::kMine; ++i) {
    const int j = wave_u + W * i;
    const bool isk = j < L::kDmaK;
    const int gpr = isk ? L::kGPR : L::vGPR;
    const int p = (isk ? j : j - L::kDmaK) * 64 + lane;
    int row = p / gpr, gr = p - row * gpr;
    if (row >= kBN) row = kBN - 1;  // rounding slack after the last row
    if (gr >= L::kCPR) gr = 0;      // pad granule
    dma_off[i] = (uint32_t)(row * D + gr * 8) * 2u;
  }
  // Start the DMA of key tile kt into buffer buf. Keys past T (last tile only)
  // are clamped to key T-1: finite values that the mask discards.
  auto issue_tile = [&](int kt, auto buf) {
    uint16_t* const Kb = buf.value ? K1 : K0;
    uint16_t* const Vb = buf.value ? V1 : V0;
    const int key0 = kt * kBN;
    const bool full = key0 + kBN <= a.T;
#pragma unroll
    for (int i = 0; i < L::kMine; ++i) {
      const int j = wave_u + W * i;
      if (j >= L::kDma) break;
      const bool isk = j < L::kDmaK;
      uint32_t off = dma_off[i];
      if (!full) {
        const int last = a.T - 1 - key0;  // >= 0: a tile is issued only if key0 < T
        if ((int)(off / (2 * D)) > last) off = (uint32_t)last * (2 * D) + (off & (2 * D - 1));
      }
      const char* base = reinterpret_cast<const char*>((isk ? kbase : vbase) + (size_t)key0 * D);
      const uint16_t* src = reinterpret_cast<const uint16_t*>(base + off);
      uint16_t* dst = isk ? Kb + j * 512 : Vb + (j - L::kDmaK) * 512;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
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

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  issue_tile(0, B0{});
  __syncthreads();

  // Q^T fragments: B operand of S^T = K Q^T. Lane half hq holds d in
  // [hq*D/2, hq*D/2 + D/2); step st uses 8 of them.
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = QOw + l32 * L::kPitch + hq * (D / 2);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 8 * st);
  }

  // Tile kt, held in buffer buf (kt % 2); the DMA of tile kt+1 goes to the other.
  auto tile_step = [&](int kt, auto buf) {
    const uint16_t* const Kb = buf.value ? K1 : K0;
    const uint16_t* const Vb = buf.value ? V1 : V0;
    if (kt + 1 < n_tiles) issue_tile(kt + 1, std::integral_constant<int, 1 - buf.value>{});
    const int key0 = kt * kBN;
    const bool active = wave_has_rows && (!a.causal || key0 <= wt_hi);
    if (active) {
      // S^T[key][row] for the 64 keys of this tile, two 32-key blocks. The 8
      // A-operand fragments of a block are read from LDS before its MFMAs.
      f32x16 s[kBN / 32];
      const uint16_t* kl = Kb;
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
      const uint16_t* vl = Vb;
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
    __syncthreads();
  };
  for (int kt = 0; kt < n_tiles; kt += 2) {
    tile_step(kt, B0{});
    if (kt + 1 < n_tiles) tile_step(kt + 1, B1{});
  }

  // Output: each pass stages D*2 bytes of each of the wave's 32 rows in QOw
  // (all of a bf16 row, half of an fp32 row), then stores them row by row, 16
  // bytes per lane.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = __int_as_float(tab[l32].w) / l_tot;
  constexpr int kRowB = L::kPitch * 2;      // staged row pitch, bytes
  constexpr int kG = D * 2 / 16;            // 16-byte granules per staged row
  constexpr int kRowsPer = 64 / kG;         // rows per store instruction
  char* const stage = reinterpret_cast<char*>(QOw);
  const int n_pass = a.out_bf16 ? 1 : 2;
  for (int pass = 0; pass < n_pass; ++pass) {
    // o[db][4*i4 + j] holds d = 32db + 8i4 + 4hq + j of this lane's row.
    if (a.out_bf16) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * db + 8 * i4 + 4 * hq;
          uint2 w = {pack_bf16x2(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv),
                     pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv)};
          *reinterpret_cast<uint2*>(stage + l32 * kRowB + d0 * 2) = w;
        }
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        if (db / (D / 64) != pass) continue;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * db + 8 * i4 + 4 * hq - pass * (D / 2);
          *reinterpret_cast<float4*>(stage + l32 * kRowB + d0 * 4) =
              make_float4(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv, o[db][4 * i4 + 2] * inv,
                          o[db][4 * i4 + 3] * inv);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32 / kRowsPer; ++i) {
      const int row = i * kRowsPer + lane / kG;
      const int gran = lane % kG;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * kRowB + gran * 16);
      const int rr = wrow0 + row;
      if (rr < n_rows) {
        const int4 ri = tab[row];
        const int oslot = a.out_slots ? gam * a.R + ri.z : ri.y;
        const size_t orow = shared ? ((size_t)b * a.T + ri.x) * D : b * a.o_b + oslot * a.o_h + ri.x * a.o_t;
        char* const outp = static_cast<char*>(shared ? a.out_sh : a.out);
        const size_t ob = orow * (a.out_bf16 ? 2 : 4) + (size_t)pass * D * 2 + gran * 16;
        *reinterpret_cast<u32x4*>(outp + ob) = v;
      }
    }
    if (pass + 1 < n_pass) __syncthreads();
  }
}

// Dispatch order of the row-tile bands of a causal grid. The hardware hands
// blocks to CUs in index order as CUs free up; a band is one row tile of every
// problem. Heaviest first leaves the last round short of work: at B=4, h=32,
// g=8, T=2048 two rounds end together and 192 light jobs remain for 256 CUs.
// The order is searched on a model of that dispatch: a job costs its key tiles
// plus a fixed cost, goes to the CU that frees first, and pairwise swaps of
// bands are kept while they shorten the simulated end. The per-job fixed cost
// (prologue and epilogue) was fitted by measurement: about 4 tiles of 32 keys.
// Cached per shape; shapes with more bands keep heaviest first.
struct OrderShape {
  int n_bands, rows, R, T, kBN, BG_main, B_sh, n_cu;
  bool operator<(const OrderShape& o) const {
    return std::tie(n_bands, rows, R, T, kBN, BG_main, B_sh, n_cu) <
           std::tie(o.n_bands, o.rows, o.R, o.T, o.kBN, o.BG_main, o.B_sh, o.n_cu);
  }
};

double simulate_dispatch(const std::vector<int>& order, const std::vector<double>& cost_main,
                         const std::vector<double>& cost_sh, int per_main, int per_sh, int n_cu) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < n_cu; ++i) free_at.push(0.0);
  double end = 0.0;
  for (int band : order)
    for (int j = 0; j < per_main + per_sh; ++j) {
      const double t = free_at.top() + (j < per_main ? cost_main[band] : cost_sh[band]);
      free_at.pop();
      free_at.push(t);
      end = std::max(end, t);
    }
  return end;
}

std::vector<uint16_t> plan_order(const OrderShape& s) {
  // Key tiles of row tile i of a problem with n_rows = T*R rows, R per token.
  auto cost = [&](int i, int R, double fixed) {
    const int n_rows = s.T * R, row0 = i * s.rows;
    if (row0 >= n_rows) return 0.0;
    const int t_last = (std::min(row0 + s.rows, n_rows) - 1) / R;
    return (double)div_up(t_last + 1, s.kBN) + fixed;
  };
  const double fixed = 128.0 / s.kBN;  // ≈ 4 tiles of 32 keys
  std::vector<double> cost_main(s.n_bands), cost_sh(s.n_bands);
  for (int i = 0; i < s.n_bands; ++i) {
    cost_main[i] = cost(i, s.R, fixed);
    cost_sh[i] = cost(i, 1, fixed);
  }
  // With whole problems per XCD slice (blocks go to XCDs round-robin), one
  // eighth of the CUs and of each band is an exact model.
  int per_main = s.BG_main, per_sh = s.B_sh, n_cu = s.n_cu;
  if (per_main % 8 == 0 && per_sh % 8 == 0 && n_cu % 8 == 0) {
    per_main /= 8;
    per_sh /= 8;
    n_cu /= 8;
  }
  std::vector<int> order(s.n_bands);
  for (int i = 0; i < s.n_bands; ++i) order[i] = s.n_bands - 1 - i;  // heaviest first
  double best = simulate_dispatch(order, cost_main, cost_sh, per_main, per_sh, n_cu);
  for (int pass = 0; pass < 4; ++pass) {
    bool improved = false;
    for (int i = 0; i < s.n_bands; ++i)
      for (int j = i + 1; j < s.n_bands; ++j) {
        std::swap(order[i], order[j]);
        const double m = simulate_dispatch(order, cost_main, cost_sh, per_main, per_sh, n_cu);
        if (m < best - 1e-9) {
          best = m;
          improved = true;
        } else {
          std::swap(order[i], order[j]);
        }
      }
    if (!improved) break;
  }
  return std::vector<uint16_t>(order.begin(), order.end());
}

void set_order(KArgs& a, const OrderShape& s) {
  a.n_order = 0;
  if (!a.causal || s.n_bands < 2 || s.n_bands > kMaxOrder) return;
  static std::mutex mu;
  static std::map<OrderShape, std::vector<uint16_t>> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(s);
  if (it == cache.end()) it = cache.emplace(s, plan_order(s)).first;
  std::copy(it->second.begin(), it->second.end(), a.order);
  a.n_order = s.n_bands;
}

template <int D, int W, int BN, int OCC>
hipError_t launch_dw(KArgs a, const AttnParams& p, hipStream_t stream, int n_cu) {
  a.n_row_tiles = div_up(p.T * p.R, W * 32);
  set_order(a, OrderShape{a.n_row_tiles, W * 32, p.R, p.T, BN, a.BG_main, a.BG - a.BG_main, n_cu});
  const dim3 grid(a.n_row_tiles * a.BG), block(W * 64);
  if (p.idx)
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, OCC, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, OCC, false>), grid, block, 0, stream, a);
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
  if (large_grid * kWavesLarge >= 24ll * n_cu)
    return launch_dw<D, kWavesLarge, kBNLarge, kOccLarge>(a, p, stream, n_cu);
  return launch_dw<D, kWavesSmall, kBNSmall, kOccSmall>(a, p, stream, n_cu);
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
