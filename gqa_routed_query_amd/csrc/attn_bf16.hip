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
//    per-tile overhead and spreading the rows over more workgroups, unless key
//    splitting (below) makes a grid of at most one 12-wave block per CU run as
//    one round.
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
  // Key-split slots (routed launches given a workspace): slot i covers key
  // tiles [0, split[i]) of its row tile when part[i] == 1 and [split[i],
  // n_tiles) when part[i] == 2, and writes its partial result to workspace
  // slot (sbi[i] * BG + bg) * 2 + part[i] - 1; part[i] == 0 covers them all.
  uint8_t part[kMaxOrder];
  uint8_t sbi[kMaxOrder];
  uint16_t split[kMaxOrder];
  float* ws;
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
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (a.out_bf16) {
      __builtin_nontemporal_store(z, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + off));
    } else {
      u32x4* p = reinterpret_cast<u32x4*>(static_cast<float*>(a.out) + off);
      __builtin_nontemporal_store(z, p);
      __builtin_nontemporal_store(z, p + 1);
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
  const int part = a.n_order ? (int)a.part[band] : 0;
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

  if (ROUTED && a.zero_unselected && !shared && part <= 1) zero_unselected_rows<D, W>(a, b, gam, row0, n_rows);

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
  const int kt_lo = part == 2 ? (int)a.split[band] : 0;
  const int kt_hi = part == 1 ? (int)a.split[band] : n_tiles;

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
  issue_tile(kt_lo, B0{});
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
    if (kt + 1 < kt_hi) issue_tile(kt + 1, std::integral_constant<int, 1 - buf.value>{});
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
  for (int kt = kt_lo; kt < kt_hi; kt += 2) {
    tile_step(kt, B0{});
    if (kt + 1 < kt_hi) tile_step(kt + 1, B1{});
  }

  // Output: each pass stages D*2 bytes of each of the wave's 32 rows in QOw
  // (all of a bf16 row, half of an fp32 row), then stores them row by row, 16
  // bytes per lane. A key-split part stores instead its partial result in its
  // workspace slot: the unnormalised O rows in fp32, then per row the
  // reference max m_ref and the sum l (rows past the end included).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool partial = part != 0;
  float* const pws =
      partial ? a.ws + ((size_t)(a.sbi[band] * a.BG + bg) * 2 + part - 1) * ((size_t)kRowsPerBlock * (D + 2))
              : nullptr;
  if (partial && hq == 0) {
    pws[kRowsPerBlock * D + wave * 32 + l32] = m_ref;
    pws[kRowsPerBlock * (D + 1) + wave * 32 + l32] = l_tot;
  }
  const float inv = partial ? 1.0f : __int_as_float(tab[l32].w) / l_tot;
  constexpr int kRowB = L::kPitch * 2;      // staged row pitch, bytes
  constexpr int kG = D * 2 / 16;            // 16-byte granules per staged row
  constexpr int kRowsPer = 64 / kG;         // rows per store instruction
  char* const stage = reinterpret_cast<char*>(QOw);
  const bool bf16_out = a.out_bf16 && !partial;
  const int n_pass = bf16_out ? 1 : 2;
  for (int pass = 0; pass < n_pass; ++pass) {
    // o[db][4*i4 + j] holds d = 32db + 8i4 + 4hq + j of this lane's row.
    if (bf16_out) {
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
      if (partial) {
        *reinterpret_cast<u32x4*>(pws + (size_t)(wave * 32 + row) * D + pass * (D / 2) + gran * 4) = v;
      } else if (rr < n_rows) {
        const int4 ri = tab[row];
        const int oslot = a.out_slots ? gam * a.R + ri.z : ri.y;
        const size_t orow = shared ? ((size_t)b * a.T + ri.x) * D : b * a.o_b + oslot * a.o_h + ri.x * a.o_t;
        char* const outp = static_cast<char*>(shared ? a.out_sh : a.out);
        const size_t ob = orow * (a.out_bf16 ? 2 : 4) + (size_t)pass * D * 2 + gran * 16;
        // Nontemporal: the output is not read again here, and streaming it
        // past L2 leaves the K/V tiles that other row tiles reuse in place.
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outp + ob));
      }
    }
    if (pass + 1 < n_pass) __syncthreads();
  }
}

// Merges the two parts of every key-split row tile. Per row the partial
// results (m_p, l_p, O_p) over the two key ranges, each taken against its own
// reference max, combine as the online softmax does within a part:
//   m = max(m_1, m_2),  w_p = 2^(m_p - m),
//   O = (w_1 O_1 + w_2 O_2) / (w_1 l_1 + w_2 l_2),
// then the row's gate and the attention kernel's output layout.
template <int D, int W, bool ROUTED>
__global__ __launch_bounds__(256) void split_merge_kernel(KArgs a) {
  constexpr int kRowsPerBlock = W * 32, kRowsPerSub = 256 / (D / 8), kSubs = kRowsPerBlock / kRowsPerSub;
  static_assert(kRowsPerBlock % kRowsPerSub == 0, "merge sub-blocks must tile the row tile");
  const int sub = blockIdx.x % kSubs, sbg = blockIdx.x / kSubs;
  const int sb = sbg / a.BG, bg = sbg % a.BG;
  int tile = 0;
  for (int i = 0; i < a.n_order; ++i)
    if (a.part[i] == 1 && a.sbi[i] == sb) tile = a.order[i];
  const int b = bg / a.g, gam = bg - b * a.g;  // split launches carry no shared head
  const int R = a.R, n_rows = a.T * R, row0 = tile * kRowsPerBlock;
  const float* const p1 = a.ws + (size_t)(sb * a.BG + bg) * 2 * ((size_t)kRowsPerBlock * (D + 2));
  const float* const p2 = p1 + (size_t)kRowsPerBlock * (D + 2);
  {
    const int row = sub * kRowsPerSub + threadIdx.x / (D / 8), ch = threadIdx.x % (D / 8);
    const int rho = row0 + row;
    if (rho >= n_rows) return;
    const float m1 = p1[kRowsPerBlock * D + row], l1 = p1[kRowsPerBlock * (D + 1) + row];
    const float m2 = p2[kRowsPerBlock * D + row], l2 = p2[kRowsPerBlock * (D + 1) + row];
    const float m = fmaxf(m1, m2);
    const float w1 = fast_exp2(m1 - m), w2 = fast_exp2(m2 - m);
    const int t = rho / R, slot = rho - t * R;
    int head;
    float gate = 1.0f;
    if (ROUTED) {
      const size_t o = ((size_t)(b * a.T + t) * a.g + gam) * a.R + slot;
      head = a.idx[o];
      gate = a.out_slots ? 1.0f : a.gate[o];
    } else {
      head = gam * a.r + slot;
    }
    const float sc = gate / (w1 * l1 + w2 * l2);
    const float4* x1 = reinterpret_cast<const float4*>(p1 + (size_t)row * D + ch * 8);
    const float4* x2 = reinterpret_cast<const float4*>(p2 + (size_t)row * D + ch * 8);
    const float4 a0 = x1[0], a1 = x1[1], b0 = x2[0], b1 = x2[1];
    const float v[8] = {(w1 * a0.x + w2 * b0.x) * sc, (w1 * a0.y + w2 * b0.y) * sc,
                        (w1 * a0.z + w2 * b0.z) * sc, (w1 * a0.w + w2 * b0.w) * sc,
                        (w1 * a1.x + w2 * b1.x) * sc, (w1 * a1.y + w2 * b1.y) * sc,
                        (w1 * a1.z + w2 * b1.z) * sc, (w1 * a1.w + w2 * b1.w) * sc};
    const int oslot = a.out_slots ? gam * a.R + slot : head;
    const size_t off = b * a.o_b + oslot * a.o_h + t * a.o_t + ch * 8;
    if (a.out_bf16) {
      const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7])};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + off));
    } else {
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<float*>(a.out) + off);
      __builtin_nontemporal_store(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                        __float_as_uint(v[3])}, dst);
      __builtin_nontemporal_store(u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                        __float_as_uint(v[7])}, dst + 1);
    }
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
//
// Key splitting (routed launches given a workspace): when the grid holds less
// than two blocks per CU, the heaviest row tiles of the upper half of the
// sequence are split at a key tile into two parts that run as separate jobs,
// and a second kernel merges their partial results. The split key tile is
// never past the tile's first token, so every row sees keys in both parts.
// A split is kept when it shortens the modelled end.
struct OrderShape {
  int n_bands, rows, R, T, kBN, BG_main, B_sh, n_cu, max_split;
  bool operator<(const OrderShape& o) const {
    return std::tie(n_bands, rows, R, T, kBN, BG_main, B_sh, n_cu, max_split) <
           std::tie(o.n_bands, o.rows, o.R, o.T, o.kBN, o.BG_main, o.B_sh, o.n_cu, o.max_split);
  }
};

struct Slot {
  uint16_t tile, split;
  uint8_t part, sbi;
};

// Key tiles of row tile i of a problem with T*R rows (R per token), and the
// key tile at which it may be split.
struct BandKeys {
  int n_tiles, split;
};
BandKeys band_keys(int i, int rows, int R, int T, int kBN) {
  const int n_rows = T * R, row0 = i * rows;
  if (row0 >= n_rows) return {0, 0};
  const int t_first = row0 / R, t_last = (std::min(row0 + rows, n_rows) - 1) / R;
  const int n_tiles = div_up(t_last + 1, kBN);
  return {n_tiles, std::min(n_tiles / 2, t_first / kBN)};
}

// Row tiles that may be split in one launch (0 when the grid has two or more
// blocks per CU): those of the upper half with a split point inside.
int split_cap(int n_bands, int rows, int R, int T, int kBN, int BG, int n_cu) {
  if ((long long)n_bands * BG >= 2ll * n_cu || n_bands >= kMaxOrder) return 0;
  int eligible = 0;
  for (int i = n_bands / 2; i < n_bands; ++i) {
    const BandKeys k = band_keys(i, rows, R, T, kBN);
    if (k.split >= 1 && k.n_tiles - k.split >= 1) ++eligible;
  }
  return std::min(eligible, kMaxOrder - n_bands);
}

double simulate_dispatch(const std::vector<int>& order, const std::vector<double>& cost_main,
                         const std::vector<double>& cost_sh, int per_main, int per_sh, int n_cu) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < n_cu; ++i) free_at.push(0.0);
  double end = 0.0;
  for (int slot : order)
    for (int j = 0; j < per_main + per_sh; ++j) {
      const double t = free_at.top() + (j < per_main ? cost_main[slot] : cost_sh[slot]);
      free_at.pop();
      free_at.push(t);
      end = std::max(end, t);
    }
  return end;
}

std::vector<Slot> plan_order(const OrderShape& s) {
  const double fixed = 128.0 / s.kBN;  // ≈ 4 tiles of 32 keys
  std::vector<Slot> slots;
  for (int i = 0; i < s.n_bands; ++i) slots.push_back(Slot{(uint16_t)i, 0, 0, 0});
  auto slot_cost = [&](const Slot& sl, int R) {
    const BandKeys k = band_keys(sl.tile, s.rows, R, s.T, s.kBN);
    if (k.n_tiles == 0) return 0.0;
    const int n = sl.part == 0 ? k.n_tiles : sl.part == 1 ? sl.split : k.n_tiles - sl.split;
    return (double)n + fixed;
  };
  // With whole problems per XCD slice (blocks go to XCDs round-robin), one
  // eighth of the CUs and of each band is an exact model.
  int per_main = s.BG_main, per_sh = s.B_sh, n_cu = s.n_cu;
  if (per_main % 8 == 0 && per_sh % 8 == 0 && n_cu % 8 == 0) {
    per_main /= 8;
    per_sh /= 8;
    n_cu /= 8;
  }
  std::vector<double> cost_main, cost_sh;
  auto costs = [&]() {
    cost_main.assign(slots.size(), 0.0);
    cost_sh.assign(slots.size(), 0.0);
    for (size_t i = 0; i < slots.size(); ++i) {
      cost_main[i] = slot_cost(slots[i], s.R);
      cost_sh[i] = slot_cost(slots[i], 1);
    }
  };
  auto heaviest_first = [&]() {
    std::vector<int> order(slots.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return cost_main[x] > cost_main[y]; });
    return order;
  };
  // Splits, heaviest row tile first, kept while the end shortens.
  if (s.max_split > 0 && s.B_sh == 0) {
    std::vector<int> cand;
    for (int i = s.n_bands / 2; i < s.n_bands; ++i) {
      const BandKeys k = band_keys(i, s.rows, s.R, s.T, s.kBN);
      if (k.split >= 1 && k.n_tiles - k.split >= 1) cand.push_back(i);
    }
    std::stable_sort(cand.begin(), cand.end(), [&](int x, int y) {
      return band_keys(x, s.rows, s.R, s.T, s.kBN).n_tiles > band_keys(y, s.rows, s.R, s.T, s.kBN).n_tiles;
    });
    costs();
    double best = simulate_dispatch(heaviest_first(), cost_main, cost_sh, per_main, per_sh, n_cu);
    int n_split = 0;
    for (int i : cand) {
      if (n_split == s.max_split) break;
      const uint16_t sp = (uint16_t)band_keys(i, s.rows, s.R, s.T, s.kBN).split;
      std::vector<Slot> keep = slots;
      for (auto& sl : slots)
        if (sl.tile == i) sl = Slot{(uint16_t)i, sp, 1, (uint8_t)n_split};
      slots.push_back(Slot{(uint16_t)i, sp, 2, (uint8_t)n_split});
      costs();
      const double m = simulate_dispatch(heaviest_first(), cost_main, cost_sh, per_main, per_sh, n_cu);
      if (m < best - 1e-9) {
        best = m;
        ++n_split;
      } else {
        slots = keep;
      }
    }
  }
  costs();
  std::vector<int> order = heaviest_first();
  double best = simulate_dispatch(order, cost_main, cost_sh, per_main, per_sh, n_cu);
  for (int pass = 0; pass < 4; ++pass) {
    bool improved = false;
    for (size_t i = 0; i < order.size(); ++i)
      for (size_t j = i + 1; j < order.size(); ++j) {
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
  std::vector<Slot> out;
  for (int i : order) out.push_back(slots[i]);
  return out;
}

void set_order(KArgs& a, const OrderShape& s) {
  a.n_order = 0;
  if (!a.causal || s.n_bands < 2 || s.n_bands > kMaxOrder) return;
  static std::mutex mu;
  static std::map<OrderShape, std::vector<Slot>> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(s);
  if (it == cache.end()) it = cache.emplace(s, plan_order(s)).first;
  const std::vector<Slot>& v = it->second;
  for (size_t i = 0; i < v.size(); ++i) {
    a.order[i] = v[i].tile;
    a.part[i] = v[i].part;
    a.sbi[i] = v[i].sbi;
    a.split[i] = v[i].split;
  }
  a.n_order = (int)v.size();
}

template <int D, int W, int BN, int OCC>
hipError_t launch_dw(KArgs a, const AttnParams& p, hipStream_t stream, int n_cu) {
  a.n_row_tiles = div_up(p.T * p.R, W * 32);
  const int max_split =
      p.split_ws ? split_cap(a.n_row_tiles, W * 32, p.R, p.T, BN, a.BG_main, n_cu) : 0;
  set_order(a, OrderShape{a.n_row_tiles, W * 32, p.R, p.T, BN, a.BG_main, a.BG - a.BG_main, n_cu,
                          a.BG == a.BG_main ? max_split : 0});
  a.ws = static_cast<float*>(p.split_ws);
  int n_split = 0;
  for (int i = 0; i < a.n_order; ++i) n_split += a.part[i] == 1;
  const dim3 grid((a.n_order ? a.n_order : a.n_row_tiles) * a.BG), block(W * 64);
  if (p.idx)
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, OCC, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, OCC, false>), grid, block, 0, stream, a);
  if (n_split == 0) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // One merge block per 256 (row, 8-column chunk) items of a split tile.
  const dim3 merge_grid(n_split * a.BG * (W * 32 * (D / 8) / 256));
  if (p.idx)
    hipLaunchKernelGGL((split_merge_kernel<D, W, true>), merge_grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((split_merge_kernel<D, W, false>), merge_grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// CU count of the current device (256 when it cannot be read).
int device_cus() {
  int n_cu = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  return n_cu;
}

// The configuration a launch takes: 12 waves / 32-key tiles when the grid
// gives every CU at least two 12-wave blocks' worth of waves, or when key
// splitting is on (a causal routed launch with a workspace) and the 12-wave
// grid is at most one block per CU; else 8 waves / 64-key tiles. In the
// second case the split 12-wave grid runs as one round and ends sooner than
// the 8-wave grid (GQE k=1 at B=2, T=4096: 118.9 against 127.4 us per call);
// at two rounds (k=2) the 8-wave grid is faster (161 against 176 us).
bool large_config(int BG, int T, int R, int n_cu, bool split) {
  const long long large_grid = (long long)BG * div_up(T * R, kWavesLarge * 32);
  return large_grid * kWavesLarge >= 24ll * n_cu || (split && large_grid <= n_cu);
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
  const int n_cu = device_cus();
  if (p.split_ws && p.q_shared) return hipErrorInvalidValue;  // key splitting is for plain routed launches
  if (large_config(a.BG, p.T, p.R, n_cu, p.split_ws && p.causal && !p.q_shared))
    return launch_dw<D, kWavesLarge, kBNLarge, kOccLarge>(a, p, stream, n_cu);
  return launch_dw<D, kWavesSmall, kBNSmall, kOccSmall>(a, p, stream, n_cu);
}

}  // namespace

bool attn_bf16_supports(int d) { return d == 64 || d == 128; }

size_t attn_bf16_split_ws_bytes(int B, int g, int T, int d, int R, int causal) {
  if (!causal || B <= 0 || T <= 0) return 0;
  const int n_cu = device_cus(), BG = B * g;
  const bool large = large_config(BG, T, R, n_cu, true);
  const int W = large ? kWavesLarge : kWavesSmall, kBN = large ? kBNLarge : kBNSmall;
  const int n_bands = div_up(T * R, W * 32);
  const int cap = split_cap(n_bands, W * 32, R, T, kBN, BG, n_cu);
  return (size_t)cap * BG * 2 * (size_t)(W * 32) * (d + 2) * sizeof(float);
}

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
