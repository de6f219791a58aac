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
#include <atomic>
#include <cstdlib>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <random>
#include <tuple>
#include <type_traits>
#include <vector>

#include "common.h"
#include "launch.h"
#include "plan.h"
#include "topk.h"

namespace gqa {
namespace {

// Two configurations: 12 waves with 32-key tiles (three waves per SIMD) for
// large grids, and 8 waves with 64-key tiles (two waves per SIMD, half the
// per-tile overhead) when a 12-wave grid would leave compute units without
// two workgroups' worth of work (short routed problems).
constexpr int kWavesLarge = 12, kBNLarge = 32, kOccLarge = 3;
constexpr int kWavesSmall = 8, kBNSmall = 64, kOccSmall = 2;
// 16 raw bytes at an address that is only 8-byte aligned (staged bf16 output rows).
typedef unsigned u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));
constexpr float kRescale = 8.0f;                      // lazy-rescale threshold, log2 units
constexpr float kRescaleSum = 256.0f;                 // 2^kRescale: a lane's tile sum above it raises the reference

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
  int32_t* idx;         // routed: kept heads (written here when logits is set)
  float* gate;          // routed: their gates (likewise)
  const float* logits;  // routed, selecting in the kernel: router logits [B, T, h]; else null
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
  // runs slot i of the planned order when n_order > 0, else row tile
  // n_row_tiles-1-i. A slot packs, in one 64-bit word read with one scalar
  // load: its row tile (bits 0-15), key-split point (16-31), part (32-39) and
  // split number sbi (40-47). Part 1 covers key tiles [0, split) of the row
  // tile, part 2 [split, n_tiles); part 0 covers them all. Part 1 writes its
  // partial result to workspace slot sbi * BG + bg and then sets
  // ready[sbi * BG + bg] to epoch; part 2 waits for that, merges the partial
  // into its own result and writes the rows.
  int n_order;
  uint64_t slot[kMaxOrder];
  float* ws;
  unsigned long long* ready;
  unsigned long long epoch;  // unique per launch (top bit set), so stale flags never match
  int wait_polls;            // bound of part 2's wait for the flag
};

__host__ __device__ inline int slot_tile(uint64_t s) { return (int)(s & 0xffffu); }
__host__ __device__ inline int slot_split(uint64_t s) { return (int)((s >> 16) & 0xffffu); }
__host__ __device__ inline int slot_part(uint64_t s) { return (int)((s >> 32) & 0xffu); }
__host__ __device__ inline int slot_sbi(uint64_t s) { return (int)((s >> 40) & 0xffu); }

// The router's selection for token t of (b, gam), made in the kernel from the
// logits: returns the kept-head mask and sets the slot-th kept head's group
// position and gate. Groups of up to 8 heads load their logits together into
// registers; larger ones read them from memory as the selection goes.
__device__ inline unsigned long long route_token(const KArgs& a, int b, int t, int gam, int slot, int* e,
                                                 float* gate) {
  const float* lg = a.logits + ((size_t)b * a.T + t) * a.h + gam * a.r;
  if (a.r <= 8) {
    float v[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = x < a.r ? lg[x] : 0.0f;
    return topk_rank_reg(v, a.r, a.R, slot, e, gate);
  }
  return topk_rank([&](int x) { return lg[x]; }, a.r, a.R, slot, e, gate);
}

// Zero rows of the heads the router did not keep, for the tokens whose first
// row lies in this block's row range. Called once the block's attention and
// output are done, with `kept` pointing to free LDS for one 64-bit mask per
// token: the kept heads of every token are gathered first, all loads
// independent, so the store loop that follows issues no loads. These rows
// (3/4 of the output at r = 4, k = 1) cost a few microseconds per block
// wherever they go; at the end they delay neither the block's first tile nor,
// in the loop, its tile copies (stores share the wait counter with the copies
// on this target).
template <int D, int W>
__device__ void zero_unselected_rows(const KArgs& a, int b, int gam, int row0, int n_rows,
                                     unsigned long long* kept) {
  constexpr int kThreads = W * 64, kRowsPerBlock = W * 32;
  const int R = a.R, r = a.r;
  const int t_lo = div_up(row0, R);
  const int t_hi = (min(row0 + kRowsPerBlock, n_rows) - 1) / R;
  if (t_hi < t_lo) return;  // uniform over the block
  const int n_tok = t_hi - t_lo + 1;  // at most kRowsPerBlock
  for (int i = threadIdx.x; i < n_tok; i += kThreads) {
    unsigned long long m = 0;
    if (a.logits) {
      int e_unused;
      float g_unused;
      m = route_token(a, b, t_lo + i, gam, 0, &e_unused, &g_unused);
    } else {
      const int32_t* sel = a.idx + ((size_t)(b * a.T + t_lo + i) * a.g + gam) * R;
      for (int j = 0; j < R; ++j) {
        const unsigned e = (unsigned)(sel[j] - gam * r);  // the kept head's place in its group
        if (e < 64u) m |= 1ull << e;
      }
    }
    kept[i] = m;
  }
  __syncthreads();
  // Each wave stores the zero rows of its tokens wave, wave + W, ...: their
  // masks are read together (one per lane) and handed out with readlane, and
  // one store instruction covers 64 / CPR rows of a token, 16 bytes per lane.
  constexpr int CPR = D / 8;             // 16-byte chunks of a bf16 row (8 elements each)
  constexpr int kHeadsPer = 64 / CPR;    // rows per store instruction
  static_assert(kRowsPerBlock / W <= 64, "a wave's tokens fit in one mask per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int my_tok = wave + W * lane;
  const unsigned long long my_mask = my_tok < n_tok ? kept[my_tok] : ~0ull;
  const unsigned mask_lo = (unsigned)my_mask, mask_hi = (unsigned)(my_mask >> 32);
  const int e_lane = lane / CPR, ch = lane % CPR;
  const size_t elt = a.out_bf16 ? 2 : 4;
  // Addresses: each lane's head offset is formed once per group of heads, and
  // the pointer then steps by a uniform stride from one of the wave's tokens to
  // the next (no 64-bit multiplies per store).
  const size_t tok_step = (size_t)W * a.o_t * elt;
  char* const base =
      static_cast<char*>(a.out) + (b * a.o_b + (size_t)(t_lo + wave) * a.o_t + (size_t)ch * 8) * elt;
  const int n_mine = n_tok > wave ? (n_tok - wave + W - 1) / W : 0;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int e0 = 0; e0 < r; e0 += kHeadsPer) {
    const int e = e0 + e_lane;
    const bool mine = e < r;
    char* p = base + (size_t)(gam * r + (mine ? e : 0)) * a.o_h * elt;
    for (int j = 0; j < n_mine; ++j, p += tok_step) {
      const unsigned long long m = ((unsigned long long)__builtin_amdgcn_readlane(mask_hi, j) << 32) |
                                   __builtin_amdgcn_readlane(mask_lo, j);
      if (mine && !((m >> e) & 1ull)) {
        __builtin_nontemporal_store(z, reinterpret_cast<u32x4*>(p));
        if (!a.out_bf16) __builtin_nontemporal_store(z, reinterpret_cast<u32x4*>(p) + 1);
      }
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
  // Per-wave table of the byte offset of each row's output row (from out or
  // out_sh), formed once with the row.
  __shared__ long long rowoff_all[W * 32];

  const int bid = blockIdx.x;
  const int bg = bid % a.BG;
  const int band = bid / a.BG;
  const uint64_t sl = a.n_order ? a.slot[__builtin_amdgcn_readfirstlane(band)] : 0;
  const int tile = !a.causal ? band : a.n_order ? slot_tile(sl) : a.n_row_tiles - 1 - band;
  const int part = slot_part(sl);
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
      if (a.logits) {
        int e;
        route_token(a, b, ri.t, gam, ri.slot, &e, &ri.gate);
        ri.head = gam * a.r + e;
      } else {
        const size_t o = ((size_t)(b * a.T + ri.t) * a.g + gam) * a.R + ri.slot;
        ri.head = a.idx[o];
        ri.gate = a.out_slots ? 1.0f : a.gate[o];
      }
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
  const int kt_lo = part == 2 ? slot_split(sl) : 0;
  const int kt_hi = part == 1 ? slot_split(sl) : n_tiles;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint16_t* const QOw = QO + wave_u * kQElems;
  int4* const tab = rowtab + wave_u * 32;
  long long* const rowoff = rowoff_all + wave_u * 32;
  const uint16_t* kbase = a.k + b * a.kv_b + gam * a.kv_g;
  const uint16_t* vbase = a.v + b * a.kv_b + gam * a.kv_g;
  // Byte offsets (from the tile's first key row) that this lane loads for the
  // wave's DMA instructions j = wave + W*i: K granules first, then V.
  // The sequence's last key tile may be partial (T not a multiple of kBN):
  // its rows past key T-1 load key T-1 instead (finite values that the mask
  // discards), so nothing past the K/V tensors is read. Its offsets are
  // formed once here; every tile then only selects between the two sets.
  const int last_full = a.T - 1 - (div_up(a.T, kBN) - 1) * kBN;  // last valid row of the last tile
  uint32_t dma_off[L::kMine], dma_off_last[L::kMine];
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
    dma_off_last[i] = (uint32_t)(min(row, last_full) * D + gr * 8) * 2u;
  }
  // Start the DMA of key tile kt into buffer buf.
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
      const uint32_t off = full ? dma_off[i] : dma_off_last[i];
      // The tile's base address is uniform: kept whole in SGPRs (readfirstlane
      // hides its parts from reassociation), so the copy takes the scalar-base
      // form (64-bit base in SGPRs + this lane's 32-bit offset) with no 64-bit
      // vector address arithmetic per tile.
      const uint64_t bu = reinterpret_cast<uint64_t>((isk ? kbase : vbase) + (size_t)key0 * D);
      const uint64_t bs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu);
      const uint16_t* src = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(bs) + off);
      uint16_t* dst = isk ? Kb + j * 512 : Vb + (j - L::kDmaK) * 512;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // The first key tile does not depend on the row table: its copy is in
  // flight while the rows are resolved and Q is requested.
  issue_tile(kt_lo, B0{});

  // Each lane resolves its own row once (rows past the end stand in as the
  // last row); lanes that move other rows read them from the table.
  if (hq == 0) {
    const RowInfo ri = row_info(min(rho, n_rows - 1));
    tab[l32] = make_int4(ri.t, ri.head, ri.slot, __float_as_int(ri.gate));
    const int oslot = a.out_slots ? gam * a.R + ri.slot : ri.head;
    rowoff[l32] = (long long)((shared ? ((size_t)b * a.T + ri.t) * D
                                      : b * a.o_b + (size_t)oslot * a.o_h + (size_t)ri.t * a.o_t) *
                              (a.out_bf16 ? 2 : 4));
    // Selecting in the kernel: each (token, slot) entry of idx and gate is
    // written once, by the lane of its row in the block that owns the row's
    // output (the first part of a key-split row tile).
    if (ROUTED && a.logits && !shared && part <= 1 && rho < n_rows) {
      const size_t o = ((size_t)(b * a.T + ri.t) * a.g + gam) * a.R + ri.slot;
      a.idx[o] = ri.head;
      a.gate[o] = ri.gate;
    }
  }
  // The table is the wave's own and one wave's LDS accesses take effect in
  // order, so its rows are read back below without a barrier. (A block
  // barrier here would first wait for the copy of the first K/V tile, and
  // only then let the Q copy start.)
  // The wave's 32 Q rows into QOw by DMA, granule by granule as for K (pad
  // granules receive a copy of granule 0).
  // The table entries of all the copies are read first, so the copies wait
  // for one LDS round trip rather than one per batch.
  int2 qrows[kQDma];
#pragma unroll
  for (int j = 0; j < kQDma; ++j) {
    const int row = min((j * 64 + lane) / L::kGPR, 31);
    const int4 ri = tab[row];
    qrows[j] = make_int2(ri.x, ri.y);
  }
#pragma unroll
  for (int j = 0; j < kQDma; ++j) {
    const int p = j * 64 + lane;
    const int row = p / L::kGPR;
    int gr = p - row * L::kGPR;
    if (gr >= L::kCPR || row > 31) gr = 0;
    const int2 ri = qrows[j];
    const uint16_t* src = (shared ? a.q_sh + (size_t)b * a.T * D : a.q + b * a.q_b + (size_t)ri.y * a.q_h) +
                          (size_t)ri.x * D + gr * 8;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(QOw + j * 512), 16, 0, 0);
  }

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
        const int lim = (a.causal ? t_row : a.T - 1) - key0 - 4 * hq;
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
      }

      // P^T as bf16 B operands: step u covers keys 16u .. 16u+15 of the tile.
      // The probabilities are taken against the current reference max first;
      // a score above it by more than kRescale (log2 units) shows as a
      // probability above 2^kRescale, so as a partial row sum above it (a sum
      // of probabilities each below 2^kRescale can exceed it too, which only
      // costs an unneeded raise of the reference). Only then is the tile's max
      // formed, the reference raised, the accumulators rescaled and the
      // probabilities taken again. This keeps the max reduction off the path
      // of every other tile. The row sum adds the rounded bf16 values, the
      // ones the MFMA uses.
      bf16x8 pf[kBN / 16];
      float lt[2] = {0.0f, 0.0f};
      auto probs = [&]() {
        lt[0] = lt[1] = 0.0f;
#pragma unroll
        for (int u = 0; u < kBN / 16; ++u) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(fmaf(s[u >> 1][8 * (u & 1) + j], a.c, -m_ref));
          pf[u] = pack_bf16x8(pv);
          const bf16x2* pp = reinterpret_cast<const bf16x2*>(&pf[u]);
#pragma unroll
          for (int j = 0; j < 4; ++j) lt[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp[j], ones, lt[u & 1], false);
        }
      };
      probs();
      // NaN and infinity (the first tile, against m_ref = -inf) take the raise too.
      if (__any(!(lt[0] + lt[1] <= kRescaleSum))) {
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) mloc = fmaxf(fmaxf(mloc, s[kb][i]), s[kb][i + 1]);
        const float mloc_s = mloc * a.c;
        const float m_new = fmaxf(m_ref, fmaxf(mloc_s, __shfl_xor(mloc_s, 32)));
        const float alpha = fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        probs();
      }
      l_run += lt[0] + lt[1];

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
  // bytes per lane (part 1 of a split tile: into its workspace slot).
  float l_tot = l_run + __shfl_xor(l_run, 32);
  // Key-split row tiles. Part 1 stores its partial result: its O rows divided
  // by their own sum l, rounded to bf16 (half the bytes of fp32 rows, written
  // and read on the critical path; the rounding is one bf16 step of a convex
  // combination of values, as for a bf16 output), then per row the reference
  // max m_ref and the sum l in fp32 (rows past the end included), and
  // publishes it. Part 2 waits for it, merges it
  // into its own rows as the online softmax merges two key ranges,
  //   m = max(m_1, m_2),  w_p = 2^(m_p - m),  O = w_1 l_1 (O_1 / l_1) + w_2 O_2,  l = w_1 l_1 + w_2 l_2,
  // and then writes the rows like an unsplit tile.
  const bool partial = part == 1;
  // Slot layout: kRowsPerBlock bf16 rows of D, then kRowsPerBlock maxima and
  // kRowsPerBlock sums (fp32): kRowsPerBlock * (D / 2 + 2) floats.
  constexpr int kMOff = kRowsPerBlock * (D / 2), kLOff = kRowsPerBlock * (D / 2 + 1);
  float* const pws = part ? a.ws + (size_t)(slot_sbi(sl) * a.BG + bg) * ((size_t)kRowsPerBlock * (D / 2 + 2)) : nullptr;
  if (part == 2) {
    unsigned long long* const flag = a.ready + slot_sbi(sl) * a.BG + bg;
    // Part 1 waits for nothing: it stores its partial as soon as its own key
    // tiles are done, at most one job after this block (fewer blocks spin here
    // than there are CUs, so part 1 always finds one). The wait is bounded all
    // the same (wait_polls, by default 2^20 polls: well over 100 ms), after
    // which the rows are NaN.
    __shared__ int ready_ok;
    if (tid == 0) {
      int ok = 0;
      for (int it = 0; it < a.wait_polls; ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) {
          ok = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // Consumed: cleared, so that a replay of this very launch (same epoch,
      // e.g. from a captured graph) waits for its own part 1 again.
      if (ok) __hip_atomic_store(flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ready_ok = ok;
    }
    // The barrier orders every wave's reads below after thread 0's acquire
    // (one cache invalidation for the block, not one per wave).
    __syncthreads();
    const int prow = wave * 32 + l32;
    const float m1 = pws[kMOff + prow], l1 = pws[kLOff + prow];
    // Part 1's rows are stored normalised (O_1 / l_1) in bf16.
    const uint16_t* const p1r = reinterpret_cast<const uint16_t*>(pws) + (size_t)prow * D;
    uint2 x[D / 32][4];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) x[db][i4] = *reinterpret_cast<const uint2*>(p1r + 32 * db + 8 * i4 + 4 * hq);
    const float mm = fmaxf(m_ref, m1);
    const float w2 = ready_ok ? fast_exp2(m_ref - mm) : NAN, w1 = fast_exp2(m1 - mm);
    const float w1l = w1 * l1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        o[db][4 * i4] = w2 * o[db][4 * i4] + w1l * __uint_as_float(x[db][i4].x << 16);
        o[db][4 * i4 + 1] = w2 * o[db][4 * i4 + 1] + w1l * __uint_as_float(x[db][i4].x & 0xffff0000u);
        o[db][4 * i4 + 2] = w2 * o[db][4 * i4 + 2] + w1l * __uint_as_float(x[db][i4].y << 16);
        o[db][4 * i4 + 3] = w2 * o[db][4 * i4 + 3] + w1l * __uint_as_float(x[db][i4].y & 0xffff0000u);
      }
    l_tot = w2 * l_tot + w1 * l1;
  }
  if (partial && hq == 0) {
    pws[kMOff + wave * 32 + l32] = m_ref;
    pws[kLOff + wave * 32 + l32] = l_tot;
  }
  const float inv = (partial ? 1.0f : __int_as_float(tab[l32].w)) / l_tot;
  constexpr int kG = D * 2 / 16;            // 16-byte granules per staged row
  constexpr int kRowsPer = 64 / kG;         // rows per store instruction
  char* const stage = reinterpret_cast<char*>(QOw);
  const bool bf16_out = a.out_bf16 || partial;  // part 1 stores its normalised rows in bf16
  const int n_pass = bf16_out ? 1 : 2;
  // Staged row pitch in bytes. A bf16 row is staged by 8-byte writes, one
  // per lane and row; at an odd multiple of 8 bytes the 32 rows of a write
  // fall in distinct banks (at the Q pitch, rows 16 apart share them). Its
  // 16-byte reads are then only 8-byte aligned. fp32 rows are staged by
  // 16-byte writes at the Q pitch.
  const int kRowB = bf16_out ? L::kPitch * 2 - 8 : L::kPitch * 2;
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
    // Each wave reads back only the rows it staged; one wave's LDS accesses
    // take effect in order, so no barrier is needed here.
    // All of the wave's staged rows (and their table entries) are read before
    // the first store, so the reads wait for LDS once rather than per store.
    constexpr int kIt = 32 / kRowsPer;
    u32x4 vs[kIt];
    long long rs[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int row = i * kRowsPer + lane / kG;
      vs[i] = *reinterpret_cast<const u32x4_a8*>(stage + row * kRowB + (lane % kG) * 16);
      rs[i] = rowoff[row];
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int row = i * kRowsPer + lane / kG;
      const int gran = lane % kG;
      const u32x4 v = vs[i];
      const int rr = wrow0 + row;
      if (partial) {
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(pws) + (size_t)(wave * 32 + row) * D + gran * 8) = v;
      } else if (rr < n_rows) {
        char* const outp = static_cast<char*>(shared ? a.out_sh : a.out);
        const size_t ob = (size_t)rs[i] + (size_t)pass * D * 2 + gran * 16;
        // Nontemporal: the output is not read again here, and streaming it
        // past L2 leaves the K/V tiles that other row tiles reuse in place.
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(outp + ob));
      }
    }
  }
  if (partial) {
    // Every wave waits for its own partial stores to complete, the barrier
    // for all waves, and thread 0's release then makes them visible
    // device-wide before the flag (one cache write-back for the block, not
    // one per wave). A workgroup barrier alone does not wait for stores.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(a.ready + slot_sbi(sl) * a.BG + bg, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The K/V buffers are free since the last tile's barrier.
  static_assert(L::kElems * 2 >= kRowsPerBlock * 8, "the kept-head masks must fit in a K buffer");
  if (ROUTED && a.zero_unselected && !shared && part <= 1)
    zero_unselected_rows<D, W>(a, b, gam, row0, n_rows, reinterpret_cast<unsigned long long*>(K0));
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
    a.slot[i] = (uint64_t)v[i].tile | ((uint64_t)v[i].split << 16) | ((uint64_t)v[i].part << 32) |
                ((uint64_t)v[i].sbi << 40);
  }
  a.n_order = (int)v.size();
}

// Partial slots of the key-split tiles: one per split tile and problem, W*32
// rows of D bf16 values plus (max, sum) in fp32 per row.
size_t split_partial_bytes(int cap, int BG, int rows, int d) {
  return (size_t)cap * BG * rows * (d / 2 + 2) * sizeof(float);
}

// Polls of the ready flag before a second part gives up: 2^20, or the
// GQA_SPLIT_WAIT_POLLS environment variable (0 .. 2^20), which lets tests take
// the timeout path (NaN rows) with every kernel still ending normally.
int split_wait_polls() {
  constexpr long kMax = 1 << 20;
  const char* env = std::getenv("GQA_SPLIT_WAIT_POLLS");
  if (!env || !*env) return (int)kMax;
  const long v = std::strtol(env, nullptr, 10);
  return (int)(v < 0 ? 0 : v > kMax ? kMax : v);
}

// A value no earlier launch of this process used and that uninitialised
// workspace is most unlikely to hold: a random start with the top bit set,
// counting up.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> next{[] {
    std::random_device rd;
    return (((unsigned long long)rd() << 32) ^ rd()) | (1ull << 63);
  }()};
  return next.fetch_add(1) | (1ull << 63);
}

template <int D, int W, int BN, int OCC>
hipError_t launch_dw(KArgs a, const AttnParams& p, hipStream_t stream, int n_cu) {
  a.n_row_tiles = div_up(p.T * p.R, W * 32);
  const int max_split =
      p.split_ws ? split_cap(a.n_row_tiles, W * 32, p.R, p.T, BN, a.BG_main, n_cu) : 0;
  set_order(a, OrderShape{a.n_row_tiles, W * 32, p.R, p.T, BN, a.BG_main, a.BG - a.BG_main, n_cu,
                          a.BG == a.BG_main ? max_split : 0});
  // Workspace: the partial slots of up to max_split split tiles per problem,
  // then their ready flags.
  a.ws = static_cast<float*>(p.split_ws);
  a.ready = p.split_ws ? reinterpret_cast<unsigned long long*>(static_cast<char*>(p.split_ws) +
                                                               split_partial_bytes(max_split, a.BG_main, W * 32, D))
                       : nullptr;
  a.epoch = p.split_ws ? next_epoch() : 0;
  a.wait_polls = split_wait_polls();
  const dim3 grid((a.n_order ? a.n_order : a.n_row_tiles) * a.BG), block(W * 64);
  if (p.idx)
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, OCC, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, W, BN, OCC, false>), grid, block, 0, stream, a);
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
  a.idx = const_cast<int32_t*>(p.idx);
  a.gate = const_cast<float*>(p.gate);
  a.logits = p.logits;
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
  if (cap == 0) return 0;
  return split_partial_bytes(cap, BG, W * 32, d) + (size_t)cap * BG * sizeof(unsigned long long);
}

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
