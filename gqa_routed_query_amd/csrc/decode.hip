// Grouped-query attention decode over a KV cache: one new query token per
// sequence, bf16 cache (fp32 caches: decode_f32_kernel below), fp32
// accumulation, split-K with a log-sum-exp merge.
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
//  * Work is balanced over the keys, not over sequences. The cached keys of
//    all (batch, KV group) streams, laid end to end, form one key range; every
//    workgroup of the grid takes an equal contiguous share of it (computed on
//    the device from lens), so sequences of very different lengths still keep
//    every CU streaming until the end. One grid holds exactly the workgroups
//    the chip keeps resident.
//  * A share crosses stream boundaries. A stream that lies wholly in one
//    share is finished by that workgroup, which writes the output rows; a
//    stream cut by share boundaries leaves one partial (max, sum, accumulator
//    per head) per piece, and a second kernel merges the pieces by
//    log-sum-exp. A workgroup writes at most two partials: for its first and
//    its last stream.
//  * Inside a piece the 4 waves take interleaved 32-key sub-blocks, so the
//    workgroup reads 128 consecutive cache rows (32 KiB of K, 32 KiB of V) per
//    step. Every cached K/V row is read once, with coalesced nontemporal
//    16-byte loads into registers (the streaming hint alone took the decode
//    workload from 5.7 to 6.3 TB/s), staged through a wave-private padded LDS
//    buffer, and serves all h/g query heads of its group. A wave's next sub-block (also in
//    a later piece) is loading while the current one is multiplied; at the end
//    of a piece the waves combine their (max, sum, accumulator) through LDS.
//  * Per 32-key sub-block: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (heads are
//    the 16-wide B columns; groups with fewer than 16 heads leave columns
//    idle -- the matrix cores have far more headroom than HBM), the online
//    softmax with a lazily raised reference max, and O^T += V^T P^T with V
//    transposed by ds_read_b64_tr_b16.
//  * Cache rows at or beyond lens[b] are never loaded: a sub-block's rows past
//    the end of its piece re-read the piece's last row (always a valid row)
//    and are masked out of the softmax. Padding may hold anything, NaN
//    included.
#include <cstdlib>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int kWaves = 4;            // waves per workgroup; they share one key share
constexpr int kThreads = kWaves * 64;
constexpr int kSub = 32;             // keys per sub-block
constexpr int kMinShare = 256;       // smallest key share per workgroup
constexpr float kRescale = 8.0f;     // lazy-rescale threshold, log2 units

template <int D>
struct DTile {
  static constexpr int kPitch = D + 8;   // 16-byte pad: A-operand reads of 16 rows hit distinct banks
  static constexpr int vPitch = D + 16;  // 32-byte pad: 8 rows of a transposing read hit distinct banks
  static constexpr int kElems = kSub * kPitch;
  static constexpr int vElems = kSub * vPitch;
  static constexpr int wElems = kElems + vElems;    // one wave's LDS staging area
  static constexpr int kCPR = D / 8;
  static constexpr int kLoads = kSub * kCPR / 64;   // 16-byte loads per lane per sub-block (K or V)
  // S^T = K Q^T on 16x16x32 MFMAs: lane group grp (lane / 16) holds d in
  // [grp * kGS, grp * kGS + 8 * kDS) of its row, in kDS steps of 8. At D = 16
  // one step covers d < 16 in groups 0 and 1; groups 2 and 3 hold zeros.
  static constexpr int kDS = D >= 32 ? D / 32 : 1;   // 32-wide reduction steps for S^T
  static constexpr int kGS = D >= 32 ? D / 4 : 8;    // first d of lane group grp: grp * kGS
  __device__ static bool group_live(int grp) { return D >= 32 || grp * kGS < D; }
};

struct KArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* lens;
  void* out;
  float* part_acc;  // [n_units, 2, R, D]
  float* part_ml;   // [n_units, 2, R, 2]: reference max (log2 units), sum
  const int32_t* idx;  // routed: [B, g, R] global head ids of the kept heads, else null
  const float* gate;   // routed: [B, g, R] gates, else null
  int B, h, g, r, T_max;
  int R;            // rows per KV group: r (dense) or the kept heads k (routed)
  int n_units;      // workgroups sharing the key range
  float c;          // scale * log2(e)
  int out_bf16;
};

__device__ __forceinline__ int seq_len(const KArgs& a, int b) {
  return min(max(a.lens[b], 0), a.T_max);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Global query head of row e (< R) of KV group gam of sequence b.
template <bool ROUTED>
__device__ __forceinline__ int head_of(const KArgs& a, int b, int gam, int e) {
  return ROUTED ? a.idx[((size_t)b * a.g + gam) * a.R + e] : gam * a.r + e;
}

// Keys of all streams: g * sum_b lens[b]. Every lane returns the total.
__device__ __forceinline__ long long total_keys(const KArgs& a, int lane) {
  long long t = 0;
  for (int b = lane; b < a.B; b += 64) t += seq_len(a, b);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  return t * a.g;
}

// The equal share of the key range each wave takes.
__device__ __forceinline__ long long share_of(long long total, int n_units) {
  const long long p = (total + n_units - 1) / n_units;
  return p > kMinShare ? p : (long long)kMinShare;
}

// A piece of one stream: keys [k0, k1) of stream (b, gam), which has len keys.
struct Piece {
  int b, gam, k0, k1, len;
};

// The stream holding global key position pos (< total), as a piece starting
// there and ending at min(stream end, pos + avail).
__device__ __forceinline__ Piece locate(const KArgs& a, long long pos, long long avail, int lane) {
  long long base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int len = b < a.B ? seq_len(a, b) : 0;
    const long long n = (long long)a.g * len;
    long long incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const long long lo = base + incl - n;
    const unsigned long long hit = __ballot(lo <= pos && pos < base + incl);
    if (hit) {
      const int src = __ffsll(hit) - 1;
      const int sl = uniform(__shfl(len, src));
      const long long off = pos - __shfl(lo, src);
      Piece p;
      p.b = uniform(b0 + src);
      p.len = sl;
      p.gam = uniform((int)(off / sl));
      p.k0 = uniform((int)(off - (long long)p.gam * sl));
      p.k1 = (int)min((long long)sl, p.k0 + avail);
      p.k1 = uniform(p.k1);
      return p;
    }
    base += __shfl(incl, 63);
  }
  return Piece{a.B, 0, 0, 0, 0};  // not reached for pos < total
}

// The piece after p, if this wave's share [.., end) goes on past it; pos is
// the global position of p.k0 and is advanced to the next piece's start.
__device__ __forceinline__ bool next_piece(const KArgs& a, const Piece& p, long long& pos, long long end, Piece& n) {
  pos += p.k1 - p.k0;
  if (pos >= end) return false;
  n = p;
  n.k0 = 0;
  if (p.gam + 1 < a.g) {
    n.gam = p.gam + 1;
  } else {
    n.gam = 0;
    int b = p.b + 1;
    while (seq_len(a, b) == 0) ++b;  // pos < total: a non-empty stream follows
    n.b = uniform(b);
    n.len = uniform(seq_len(a, b));
  }
  n.k1 = uniform((int)min((long long)n.len, end - pos));
  return true;
}

template <int D, int HB, bool ROUTED>
__device__ __forceinline__ void load_q(const KArgs& a, const Piece& p, int grp, int i16,
                                       bf16x8 (&qf)[HB][DTile<D>::kDS]) {
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int e = hb * 16 + i16;
    const int head = head_of<ROUTED>(a, p.b, p.gam, min(e, a.R - 1));
    const bool live = DTile<D>::group_live(grp);
    const uint16_t* qrow = a.q + ((size_t)p.b * a.h + head) * D + (live ? grp * DTile<D>::kGS : 0);
#pragma unroll
    for (int ds = 0; ds < DTile<D>::kDS; ++ds) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 8 * ds);
      if (e >= a.R || !live) x = bf16x8{};
      qf[hb][ds] = x;
    }
  }
}

// Coalesced 16-byte loads of one 32-key sub-block of K and V into registers:
// chunk c = lane + 64i is row c / (D/8), column (c % (D/8)) * 8. Rows at or
// past the piece end k1 re-read row k1-1 (masked out of the softmax later).
template <int D>
__device__ __forceinline__ void load_sub(const KArgs& a, const Piece& p, int sb0, int lane,
                                         u32x4 (&kr)[DTile<D>::kLoads], u32x4 (&vr)[DTile<D>::kLoads]) {
  using L = DTile<D>;
  const size_t base = ((size_t)p.b * a.g + p.gam) * a.T_max * D;
#pragma unroll
  for (int i = 0; i < L::kLoads; ++i) {
    const int cidx = lane + 64 * i;
    const int key = min(sb0 + cidx / L::kCPR, p.k1 - 1);
    const size_t off = base + (size_t)key * D + (cidx % L::kCPR) * 8;
    // Nontemporal: every cached row is read once per call.
    kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.kc + off));
    vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vc + off));
  }
}

// The sub-block of this wave that follows (p, sb) in the block's piece
// sequence, for sub-blocks of SUB keys: the next one of the piece, else the
// wave's first one in a later piece (pieces shorter than SUB * wave keys have
// none for this wave). pos is the global position of p.k0 and moves along
// with p. False when the share has no further sub-block for this wave.
template <int SUB = kSub>
__device__ __forceinline__ bool next_sub(const KArgs& a, Piece& p, long long& pos, long long end,
                                         int& sb, int& pi, int wave) {
  if (sb + kWaves * SUB < p.k1) {
    sb += kWaves * SUB;
    return true;
  }
  while (true) {
    Piece n;
    if (!next_piece(a, p, pos, end, n)) return false;
    p = n;
    ++pi;
    if (wave * SUB < p.k1) {
      sb = wave * SUB;
      return true;
    }
  }
}

// The end of a piece, after each wave has put its (max, sum, accumulator) of
// heads e0 .. e0+15 in LDS (row wave * 16 + head - e0, pitch D + 4: D values,
// max, sum): the waves' results merge by log-sum-exp, and the rows go out as
// output when the piece is the whole stream (whole), else as the partial of
// slot `slot` of this unit. Rows e >= R are skipped.
template <int D, bool ROUTED>
__device__ __forceinline__ void combine_rows(const KArgs& a, const float* comb, const Piece& cur, int e0,
                                             int unit, int slot, bool whole, int tid) {
  constexpr int kCP = D + 4;
  for (int x = tid; x < 16 * D; x += kThreads) {
    const int hh = x / D;
    const int d = x - hh * D;
    const int e = e0 + hh;
    if (e >= a.R) break;  // x only grows
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, comb[(wv * 16 + hh) * kCP + D]);
    float acc = 0.0f, den = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float* src = comb + (wv * 16 + hh) * kCP;
      const float mw = src[D];
      const float sc = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
      acc += sc * src[d];
      den += sc * src[D + 1];
    }
    if (whole) {
      const int head = head_of<ROUTED>(a, cur.b, cur.gam, e);
      const size_t off = ((size_t)cur.b * a.h + head) * D + d;
      float y = acc / den;
      if (ROUTED) y *= a.gate[((size_t)cur.b * a.g + cur.gam) * a.R + e];
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[off] = static_cast<uint16_t>(pack_bf16x2(y, 0.0f) & 0xffffu);
      else
        static_cast<float*>(a.out)[off] = y;
    } else {
      const size_t prow = ((size_t)unit * 2 + slot) * a.R + e;
      a.part_acc[prow * D + d] = acc;
      if (d == 0) {
        a.part_ml[prow * 2 + 0] = M;
        a.part_ml[prow * 2 + 1] = den;
      }
    }
  }
}

template <int D, int HB, bool ROUTED>
__global__ __launch_bounds__(kThreads) void decode_kernel(KArgs a) {
  using L = DTile<D>;
  constexpr int kCP = D + 4;                     // combine row: D values, max, sum, 16-byte pitch
  constexpr int kComb = kWaves * 16 * kCP;      // floats of one head block's combine
  constexpr int kSmemBytes =
      (kWaves * L::wElems * 2 > kComb * 4) ? kWaves * L::wElems * 2 : kComb * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int unit = blockIdx.x;
  const long long total = total_keys(a, lane);
  const long long share = share_of(total, a.n_units);
  const long long start = (long long)unit * share;
  if (start >= total) return;  // uniform over the block
  const long long end = min(start + share, total);

  const int grp = lane >> 4;
  const int i16 = lane & 15;
  uint16_t* Kw = reinterpret_cast<uint16_t*>(smem) + wave * L::wElems;
  uint16_t* Vw = Kw + L::kElems;
  const int tr_row = 4 * grp + (i16 >> 2);
  const int tr_col = 4 * (i16 & 3);

  // cur: the piece being reduced (same on every wave). ld: the piece of the
  // sub-block this wave has in flight (ld_pi its index, ld_sb its first key).
  long long cur_pos = start;
  Piece cur = locate(a, start, end - start, lane);
  long long ld_pos = cur_pos;
  Piece ld = cur;
  int ld_pi = 0, ld_sb = cur.k0 + wave * kSub;
  bool ld_ok = ld_sb < cur.k1 || next_sub(a, ld, ld_pos, end, ld_sb, ld_pi, wave);
  if (ld_sb >= ld.k1) ld_ok = false;

  u32x4 kr[L::kLoads], vr[L::kLoads];
  if (ld_ok) load_sub<D>(a, ld, ld_sb, lane, kr, vr);
  bf16x8 qf[HB][L::kDS];
  float* comb = reinterpret_cast<float*>(smem);

  for (int pi = 0;; ++pi) {
    load_q<D, HB, ROUTED>(a, cur, grp, i16, qf);
    f32x4 o[HB][D / 16];
    float m_run[HB], l_run[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m_run[hb] = -INFINITY;
      l_run[hb] = 0.0f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[hb][db] = f32x4{};
    }
    const int k1 = cur.k1;

    // This wave's sub-blocks of the piece: keys k0 + 32*wave + 128*i.
    while (ld_ok && ld_pi == pi) {
#pragma unroll
      for (int i = 0; i < L::kLoads; ++i) {
        const int cidx = lane + 64 * i;
        const int row = cidx / L::kCPR, col = (cidx % L::kCPR) * 8;
        *reinterpret_cast<u32x4*>(Kw + row * L::kPitch + col) = kr[i];
        *reinterpret_cast<u32x4*>(Vw + row * L::vPitch + col) = vr[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int cur_sb = ld_sb;
      ld_ok = next_sub(a, ld, ld_pos, end, ld_sb, ld_pi, wave);
      if (ld_ok) load_sub<D>(a, ld, ld_sb, lane, kr, vr);

      // S^T[key][head]: lane holds keys cur_sb + 16kb + 4grp + i.
      f32x4 s[HB][2];
      {
        bf16x8 kf[2][L::kDS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ds = 0; ds < L::kDS; ++ds)
            kf[kb][ds] = L::group_live(grp)
                             ? *reinterpret_cast<const bf16x8*>(Kw + (16 * kb + i16) * L::kPitch + grp * L::kGS + 8 * ds)
                             : bf16x8{};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            s[hb][kb] = f32x4{};
#pragma unroll
            for (int ds = 0; ds < L::kDS; ++ds) s[hb][kb] = mfma16x16x32(kf[kb][ds], qf[hb][ds], s[hb][kb]);
          }
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (cur_sb + 16 * kb + 4 * grp + i >= k1) s[hb][kb][i] = -INFINITY;
            mloc = fmaxf(mloc, s[hb][kb][i]);
          }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_cand = mloc * a.c;
        // Raise the reference max only when a score exceeds it by more than
        // 2^kRescale; otherwise keep it (probabilities stay below 2^kRescale).
        if (__any(m_cand > m_run[hb] + kRescale)) {
          const float m_new = fmaxf(m_run[hb], m_cand);
          const float alpha = fast_exp2(m_run[hb] - m_new);
          m_run[hb] = m_new;
          l_run[hb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) o[hb][db] = o[hb][db] * alpha;
        }
        float pv[8];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp2(fmaf(s[hb][j >> 2][j & 3], a.c, -m_run[hb]));
          psum += pv[j];
        }
        l_run[hb] += psum;
        const bf16x8 pf = pack_bf16x8(pv);
        // Element j of pf is key 4grp + j (j < 4) or 16 + 4grp + j-4.
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const uint16_t* p0 = Vw + tr_row * L::vPitch + 16 * db + tr_col;
          const bf16x8 vf = lds_read_tr_pair(p0, p0 + 16 * L::vPitch);
          o[hb][db] = mfma16x16x32(vf, pf, o[hb][db]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }

    // Combine the 4 waves through LDS, one head block at a time; write the
    // output rows when the piece is the whole stream, else a partial in slot 0
    // (the share's first piece) or 1 (its last).
    const bool whole = cur.k0 == 0 && k1 == cur.len;
    const int slot = pi == 0 ? 0 : 1;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float lsum = l_run[hb];
      lsum += __shfl_xor(lsum, 16);
      lsum += __shfl_xor(lsum, 32);
      __syncthreads();  // LDS is free: staging buffers consumed, previous head block read
      float* w = comb + (wave * 16 + i16) * kCP;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4*>(w + 16 * db + 4 * grp) = o[hb][db];
      if (grp == 0) {
        w[D] = m_run[hb];
        w[D + 1] = lsum;
      }
      __syncthreads();
      combine_rows<D, ROUTED>(a, comb, cur, hb * 16, unit, slot, whole, tid);
    }
    Piece n;
    if (!next_piece(a, cur, cur_pos, end, n)) break;
    cur = n;
    __syncthreads();  // combine reads done before the staging buffers are rewritten
  }
}

// fp32 caches. The shares, pieces and combine of decode_kernel, with the
// matrix work on v_mfma_f32_16x16x4_f32 (full fp32 operands) and no LDS in the
// key loop: both operands are loaded from HBM straight into the MFMA lane
// layout. For lane l = 16 grp + i16 the instruction takes A[i16][grp] and
// B[grp][i16] and returns rows 4 grp + v (v < 4) of column i16.
//  * S^T = K Q^T per 16-key sub-block (heads are the 16 columns): MFMA (i, j),
//    i < D/16, j < 4, reduces over d = 16 i + 4 grp + j, so lane (i16, grp)
//    reads 4 values at d = 16 i + 4 grp of key row i16 and of its head's
//    query row; one load instruction covers 64 contiguous bytes of 16 rows.
//  * O^T += V^T P^T: MFMA (v, db) reduces over keys 4 grp + v -- the keys
//    whose probabilities lane (i16, grp) holds after the scores -- and its
//    result row i is d = i * D/16 + db, so lane (i16, grp) reads the D/16
//    contiguous values at d = i16 * D/16 of V row 4 grp + v.
// A wave takes 16-key sub-blocks (keys k0 + 16 wave + 64 i of a piece) and
// loads its next one while the current one is multiplied. One launch covers
// 16 heads of each group per blockIdx.y (e0 = 16 blockIdx.y), so groups of
// more than 16 heads read their cache once per 16 heads.
constexpr int kSubF = 16;

__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// N contiguous floats at p (16-byte aligned for N >= 4, 8-byte for N == 2),
// nontemporal: every cached row is read once per call.
template <int N>
__device__ __forceinline__ void load_floats_nt(const float* p, float (&x)[N]) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * i + j] = t[j];
    }
  } else if constexpr (N == 2) {
    const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    x[0] = t[0];
    x[1] = t[1];
  } else {
    x[0] = __builtin_nontemporal_load(p);
  }
}

// K and V operands of the 16-key sub-block at sb0 of piece p (rows at or past
// p.k1 re-read row k1-1 and are masked out of the softmax later).
template <int D>
__device__ __forceinline__ void load_sub_f32(const KArgs& a, const Piece& p, int sb0, int grp, int i16,
                                             float (&kf)[D / 4], float (&vf)[4][D / 16]) {
  const float* kc = reinterpret_cast<const float*>(a.kc);
  const float* vc = reinterpret_cast<const float*>(a.vc);
  const size_t base = ((size_t)p.b * a.g + p.gam) * a.T_max * D;
  const size_t krow = base + (size_t)min(sb0 + i16, p.k1 - 1) * D;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    float t[4];
    load_floats_nt<4>(kc + krow + 16 * i + 4 * grp, t);
#pragma unroll
    for (int j = 0; j < 4; ++j) kf[4 * i + j] = t[j];
  }
#pragma unroll
  for (int v = 0; v < 4; ++v)
    load_floats_nt<D / 16>(vc + base + (size_t)min(sb0 + 4 * grp + v, p.k1 - 1) * D + i16 * (D / 16), vf[v]);
}

template <int D, bool ROUTED>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(KArgs a) {
  constexpr int kCP = D + 4;                 // combine row: D values, max, sum, 16-byte pitch
  __shared__ __attribute__((aligned(16))) float comb[kWaves * 16 * kCP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int unit = blockIdx.x;
  const int e0 = 16 * blockIdx.y;  // this block's heads of each group: e0 .. e0+15
  const long long total = total_keys(a, lane);
  const long long share = share_of(total, a.n_units);
  const long long start = (long long)unit * share;
  if (start >= total) return;  // uniform over the block
  const long long end = min(start + share, total);

  const int grp = lane >> 4;
  const int i16 = lane & 15;
  const float* qs = reinterpret_cast<const float*>(a.q);

  long long cur_pos = start;
  Piece cur = locate(a, start, end - start, lane);
  long long ld_pos = cur_pos;
  Piece ld = cur;
  int ld_pi = 0, ld_sb = cur.k0 + wave * kSubF;
  bool ld_ok = ld_sb < cur.k1 || next_sub<kSubF>(a, ld, ld_pos, end, ld_sb, ld_pi, wave);
  if (ld_sb >= ld.k1) ld_ok = false;

  float kr[D / 4], vr[4][D / 16];
  if (ld_ok) load_sub_f32<D>(a, ld, ld_sb, grp, i16, kr, vr);

  for (int pi = 0;; ++pi) {
    // Q^T operand: lane (i16, grp) holds d = 16 i + 4 grp + j of head row e0 + i16.
    float qf[D / 4];
    {
      const int e = e0 + i16;
      const int head = head_of<ROUTED>(a, cur.b, cur.gam, min(e, a.R - 1));
      const float* qrow = qs + ((size_t)cur.b * a.h + head) * D;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        float t[4];
        load_floats_nt<4>(qrow + 16 * i + 4 * grp, t);
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[4 * i + j] = e < a.R ? t[j] : 0.0f;
      }
    }
    f32x4 o[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.0f;
    const int k1 = cur.k1;

    while (ld_ok && ld_pi == pi) {
      float kc[D / 4], vc[4][D / 16];
#pragma unroll
      for (int i = 0; i < D / 4; ++i) kc[i] = kr[i];
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < D / 16; ++i) vc[v][i] = vr[v][i];
      const int cur_sb = ld_sb;
      ld_ok = next_sub<kSubF>(a, ld, ld_pos, end, ld_sb, ld_pi, wave);
      if (ld_ok) load_sub_f32<D>(a, ld, ld_sb, grp, i16, kr, vr);

      // S^T[key][head]: lane holds keys cur_sb + 4 grp + v of head e0 + i16.
      f32x4 s = f32x4{};
#pragma unroll
      for (int i = 0; i < D / 4; ++i) s = mfma16x16x4f32(kc[i], qf[i], s);
      float mloc = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (cur_sb + 4 * grp + v >= k1) s[v] = -INFINITY;
        mloc = fmaxf(mloc, s[v]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_cand = mloc * a.c;
      // The reference max is raised only when a score exceeds it by more than
      // 2^kRescale (probabilities stay below 2^kRescale); the final division
      // by the row sum is exact whatever reference was used.
      if (__any(m_cand > m_run + kRescale)) {
        const float m_new = fmaxf(m_run, m_cand);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[db] = o[db] * alpha;
      }
      float pv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[v] = fast_exp2(fmaf(s[v], a.c, -m_run));
        l_run += pv[v];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[db] = mfma16x16x4f32(vc[v][db], pv[v], o[db]);
    }

    // Combine the 4 waves through LDS; rows e0 .. e0+15 go out as output or
    // as a partial in slot 0 (the share's first piece) or 1 (its last).
    const bool whole = cur.k0 == 0 && k1 == cur.len;
    const int slot = pi == 0 ? 0 : 1;
    float lsum = l_run;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    __syncthreads();  // the previous piece's combine reads are done
    float* w = comb + (wave * 16 + i16) * kCP;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) w[(4 * grp + v) * (D / 16) + db] = o[db][v];
    if (grp == 0) {
      w[D] = m_run;
      w[D + 1] = lsum;
    }
    __syncthreads();
    combine_rows<D, ROUTED>(a, comb, cur, e0, unit, slot, whole, tid);
    Piece n;
    if (!next_piece(a, cur, cur_pos, end, n)) break;
    cur = n;
  }
}

// 17 to 32 query heads per KV group (MQA at h = 32): the shares, pieces and
// staging of decode_kernel, with the group's heads as the 32 columns of
// v_mfma_f32_32x32x16_bf16 -- the prefill kernel's layout: S^T of a 32-key
// sub-block is one 32x32 accumulator, O^T four, and lane l holds head l % 32.
// With the heads in 16-wide blocks a wave needs ~346 registers and spills, and
// a CU holds one workgroup; in this form it stays within 256 (two workgroups
// per CU) and does half the matrix work. Measured at 32 heads per group (B=32,
// T=16384, 268 MB of cache) it streams at the same rate as one workgroup per
// CU: the cache bytes already in flight were not what limited it there.
template <int D, bool ROUTED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode32_kernel(KArgs a) {
  using L = DTile<D>;
  constexpr int kCP = D + 4;                     // combine row: D values, max, sum, 16-byte pitch
  constexpr int kComb = kWaves * 32 * kCP;      // floats of the combine (32 heads per wave)
  constexpr int kSmemBytes =
      (kWaves * L::wElems * 2 > kComb * 4) ? kWaves * L::wElems * 2 : kComb * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int unit = blockIdx.x;
  const long long total = total_keys(a, lane);
  const long long share = share_of(total, a.n_units);
  const long long start = (long long)unit * share;
  if (start >= total) return;  // uniform over the block
  const long long end = min(start + share, total);

  const int l32 = lane & 31;
  const int hq = lane >> 5;
  const int grp = lane >> 4;
  const int i16 = lane & 15;
  uint16_t* Kw = reinterpret_cast<uint16_t*>(smem) + wave * L::wElems;
  uint16_t* Vw = Kw + L::kElems;
  // transposing V reads (A operand of O^T += V^T P^T), as in the prefill kernel
  const int tr_row = 4 * hq + (i16 >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (i16 & 3);

  // cur: the piece being reduced (same on every wave). ld: the piece of the
  // sub-block this wave has in flight (ld_pi its index, ld_sb its first key).
  long long cur_pos = start;
  Piece cur = locate(a, start, end - start, lane);
  long long ld_pos = cur_pos;
  Piece ld = cur;
  int ld_pi = 0, ld_sb = cur.k0 + wave * kSub;
  bool ld_ok = ld_sb < cur.k1 || next_sub(a, ld, ld_pos, end, ld_sb, ld_pi, wave);
  if (ld_sb >= ld.k1) ld_ok = false;

  u32x4 kr[L::kLoads], vr[L::kLoads];
  if (ld_ok) load_sub<D>(a, ld, ld_sb, lane, kr, vr);
  // Q^T (B operand of S^T = K Q^T): head l32, d = hq * D/2 + 8 st.
  bf16x8 qf[D / 16];
  float* comb = reinterpret_cast<float*>(smem);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (int pi = 0;; ++pi) {
    {
      const int head = head_of<ROUTED>(a, cur.b, cur.gam, min(l32, a.R - 1));
      const uint16_t* qrow = a.q + ((size_t)cur.b * a.h + head) * D + hq * (D / 2);
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 8 * st);
        if (l32 >= a.R) x = bf16x8{};
        qf[st] = x;
      }
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const int k1 = cur.k1;

    // This wave's sub-blocks of the piece: keys k0 + 32*wave + 128*i.
    while (ld_ok && ld_pi == pi) {
#pragma unroll
      for (int i = 0; i < L::kLoads; ++i) {
        const int cidx = lane + 64 * i;
        const int row = cidx / L::kCPR, col = (cidx % L::kCPR) * 8;
        *reinterpret_cast<u32x4*>(Kw + row * L::kPitch + col) = kr[i];
        *reinterpret_cast<u32x4*>(Vw + row * L::vPitch + col) = vr[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int cur_sb = ld_sb;
      ld_ok = next_sub(a, ld, ld_pos, end, ld_sb, ld_pi, wave);
      if (ld_ok) load_sub<D>(a, ld, ld_sb, lane, kr, vr);

      // S^T[key][head]: lane holds keys cur_sb + 8(i/4) + 4hq + i%4 of head l32.
      f32x16 s = f32x16{};
      {
        const uint16_t* krow = Kw + l32 * L::kPitch + hq * (D / 2);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(krow + 8 * st), qf[st], s);
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (cur_sb + 8 * (i >> 2) + 4 * hq + (i & 3) >= k1) s[i] = -INFINITY;
        mloc = fmaxf(mloc, s[i]);
      }
      const float m_cand = fmaxf(mloc, __shfl_xor(mloc, 32)) * a.c;
      // Raise the reference max only when a score exceeds it by more than
      // 2^kRescale; otherwise keep it (probabilities stay below 2^kRescale).
      if (__any(m_cand > m_run + kRescale)) {
        const float m_new = fmaxf(m_run, m_cand);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      }
      // P^T as bf16 B operands: element j of step u is key 16u + 8(j/4) + 4hq + j%4.
      bf16x8 pf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(fmaf(s[8 * u + j], a.c, -m_run));
        pf[u] = pack_bf16x8(pv);
        const bf16x2* pp = reinterpret_cast<const bf16x2*>(&pf[u]);
#pragma unroll
        for (int j = 0; j < 4; ++j) l_run = __builtin_amdgcn_fdot2_f32_bf16(pp[j], ones, l_run, false);
      }
      // O^T += V^T P^T, V^T by two transposing reads per step and 32-wide d block.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint16_t* p0 = Vw + (16 * u + tr_row) * L::vPitch + tr_col;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = mfma32x32x16(lds_read_tr_pair(p0 + 32 * db, p0 + 8 * L::vPitch + 32 * db), pf[u], o[db]);
      }
      __builtin_amdgcn_wave_barrier();
    }

    // Combine the 4 waves through LDS, one head block at a time; write the
    // output rows when the piece is the whole stream, else a partial in slot 0
    // (the share's first piece) or 1 (its last).
    const bool whole = cur.k0 == 0 && k1 == cur.len;
    const int slot = pi == 0 ? 0 : 1;
    {
      const float lsum = l_run + __shfl_xor(l_run, 32);
      __syncthreads();  // LDS is free: the staging buffers are consumed
      float* w = comb + (wave * 32 + l32) * kCP;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4*>(w + 32 * db + 8 * i4 + 4 * hq) =
              f32x4{o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]};
      if (hq == 0) {
        w[D] = m_run;
        w[D + 1] = lsum;
      }
      __syncthreads();
      for (int x = tid; x < 32 * D; x += kThreads) {
        const int e = x / D;
        const int d = x - e * D;
        if (e >= a.R) break;  // x only grows
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, comb[(wv * 32 + e) * kCP + D]);
        float acc = 0.0f, den = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
          const float* src = comb + (wv * 32 + e) * kCP;
          const float mw = src[D];
          const float sc = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
          acc += sc * src[d];
          den += sc * src[D + 1];
        }
        if (whole) {
          const int head = head_of<ROUTED>(a, cur.b, cur.gam, e);
          const size_t off = ((size_t)cur.b * a.h + head) * D + d;
          float y = acc / den;
          if (ROUTED) y *= a.gate[((size_t)cur.b * a.g + cur.gam) * a.R + e];
          if (a.out_bf16)
            static_cast<uint16_t*>(a.out)[off] = static_cast<uint16_t>(pack_bf16x2(y, 0.0f) & 0xffffu);
          else
            static_cast<float*>(a.out)[off] = y;
        } else {
          const size_t prow = ((size_t)unit * 2 + slot) * a.R + e;
          a.part_acc[prow * D + d] = acc;
          if (d == 0) {
            a.part_ml[prow * 2 + 0] = M;
            a.part_ml[prow * 2 + 1] = den;
          }
        }
      }
    }
    Piece n;
    if (!next_piece(a, cur, cur_pos, end, n)) break;
    cur = n;
    __syncthreads();  // combine reads done before the staging buffers are rewritten
  }
}

// One wave per (sequence, head): a stream cut over several shares has its
// pieces merged by log-sum-exp; a sequence with no cached keys gets a zero
// row, and so does (routed) a head the router did not keep. Streams that lie
// in one share were written by decode_kernel.
template <int D, bool ROUTED>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(KArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);  // b * h + head
  if (row >= a.B * a.h) return;
  const int b = row / a.h;
  const int head = row - b * a.h;
  const int gam = head / a.r;
  int e = head - gam * a.r;  // the head's row in its group
  // Columns per lane: D/64, or one for D = 32, where lanes 32-63 read column
  // D-1 (in bounds) and write nothing.
  constexpr int EPL = D >= 64 ? D / 64 : 1;
  const bool col_ok = D >= 64 || lane < D;
  const int col = D >= 64 ? lane : min(lane, D - 1);
  if (ROUTED) {
    const int32_t* sel = a.idx + ((size_t)b * a.g + gam) * a.R;
    e = -1;
    for (int j = 0; j < a.R; ++j)
      if (sel[j] == head) e = j;
    if (e < 0) {
#pragma unroll
      for (int x = 0; x < EPL; ++x) {
        const size_t off = (size_t)row * D + col + 64 * x;
        if (!col_ok) break;
        if (a.out_bf16)
          static_cast<uint16_t*>(a.out)[off] = 0;
        else
          static_cast<float*>(a.out)[off] = 0.0f;
      }
      return;
    }
  }
  // Global position of the stream, g * (keys of sequences before b) + gam *
  // len, and the total, from one pass over lens (len is read first, so both
  // loads share one memory latency).
  const int len = seq_len(a, b);
  long long before = 0, total = 0;
  for (int bb = lane; bb < a.B; bb += 64) {
    const long long l = seq_len(a, bb);
    total += l;
    before += bb < b ? l : 0;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    before += __shfl_xor(before, o);
    total += __shfl_xor(total, o);
  }
  if (len == 0) {
#pragma unroll
    for (int x = 0; x < EPL; ++x) {
      const size_t off = (size_t)row * D + col + 64 * x;
      if (!col_ok) break;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[off] = 0;
      else
        static_cast<float*>(a.out)[off] = 0.0f;
    }
    return;
  }
  total *= a.g;
  const long long share = share_of(total, a.n_units);
  const long long start = before * a.g + (long long)gam * len;
  const int u0 = (int)(start / share);
  const int u1 = (int)((start + len - 1) / share);
  if (u0 == u1) return;
  // The first piece sits in slot 1 of unit u0 when that share began in an
  // earlier stream, else in slot 0; every later piece is its unit's first.
  const int slot0 = (long long)u0 * share < start ? 1 : 0;
  const int n = u1 - u0 + 1;
  auto prow_of = [&](int j) {
    return ((size_t)(u0 + j) * 2 + (j == 0 ? slot0 : 0)) * a.R + e;
  };
  // Pieces in rounds of 64: lane j holds piece j's (max, sum). The
  // accumulator rows are read kBatch pieces at a time, every load of a batch
  // issued before the first is used (a batch past the last piece re-reads the
  // last one and weighs it 0), so a round costs a few memory latencies, not
  // one per piece. The first batch is in flight while the max is reduced.
  constexpr int kBatch = 16;
  float M = -INFINITY, den = 0.0f;
  float acc[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) acc[x] = 0.0f;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int nj = min(64, n - j0);
    // Branch-free loads (lanes past the last piece re-read it), so the first
    // batch issues in the same block as the (max, sum) loads.
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + prow_of(j0 + min(lane, nj - 1)) * 2);
    float v[kBatch][EPL];
    auto fetch = [&](int jb) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const size_t pr = prow_of(j0 + min(jb + u, nj - 1));
#pragma unroll
        for (int x = 0; x < EPL; ++x) v[u][x] = a.part_acc[pr * D + col + 64 * x];
      }
    };
    auto consume = [&](int jb, float scl) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float sc = __shfl(scl, min(jb + u, 63));  // 0 past the last piece
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc[x] += sc * v[u][x];
      }
    };
    fetch(0);
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of the reduction
    const float mj = lane < nj ? ml.x : -INFINITY;
    const float lj = lane < nj ? ml.y : 0.0f;
    float Mr = mj;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Mr = fmaxf(Mr, __shfl_xor(Mr, o));
    const float Mn = fmaxf(M, Mr);
    const float alpha = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
    float dj = lane < nj ? fast_exp2(mj - Mn) * lj : 0.0f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) dj += __shfl_xor(dj, o);
    den = den * alpha + dj;
#pragma unroll
    for (int x = 0; x < EPL; ++x) acc[x] *= alpha;
    const float scl = lane < nj ? fast_exp2(mj - Mn) : 0.0f;  // lane j: piece j's weight
    consume(0, scl);
    for (int jb = kBatch; jb < nj; jb += kBatch) {
      fetch(jb);
      consume(jb, scl);
    }
    M = Mn;
  }
  const float inv = (ROUTED ? a.gate[((size_t)b * a.g + gam) * a.R + e] : 1.0f) / den;
#pragma unroll
  for (int x = 0; x < EPL; ++x) {
    if (!col_ok) break;
    const float y = acc[x] * inv;
    const size_t off = (size_t)row * D + col + 64 * x;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[off] = static_cast<uint16_t>(pack_bf16x2(y, 0.0f) & 0xffffu);
    else
      static_cast<float*>(a.out)[off] = y;
  }
}

// 17-32 heads per group run on the 32-column kernel, except at D = 16, whose
// 16-row O^T fits the 16x16x32 kernel with two head blocks in few registers.
template <int D>
const void* kernel_for_hb(int hb) {
  if (hb == 1) return reinterpret_cast<const void*>(&decode_kernel<D, 1, false>);
  if (hb == 2) {
    if constexpr (D == 16) return reinterpret_cast<const void*>(&decode_kernel<D, 2, false>);
    else return reinterpret_cast<const void*>(&decode32_kernel<D, false>);
  }
  if (hb <= 4) return reinterpret_cast<const void*>(&decode_kernel<D, 4, false>);
  return nullptr;
}

const void* decode_kernel_for(int d, int hb) {
  if (d == 16) return kernel_for_hb<16>(hb);
  if (d == 32) return kernel_for_hb<32>(hb);
  if (d == 64) return kernel_for_hb<64>(hb);
  if (d == 128) return kernel_for_hb<128>(hb);
  return nullptr;
}

template <int D, bool ROUTED>
hipError_t launch_dr(const KArgs& a, const dim3 grid, bool in_f32, hipStream_t stream) {
  const dim3 block(kThreads);
  const int hb = div_up(a.R, 16);
  if (hb > 4) return hipErrorInvalidValue;
  if (in_f32) {
    hipLaunchKernelGGL((decode_f32_kernel<D, ROUTED>), dim3(grid.x, hb), block, 0, stream, a);
  } else if (hb == 1) {
    hipLaunchKernelGGL((decode_kernel<D, 1, ROUTED>), grid, block, 0, stream, a);
  } else if (hb == 2) {
    if constexpr (D == 16)
      hipLaunchKernelGGL((decode_kernel<D, 2, ROUTED>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode32_kernel<D, ROUTED>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, 4, ROUTED>), grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, ROUTED>), dim3(div_up(a.B * a.h, kWaves)), block, 0,
                     stream, a);
  return hipGetLastError();
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
  a.idx = p.idx;
  a.gate = p.gate;
  a.B = p.B;
  a.h = p.h;
  a.g = p.g;
  a.r = p.h / p.g;
  a.R = p.idx ? p.top_k : a.r;
  a.T_max = p.T_max;
  a.n_units = p.n_units;
  a.c = p.scale * kLog2e;
  a.out_bf16 = p.out_bf16;
  const dim3 grid(p.n_units);
  return p.idx ? launch_dr<D, true>(a, grid, p.in_f32, stream) : launch_dr<D, false>(a, grid, p.in_f32, stream);
}

}  // namespace

bool decode_supports(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int decode_units(int h, int g, int d) {
  if (const char* env = std::getenv("GQA_DECODE_UNITS")) {
    const int u = std::atoi(env);
    if (u > 0) return u;
  }
  // One workgroup per resident workgroup slot of the chip: every share is
  // streamed concurrently and they all end together.
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
  return n_cu * per_cu;
}

// Device scratch of the allocation-free decode entry point: the split
// partials live in this array instead of a caller's workspace. Each device the
// library runs on holds its own copy until the process ends. Host code must
// never pass the array's name to a kernel or a copy (on the host it is only a
// stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.d) {
    case 16: return launch_d<16>(p, stream);
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
