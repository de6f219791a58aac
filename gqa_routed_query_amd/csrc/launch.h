// Host-side launch interface between the C ABI (api.hip) and the kernels.
// Every function here enqueues work on `stream` and returns the launch status;
// arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// One attention row is one (token, query head) pair of one (batch, KV group).
// Rows are ordered token-major: row rho of group (b, gamma) is token rho / R,
// slot rho % R. Dense GQA uses R = h/g and slot j is head gamma*(h/g) + j.
// Routed GQE uses R = top_k and slot j is head idx[b, t, gamma, j], with the
// output row multiplied by gate[b, t, gamma, j].
struct AttnParams {
  const void* q;        // [B, h, T, d]
  const void* k;        // [B, g, T, d]
  const void* v;        // [B, g, T, d]
  void* out;            // [B, h, T, d]
  const int32_t* idx;   // routed only: [B, T, g, R] global head ids, else null
  const float* gate;    // routed only: [B, T, g, R], else null
  // Routed bf16 launches only (null: idx and gate are inputs): router logits
  // [B, T, h]; the kernel selects the kept heads itself and writes idx and gate.
  const float* logits;
  int B, h, g, T, d;
  int R;                // rows per token
  float scale;          // > 0
  int causal;           // 0 or 1
  int out_bf16;         // 1: bf16 output, 0: fp32 output
  int in_bf16;          // fp32-arithmetic kernel only: 1 when q, k, v are bf16 (d 16 or 32)
  int zero_unselected;  // routed only: write zeros to the rows of unselected heads
  // Layout overrides (bf16 kernel only; 0 keeps the [B,h,T,d] / [B,g,T,d] default):
  int out_slots;        // routed: row (t, gam, j) goes to output slot gam*R + j, ungated
  size_t q_b;           // elements between batches of q
  size_t kv_b;          // elements between batches of k and v
  size_t o_b, o_h, o_t; // output strides: batch, head (or slot), token
  // Shared head run in the same launch (bf16 kernel only; null: none): one
  // query row per token, q_shared / out_shared [B, T, d], on KV head shared_kv.
  const void* q_shared;
  void* out_shared;
  int shared_kv;
  // Routed causal launches (bf16 kernel only; null: none): workspace of at
  // least attn_bf16_split_ws_bytes(...) bytes for the partial results of
  // key-split row tiles.
  void* split_ws;
};

struct RouterParams {
  const float* logits;  // [B, T, h]
  int32_t* idx;         // [B, T, g, k]
  float* gate;          // [B, T, g, k]
  int B, T, h, g, k;
};

struct WsumParams {
  const void* concat;   // [n, k, d] rows of the kept experts (out dtype)
  const float* gate;    // [n, k]
  void* wsum;           // [n, d]
  long long n;          // (batch, token, group) triples
  int k, d, bf16;
};

struct RouterProjParams {
  const void* x;        // [n_tok, d_model] bf16
  const void* w;        // [h, d_model] bf16
  float* logits;        // [n_tok, h] or null
  int32_t* idx;         // [n_tok, g, k]
  float* gate;          // [n_tok, g, k]
  int n_tok, d_model, h, g, k;
};

struct DecodeParams {
  const void* q;        // [B, h, d] bf16, or fp32 with in_f32
  const void* k_cache;  // [B, g, T_max, d], dtype of q
  const void* v_cache;  // [B, g, T_max, d], dtype of q
  const int32_t* lens;  // [B] on the device
  void* out;            // [B, h, d]
  float* part_acc;      // [n_units, 2, h/g, d] fp32 workspace
  float* part_ml;       // [n_units, 2, h/g, 2] fp32 workspace
  const int32_t* idx;   // routed: [B, g, top_k] kept heads (router output), else null
  const float* gate;    // routed: [B, g, top_k] their gates, else null
  int top_k;            // routed: kept heads per group
  int B, h, g, T_max, d;
  int n_units;          // waves that share the key range
  float scale;
  int out_bf16;
  int in_f32;           // q and the caches are fp32 (fp32-operand kernel)
};

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);
hipError_t launch_router(const RouterParams& p, hipStream_t stream);
hipError_t launch_router_proj(const RouterProjParams& p, hipStream_t stream);
hipError_t launch_wsum(const WsumParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// Bytes of the static device scratch that the allocation-free decode uses for
// its split partials, and its address on the current device (looked up with
// hipGetSymbolAddress on the first call per device, then cached).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);
// Peak microbenchmarks: read `bytes` (a multiple of 16) of buf once and XOR
// all 32-bit words into *x_out; run the MFMA-only loop, add the sum of its
// accumulators to *sum_out and report the flops it performs.
hipError_t launch_peak_hbm_read(const void* buf, size_t bytes, unsigned* x_out, hipStream_t stream);
hipError_t launch_peak_mfma_bf16(const void* operands, int iters, float* sum_out, double* flops, hipStream_t stream);
// The attention tile loop on register operands (q, k, v of one 32x128 tile);
// writes the normalised output of one wave and reports the flops.
hipError_t launch_peak_attn_tile(const void* qkv, int iters, float scale, float* out, double* flops,
                                 hipStream_t stream);

// Head dims with a bf16 MFMA prefill kernel / an fp32-arithmetic kernel (fp32
// inputs at every listed d, bf16 inputs at d 16 and 32) / a decode kernel.
bool attn_bf16_supports(int d);
// Workspace bytes a routed causal bf16 launch of this shape may use for key splits
// (0 when it would split nothing); R is the number of rows per token.
size_t attn_bf16_split_ws_bytes(int B, int g, int T, int d, int R, int causal);
bool attn_f32_supports(int d);
bool decode_supports(int d);
bool router_proj_supports(int d_model, int h);

// Waves that share a decode call's key range (honours GQA_DECODE_UNITS).
int decode_units(int h, int g, int d);

}  // namespace gqa
