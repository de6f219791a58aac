// C ABI of libgqa: argument checks, dispatch and launches on the caller's
// stream. Declarations and the contract of each entry point are in gqa.h.
#include "gqa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

gqa_status fail(gqa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int dt) { return dt == GQA_F32 || dt == GQA_BF16; }

// Checks shared by the prefill-shaped entry points.
gqa_status check_prefill_shape(const void* q, const void* k, const void* v, const void* out,
                               int B, int h, int g, int T, int d, int in_dt, int out_dt,
                               float scale, int causal) {
  if (B < 0 || T < 0) return fail(GQA_ERR_INVALID_ARG, "B=%d and T=%d must be >= 0", B, T);
  if (h < 1 || g < 1) return fail(GQA_ERR_INVALID_ARG, "h=%d and g=%d must be >= 1", h, g);
  if (h % g != 0) return fail(GQA_ERR_INVALID_ARG, "g=%d must divide h=%d", g, h);
  if (d < 1) return fail(GQA_ERR_INVALID_ARG, "d=%d must be >= 1", d);
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt))
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype (in %d, out %d)", in_dt, out_dt);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(GQA_ERR_INVALID_ARG, "scale=%g must be finite and > 0", (double)scale);
  if (causal != 0 && causal != 1) return fail(GQA_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
  if ((long long)h * T >= (1ll << 31))
    return fail(GQA_ERR_INVALID_ARG, "h*T=%lld exceeds the 2^31 row limit", (long long)h * T);
  if (B == 0 || T == 0) return GQA_OK;
  if (!q || !k || !v || !out) return fail(GQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(GQA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (in_dt == GQA_BF16 && !gqa::attn_bf16_supports(d) && d != 16 && d != 32)
    return fail(GQA_ERR_UNSUPPORTED, "bf16 prefill supports d in {16, 32, 64, 128}, got %d", d);
  if (in_dt == GQA_F32 && !gqa::attn_f32_supports(d))
    return fail(GQA_ERR_UNSUPPORTED, "fp32 prefill supports d in {16, 32, 64, 128}, got %d", d);
  return GQA_OK;
}

// bf16 inputs run on the MFMA kernel where its tiles fit the head dim (64,
// 128), else (16, 32) on the fp32-arithmetic kernel; fp32 inputs always on
// the latter.
hipError_t launch_prefill(gqa::AttnParams& p, gqa_dtype in_dtype, hipStream_t st) {
  if (in_dtype == GQA_BF16 && gqa::attn_bf16_supports(p.d)) return gqa::launch_attn_bf16(p, st);
  p.in_bf16 = in_dtype == GQA_BF16;
  return gqa::launch_attn_f32(p, st);
}

gqa_status check_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return fail(GQA_ERR_NO_DEVICE, "no HIP device visible");
  }
  return GQA_OK;
}

gqa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GQA_OK;
  return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct DecodeLayout {
  int n_units;
  size_t acc_bytes, ml_bytes, total;
};

// Two partials (r heads each) per wave of the decode grid.
DecodeLayout decode_layout(int h, int g, int d) {
  DecodeLayout L{};
  L.n_units = gqa::decode_units(h, g, d);
  const size_t rows = (size_t)L.n_units * 2 * (h / g);
  L.acc_bytes = (rows * d * sizeof(float) + 255) & ~(size_t)255;
  L.ml_bytes = rows * 2 * sizeof(float);
  L.total = L.acc_bytes + L.ml_bytes;
  return L;
}

// Argument checks shared by the decode entry points (no kernel launch); on
// success fills p (everything but the routing fields). B == 0 is accepted
// before pointers are looked at. With own_scratch the partials go to the
// library's static device scratch (set by the caller) instead of a workspace,
// and the shape must fit it.
gqa_status prepare_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens,
                          void* out, int B, int h, int g, int T_max, int d, gqa_dtype in_dtype,
                          gqa_dtype out_dtype, float scale, void* workspace, size_t workspace_bytes,
                          gqa::DecodeParams& p, bool own_scratch = false) {
  if (B < 0 || T_max < 0) return fail(GQA_ERR_INVALID_ARG, "B=%d and T_max=%d must be >= 0", B, T_max);
  if (h < 1 || g < 1) return fail(GQA_ERR_INVALID_ARG, "h=%d and g=%d must be >= 1", h, g);
  if (h % g != 0) return fail(GQA_ERR_INVALID_ARG, "g=%d must divide h=%d", g, h);
  if (d < 1) return fail(GQA_ERR_INVALID_ARG, "d=%d must be >= 1", d);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype (in %d, out %d)", in_dtype, out_dtype);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(GQA_ERR_INVALID_ARG, "scale=%g must be finite and > 0", (double)scale);
  if ((long long)g * T_max >= (1ll << 31))
    return fail(GQA_ERR_INVALID_ARG, "g*T_max=%lld exceeds the 2^31 row limit", (long long)g * T_max);
  if (B == 0) return GQA_OK;
  if (!q || !out || !lens) return fail(GQA_ERR_INVALID_ARG, "null q, out or lens pointer");
  if (T_max > 0 && (!k_cache || !v_cache)) return fail(GQA_ERR_INVALID_ARG, "null cache pointer");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(GQA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!gqa::decode_supports(d)) return fail(GQA_ERR_UNSUPPORTED, "decode supports d in {16, 32, 64, 128}, got %d", d);
  if (h / g > 64) return fail(GQA_ERR_UNSUPPORTED, "decode supports h/g <= 64, got %d", h / g);
  const DecodeLayout L = decode_layout(h, g, d);
  if (own_scratch) {
    if (L.total > gqa::kDecodeScratchBytes)
      return fail(GQA_ERR_WORKSPACE, "this shape needs %zu bytes of split partials; the static scratch holds %zu",
                  L.total, gqa::kDecodeScratchBytes);
  } else {
    if (workspace_bytes < L.total)
      return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, L.total);
    if (!workspace || !aligned16(workspace))
      return fail(GQA_ERR_INVALID_ARG, "workspace must be a 16-byte aligned device pointer");
  }
  p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.lens = lens; p.out = out;
  p.B = B; p.h = h; p.g = g; p.T_max = T_max; p.d = d;
  p.n_units = L.n_units;
  p.part_acc = static_cast<float*>(workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.acc_bytes);
  p.scale = scale;
  p.out_bf16 = out_dtype == GQA_BF16;
  p.in_f32 = in_dtype == GQA_F32;
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_abi_version(void) { return 2; }

const char* gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_WORKSPACE: return "workspace too small";
    case GQA_ERR_NO_DEVICE: return "no HIP device";
    case GQA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* gqa_last_error(void) { return g_last_error; }

uint64_t gqa_kv_cache_bytes(int B, int n_kv, int T, int d, gqa_dtype dtype) {
  if (B < 0 || n_kv < 0 || T < 0 || d < 0 || !valid_dtype(dtype)) return 0;
  const uint64_t elt = dtype == GQA_BF16 ? 2 : 4;
  return 2ull * (uint64_t)n_kv * (uint64_t)d * (uint64_t)T * elt * (uint64_t)B;
}

gqa_status gqa_prefill(const void* q, const void* k, const void* v, void* out, int B, int h, int g,
                       int T, int d, gqa_dtype in_dtype, gqa_dtype out_dtype, float scale, int causal,
                       void* stream) {
  g_last_error[0] = '\0';
  gqa_status s = check_prefill_shape(q, k, v, out, B, h, g, T, d, in_dtype, out_dtype, scale, causal);
  if (s != GQA_OK || B == 0 || T == 0) return s;
  if ((s = check_device()) != GQA_OK) return s;
  gqa::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out;
  p.B = B; p.h = h; p.g = g; p.T = T; p.d = d;
  p.R = h / g;
  p.scale = scale;
  p.causal = causal;
  p.out_bf16 = out_dtype == GQA_BF16;
  auto st = static_cast<hipStream_t>(stream);
  return hip_status(launch_prefill(p, in_dtype, st), "gqa_prefill launch");
}

size_t gqa_decode_workspace_bytes(int B, int h, int g, int T_max, int d) {
  if (B < 0 || h < 1 || g < 1 || h % g || T_max < 0 || d <= 0) return 0;
  return decode_layout(h, g, d).total;
}

gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens,
                      void* out, int B, int h, int g, int T_max, int d, gqa_dtype in_dtype,
                      gqa_dtype out_dtype, float scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_last_error[0] = '\0';
  gqa::DecodeParams p{};
  gqa_status s = prepare_decode(q, k_cache, v_cache, lens, out, B, h, g, T_max, d, in_dtype, out_dtype,
                                scale, workspace, workspace_bytes, p);
  if (s != GQA_OK || B == 0) return s;
  if ((s = check_device()) != GQA_OK) return s;
  return hip_status(gqa::launch_decode(p, static_cast<hipStream_t>(stream)), "gqa_decode launch");
}

gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens,
                              void* out, int B, int h, int g, int T_max, int d, gqa_dtype in_dtype,
                              gqa_dtype out_dtype, float scale, void* stream) {
  g_last_error[0] = '\0';
  gqa::DecodeParams p{};
  gqa_status s = prepare_decode(q, k_cache, v_cache, lens, out, B, h, g, T_max, d, in_dtype, out_dtype,
                                scale, nullptr, 0, p, /*own_scratch=*/true);
  if (s != GQA_OK || B == 0) return s;
  if ((s = check_device()) != GQA_OK) return s;
  void* scratch = nullptr;
  if ((s = hip_status(gqa::decode_scratch(&scratch), "gqa_decode_noalloc scratch lookup")) != GQA_OK) return s;
  const DecodeLayout L = decode_layout(h, g, d);
  p.part_acc = static_cast<float*>(scratch);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(scratch) + L.acc_bytes);
  return hip_status(gqa::launch_decode(p, static_cast<hipStream_t>(stream)), "gqa_decode_noalloc launch");
}

gqa_status gqe_routed_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* lens, const float* router_logits, int top_k, void* out,
                             int32_t* topk_idx, float* topk_gate, int B, int h, int g, int T_max,
                             int d, gqa_dtype in_dtype, gqa_dtype out_dtype, float scale,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  gqa::DecodeParams p{};
  gqa_status s = prepare_decode(q, k_cache, v_cache, lens, out, B, h, g, T_max, d, in_dtype, out_dtype,
                                scale, workspace, workspace_bytes, p);
  if (s != GQA_OK) return s;
  const int r = h / g;
  if (top_k < 1 || top_k > r) return fail(GQA_ERR_INVALID_ARG, "top_k=%d must be in [1, h/g=%d]", top_k, r);
  if (B == 0) return GQA_OK;
  if (!router_logits || !topk_idx || !topk_gate)
    return fail(GQA_ERR_INVALID_ARG, "null router_logits, topk_idx or topk_gate pointer");
  if ((s = check_device()) != GQA_OK) return s;
  auto st = static_cast<hipStream_t>(stream);
  gqa::RouterParams rp{router_logits, topk_idx, topk_gate, B, 1, h, g, top_k};
  if ((s = hip_status(gqa::launch_router(rp, st), "gqe decode router launch")) != GQA_OK) return s;
  p.idx = topk_idx;
  p.gate = topk_gate;
  p.top_k = top_k;
  return hip_status(gqa::launch_decode(p, st), "gqe routed decode launch");
}

gqa_status gqe_prefill_build(const void* q, const void* q_shared, const void* k, const void* v,
                             const float* router_logits, int top_k, int shared_kv, void* out_concat,
                             void* out_wsum, void* out_shared, int32_t* topk_idx, float* topk_gate,
                             int B, int h, int g, int T, int d, gqa_dtype in_dtype,
                             gqa_dtype out_dtype, float scale, int causal, void* stream) {
  g_last_error[0] = '\0';
  gqa_status s = check_prefill_shape(q, k, v, out_concat, B, h, g, T, d, in_dtype, out_dtype, scale, causal);
  if (s != GQA_OK) return s;
  const int r = h / g;
  if (top_k < 1 || top_k > r) return fail(GQA_ERR_INVALID_ARG, "top_k=%d must be in [1, h/g=%d]", top_k, r);
  if (shared_kv < 0 || shared_kv >= g) return fail(GQA_ERR_INVALID_ARG, "shared_kv=%d must be in [0, g=%d)", shared_kv, g);
  if (in_dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "the GQE output build takes bf16 inputs");
  if (!gqa::attn_bf16_supports(d)) return fail(GQA_ERR_UNSUPPORTED, "the GQE output build supports d in {64, 128}, got %d", d);
  if (r > 64) return fail(GQA_ERR_UNSUPPORTED, "routing supports h/g <= 64, got %d", r);
  if (B == 0 || T == 0) return GQA_OK;
  if (!q_shared || !router_logits || !out_wsum || !out_shared || !topk_idx || !topk_gate)
    return fail(GQA_ERR_INVALID_ARG, "null q_shared, router_logits, output, topk_idx or topk_gate pointer");
  if (!aligned16(q_shared) || !aligned16(out_wsum) || !aligned16(out_shared))
    return fail(GQA_ERR_INVALID_ARG, "q_shared and the outputs must be 16-byte aligned");
  if ((s = check_device()) != GQA_OK) return s;
  auto st = static_cast<hipStream_t>(stream);
  // 1. router: kept experts and gates per (token, group)
  gqa::RouterParams rp{router_logits, topk_idx, topk_gate, B, T, h, g, top_k};
  if ((s = hip_status(gqa::launch_router(rp, st), "gqe build router launch")) != GQA_OK) return s;
  // 2. kept experts' rows, ungated, into out_concat [B, T, g, k, d]
  gqa::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out_concat;
  p.idx = topk_idx;
  p.gate = topk_gate;
  p.B = B; p.h = h; p.g = g; p.T = T; p.d = d;
  p.R = top_k;
  p.scale = scale;
  p.causal = causal;
  p.out_bf16 = out_dtype == GQA_BF16;
  p.out_slots = 1;
  p.o_b = (size_t)T * g * top_k * d;
  p.o_h = d;
  p.o_t = (size_t)g * top_k * d;
  // 3. the shared head, one query per token on KV head shared_kv, as extra
  //    problems of the same launch (its row tiles are scheduled with the routed ones)
  p.q_shared = q_shared;
  p.out_shared = out_shared;
  p.shared_kv = shared_kv;
  if ((s = hip_status(gqa::launch_attn_bf16(p, st), "gqe build attention launch")) != GQA_OK) return s;
  // 4. the weighted-sum slot of every (token, group)
  gqa::WsumParams wp{out_concat, topk_gate, out_wsum, (long long)B * T * g, top_k, d, out_dtype == GQA_BF16};
  return hip_status(gqa::launch_wsum(wp, st), "gqe build weighted-sum launch");
}

gqa_status gqe_router(const void* x, const void* w_r, int top_k, float* logits, int32_t* topk_idx,
                      float* topk_gate, int n_tokens, int d_model, int h, int g, gqa_dtype in_dtype,
                      void* stream) {
  g_last_error[0] = '\0';
  if (n_tokens < 0 || d_model < 1) return fail(GQA_ERR_INVALID_ARG, "n_tokens=%d must be >= 0 and d_model=%d >= 1", n_tokens, d_model);
  if (h < 1 || g < 1) return fail(GQA_ERR_INVALID_ARG, "h=%d and g=%d must be >= 1", h, g);
  if (h % g != 0) return fail(GQA_ERR_INVALID_ARG, "g=%d must divide h=%d", g, h);
  const int r = h / g;
  if (top_k < 1 || top_k > r) return fail(GQA_ERR_INVALID_ARG, "top_k=%d must be in [1, h/g=%d]", top_k, r);
  if (!valid_dtype(in_dtype)) return fail(GQA_ERR_INVALID_ARG, "unknown dtype %d", in_dtype);
  if (in_dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "the router projection takes bf16 x and w_r");
  if (!gqa::router_proj_supports(d_model, h))
    return fail(GQA_ERR_UNSUPPORTED, "router projection supports h <= 64 and d_model a multiple of 128, got h=%d d_model=%d", h, d_model);
  if (n_tokens == 0) return GQA_OK;
  if (!x || !w_r || !topk_idx || !topk_gate)
    return fail(GQA_ERR_INVALID_ARG, "null x, w_r, topk_idx or topk_gate pointer");
  if (!aligned16(x) || !aligned16(w_r)) return fail(GQA_ERR_INVALID_ARG, "x and w_r must be 16-byte aligned");
  gqa_status s = check_device();
  if (s != GQA_OK) return s;
  gqa::RouterProjParams p{x, w_r, logits, topk_idx, topk_gate, n_tokens, d_model, h, g, top_k};
  return hip_status(gqa::launch_router_proj(p, static_cast<hipStream_t>(stream)), "gqe_router launch");
}

size_t gqe_workspace_bytes(int B, int h, int g, int T, int d, int top_k) {
  if (B <= 0 || T <= 0 || h <= 0 || g <= 0 || h % g != 0 || top_k < 1 || top_k > h / g) return 0;
  if (!gqa::attn_bf16_supports(d)) return 0;
  return gqa::attn_bf16_split_ws_bytes(B, g, T, d, top_k, 1);
}

gqa_status gqe_routed_prefill(const void* q, const void* k, const void* v, const float* router_logits,
                              int top_k, void* out, int32_t* topk_idx, float* topk_gate, int B, int h,
                              int g, int T, int d, gqa_dtype in_dtype, gqa_dtype out_dtype, float scale,
                              int causal, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  gqa_status s = check_prefill_shape(q, k, v, out, B, h, g, T, d, in_dtype, out_dtype, scale, causal);
  if (s != GQA_OK) return s;
  const int r = h / g;
  if (top_k < 1 || top_k > r) return fail(GQA_ERR_INVALID_ARG, "top_k=%d must be in [1, h/g=%d]", top_k, r);
  if (r > 64) return fail(GQA_ERR_UNSUPPORTED, "routing supports h/g <= 64, got %d", r);
  if (B == 0 || T == 0) return GQA_OK;
  if (!router_logits || !topk_idx || !topk_gate)
    return fail(GQA_ERR_INVALID_ARG, "null router_logits, topk_idx or topk_gate pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if ((s = check_device()) != GQA_OK) return s;
  // Key splitting (bf16 causal launches only) needs the workspace.
  const size_t need = in_dtype == GQA_BF16 && gqa::attn_bf16_supports(d)
                          ? gqa::attn_bf16_split_ws_bytes(B, g, T, d, top_k, causal) : 0;
  if (workspace && workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  auto st = static_cast<hipStream_t>(stream);
  // The bf16 attention kernel selects the kept heads itself (one launch less);
  // the fp32-arithmetic kernel reads them from the router kernel.
  const bool select_in_kernel = in_dtype == GQA_BF16 && gqa::attn_bf16_supports(d);
  if (!select_in_kernel) {
    gqa::RouterParams rp{router_logits, topk_idx, topk_gate, B, T, h, g, top_k};
    if ((s = hip_status(gqa::launch_router(rp, st), "gqe router launch")) != GQA_OK) return s;
  }
  gqa::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.out = out;
  p.idx = topk_idx;
  p.gate = topk_gate;
  p.logits = select_in_kernel ? router_logits : nullptr;
  p.B = B; p.h = h; p.g = g; p.T = T; p.d = d;
  p.R = top_k;
  p.scale = scale;
  p.causal = causal;
  p.out_bf16 = out_dtype == GQA_BF16;
  p.zero_unselected = 1;
  p.split_ws = need > 0 ? workspace : nullptr;
  return hip_status(launch_prefill(p, in_dtype, st), "gqe routed attention launch");
}

gqa_status gqa_peak_hbm_read(const void* buf, size_t bytes, uint32_t* xor_out, void* stream) {
  g_last_error[0] = '\0';
  if (bytes % 16 != 0) return fail(GQA_ERR_INVALID_ARG, "bytes=%zu must be a multiple of 16", bytes);
  if (bytes == 0) return GQA_OK;
  if (!buf || !xor_out) return fail(GQA_ERR_INVALID_ARG, "null buffer or result pointer");
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(xor_out) & 3u))
    return fail(GQA_ERR_INVALID_ARG, "buf must be 16-byte and xor_out 4-byte aligned");
  gqa_status s = check_device();
  if (s != GQA_OK) return s;
  return hip_status(gqa::launch_peak_hbm_read(buf, bytes, xor_out, static_cast<hipStream_t>(stream)),
                    "gqa_peak_hbm_read launch");
}

gqa_status gqa_peak_mfma_bf16(const void* operands, int iters, float* sum_out, double* flops, void* stream) {
  g_last_error[0] = '\0';
  if (iters < 1) return fail(GQA_ERR_INVALID_ARG, "iters=%d must be >= 1", iters);
  if (!operands || !sum_out || !flops) return fail(GQA_ERR_INVALID_ARG, "null operands, sum or flops pointer");
  if (!aligned16(operands) || (reinterpret_cast<uintptr_t>(sum_out) & 3u))
    return fail(GQA_ERR_INVALID_ARG, "operands must be 16-byte and sum_out 4-byte aligned");
  gqa_status s = check_device();
  if (s != GQA_OK) return s;
  return hip_status(gqa::launch_peak_mfma_bf16(operands, iters, sum_out, flops, static_cast<hipStream_t>(stream)),
                    "gqa_peak_mfma_bf16 launch");
}

gqa_status gqa_peak_attn_tile(const void* qkv, int iters, float scale, float* out, double* flops, void* stream) {
  g_last_error[0] = '\0';
  if (iters < 1) return fail(GQA_ERR_INVALID_ARG, "iters=%d must be >= 1", iters);
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(GQA_ERR_INVALID_ARG, "scale=%g must be finite and > 0", (double)scale);
  if (!qkv || !out || !flops) return fail(GQA_ERR_INVALID_ARG, "null qkv, out or flops pointer");
  if (!aligned16(qkv) || (reinterpret_cast<uintptr_t>(out) & 3u))
    return fail(GQA_ERR_INVALID_ARG, "qkv must be 16-byte and out 4-byte aligned");
  gqa_status s = check_device();
  if (s != GQA_OK) return s;
  return hip_status(gqa::launch_peak_attn_tile(qkv, iters, scale, out, flops, static_cast<hipStream_t>(stream)),
                    "gqa_peak_attn_tile launch");
}

}  // extern "C"
