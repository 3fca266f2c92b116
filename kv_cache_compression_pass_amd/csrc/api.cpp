// C ABI of libkvc: argument validation, workspace sizing, status reporting and dispatch to the
// kernel launchers.  Every argument error is detected here, before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"
#include "kvc.h"

namespace kvc {

namespace {

thread_local std::string g_last_error;

kvc_status fail(kvc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvc_status ok() {
  g_last_error.clear();
  return KVC_OK;
}

kvc_status hip_fail(hipError_t e, const char* where) {
  return fail(KVC_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kMaxRidgePairs = 8192;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validate and convert a layer descriptor.  more_queries: Nq > N is allowed when the layer
// is not causal (query rows that see every key; used by the ridge fit's training queries).
kvc_status make_layer(const kvc_layer_desc* d, Layer* L, bool more_queries = false) {
  if (!d) return fail(KVC_ERR_INVALID_ARG, "desc is NULL");
  if (d->reserved != 0) return fail(KVC_ERR_INVALID_ARG, "desc.reserved must be 0");
  if (d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(KVC_ERR_INVALID_ARG, "head counts must be >= 1 (H_q=%d, H_kv=%d)", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(KVC_ERR_INVALID_ARG, "H_q %% H_kv != 0 (H_q=%d, H_kv=%d)", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads / d->n_kv_heads > 16)
    return fail(KVC_ERR_UNSUPPORTED, "query heads per KV head > 16");
  if (d->n_kv_heads > 256) return fail(KVC_ERR_UNSUPPORTED, "H_kv > 256");
  if (d->head_dim <= 0) return fail(KVC_ERR_INVALID_ARG, "head_dim must be > 0");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVC_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", d->head_dim);
  if (d->causal != 0 && d->causal != 1) return fail(KVC_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (d->n_keys < 1 || d->n_queries < 1)
    return fail(KVC_ERR_INVALID_ARG, "N and Nq must be >= 1 (N=%lld, Nq=%lld)", (long long)d->n_keys, (long long)d->n_queries);
  if (d->n_queries > d->n_keys && !(more_queries && d->causal == 0))
    return fail(KVC_ERR_INVALID_ARG, "Nq > N (Nq=%lld, N=%lld)", (long long)d->n_queries, (long long)d->n_keys);
  if (d->n_queries >= (int64_t(1) << 29)) return fail(KVC_ERR_UNSUPPORTED, "Nq >= 2^29");
  if (d->n_keys >= (int64_t(1) << 29)) return fail(KVC_ERR_UNSUPPORTED, "N >= 2^29");
  if (!std::isfinite(d->softmax_scale) || d->softmax_scale < 0.f)
    return fail(KVC_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  L->hq = d->n_q_heads;
  L->hkv = d->n_kv_heads;
  L->d = d->head_dim;
  L->G = d->n_q_heads / d->n_kv_heads;
  L->causal = d->causal;
  L->n = d->n_keys;
  L->nq = d->n_queries;
  L->scale = d->softmax_scale == 0.f ? 1.0 / std::sqrt((double)d->head_dim) : (double)d->softmax_scale;
  L->c_log2 = (float)(L->scale * 1.4426950408889634074);
  return KVC_OK;
}

kvc_status need_bf16(const void* p, const char* name) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(KVC_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return KVC_OK;
}

kvc_status need_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(KVC_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return KVC_OK;
}

kvc_status need_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return KVC_OK;
  if (!ws) return fail(KVC_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned(ws, 256)) return fail(KVC_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (have < need) return fail(KVC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return KVC_OK;
}

// The current device must be a gfx950; checked once per device.
std::mutex g_dev_mu;
int g_dev_ok[64] = {0};   // 0 unknown, 1 ok, -1 not gfx950

kvc_status need_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return fail(KVC_ERR_NO_DEVICE, "no HIP device available");
  }
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KVC_ERR_NO_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  if (g_dev_ok[dev] != 1) return fail(KVC_ERR_NO_DEVICE, "device %d is not a gfx950", dev);
  return KVC_OK;
}

#define KVC_TRY(expr)               \
  do {                              \
    kvc_status _st = (expr);        \
    if (_st != KVC_OK) return _st;  \
  } while (0)

kvc_status finish(hipError_t e, const char* where) {
  if (e != hipSuccess) return hip_fail(e, where);
  return ok();
}

__global__ void reset_status_kernel(int32_t* status) { *status = 0; }

}  // namespace

hipError_t launch_reset_status(char* ws, hipStream_t s) {
  reset_status_kernel<<<1, 1, 0, s>>>(reinterpret_cast<int32_t*>(ws));
  return hipGetLastError();
}

}  // namespace kvc

using namespace kvc;

extern "C" {

size_t kvc_workspace_size(int32_t op, const kvc_layer_desc* desc, int32_t mode) {
  Layer L;
  std::string saved = g_last_error;
  if (make_layer(desc, &L, op == KVC_OP_RIDGE_FIT) != KVC_OK) return 0;
  g_last_error = saved;
  switch (op) {
    case KVC_OP_ROW_LSE: return lse_ws_bytes(L);
    case KVC_OP_SCORE_TOKENS:
      if (mode != KVC_SCORE_SUM && mode != KVC_SCORE_MAX) return 0;
      return score_ws_bytes(L, mode, 0);
    case KVC_OP_CHANNEL_WEIGHTS: return chanw_ws_bytes(L);
    case KVC_OP_ALLOCATE_BITS:
      if (mode < KVC_ALLOC_V_TOKENS || mode > KVC_ALLOC_TOPK) return 0;
      return alloc_ws_bytes(L, mode);
    case KVC_OP_QUANTIZE_PACK: return pack_ws_bytes(L);
    case KVC_OP_COMPRESSED_ATTEND: return attend_ws_bytes(L);
    case KVC_OP_RIDGE_FIT:
      if (mode < 1 || mode > L.n || mode > kMaxRidgePairs) return 0;
      return ridge_ws_bytes(L, mode);
    default: return 0;
  }
}

kvc_status kvc_row_lse(const kvc_layer_desc* desc, const void* q, const void* k, float* lse,
                       void* ws, size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(need_bf16(k, "k"));
  KVC_TRY(need_ptr(lse, 4, "lse"));
  KVC_TRY(need_ws(ws, ws_bytes, lse_ws_bytes(L)));
  KVC_TRY(need_device());
  return finish(launch_row_lse(L, (const uint16_t*)q, (const uint16_t*)k, lse, (char*)ws,
                               (hipStream_t)hip_stream),
                "kvc_row_lse launch");
}

kvc_status kvc_row_lse_noalloc(const kvc_layer_desc* desc, const void* q, const void* k, float* lse,
                               void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(need_bf16(k, "k"));
  KVC_TRY(need_ptr(lse, 4, "lse"));
  const size_t need = lse_ws_bytes(L);
  if (need > kLseScratchBytes)
    return fail(KVC_ERR_UNSUPPORTED,
                "kvc_row_lse_noalloc: this layer needs %zu bytes of scratch, more than the %zu bytes the library "
                "holds (call kvc_row_lse with a workspace)", need, kLseScratchBytes);
  KVC_TRY(need_device());
  char* scratch_dev = nullptr;
  hipError_t e = row_lse_scratch(&scratch_dev);
  if (e != hipSuccess) return hip_fail(e, "kvc_row_lse_noalloc: hipGetSymbolAddress(scratch)");
  return finish(launch_row_lse(L, (const uint16_t*)q, (const uint16_t*)k, lse, scratch_dev, (hipStream_t)hip_stream),
                "kvc_row_lse_noalloc launch");
}

kvc_status kvc_score_tokens(const kvc_layer_desc* desc, kvc_score_mode mode, const void* q,
                            const void* k, const float* lse, const kvc_kvzip_args* zip,
                            float* scores, void* ws, size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  if (mode != KVC_SCORE_SUM && mode != KVC_SCORE_MAX) return fail(KVC_ERR_INVALID_ARG, "bad score mode %d", (int)mode);
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(need_bf16(k, "k"));
  KVC_TRY(need_ptr(lse, 4, "lse"));
  KVC_TRY(need_ptr(scores, 4, "scores"));
  int hd = 0;
  if (mode == KVC_SCORE_MAX) {
    if (!zip) return fail(KVC_ERR_INVALID_ARG, "MAX mode needs kvzip args");
    if (zip->reserved != 0) return fail(KVC_ERR_INVALID_ARG, "kvzip.reserved must be 0");
    if (zip->hidden_dim < 1) return fail(KVC_ERR_INVALID_ARG, "hidden_dim must be >= 1");
    KVC_TRY(need_ptr(zip->hidden, 2, "hidden"));
    KVC_TRY(need_ptr(zip->w_o, 2, "w_o"));
    KVC_TRY(need_bf16(zip->v, "v"));
    hd = zip->hidden_dim;
  }
  KVC_TRY(need_ws(ws, ws_bytes, score_ws_bytes(L, mode, hd)));
  KVC_TRY(need_device());
  return finish(launch_score(L, mode, (const uint16_t*)q, (const uint16_t*)k, lse,
                             zip ? (const uint16_t*)zip->hidden : nullptr,
                             zip ? (const uint16_t*)zip->w_o : nullptr,
                             zip ? (const uint16_t*)zip->v : nullptr, hd, scores, (char*)ws,
                             (hipStream_t)hip_stream),
                "kvc_score_tokens launch");
}

kvc_status kvc_channel_weights(const kvc_layer_desc* desc, const void* q, const void* k,
                               float* w_c, void* ws, size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(need_bf16(k, "k"));
  KVC_TRY(need_ptr(w_c, 4, "w_c"));
  KVC_TRY(need_ws(ws, ws_bytes, chanw_ws_bytes(L)));
  KVC_TRY(need_device());
  return finish(launch_channel_weights(L, (const uint16_t*)q, (const uint16_t*)k, w_c, (char*)ws,
                                       (hipStream_t)hip_stream),
                "kvc_channel_weights launch");
}

kvc_status kvc_allocate_bits(const kvc_layer_desc* desc, kvc_alloc_stage stage,
                             const float* weight, const float* sigma, const uint8_t* bits_v,
                             double avg_bits_per_elem, double keep_fraction, uint8_t keep_bits,
                             uint8_t* bits_out, kvc_alloc_result* result_dev, void* ws,
                             size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  if (stage < KVC_ALLOC_V_TOKENS || stage > KVC_ALLOC_TOPK)
    return fail(KVC_ERR_INVALID_ARG, "bad allocation stage %d", (int)stage);
  KVC_TRY(need_ptr(weight, 4, "weight"));
  if (sigma && !aligned(sigma, 4)) return fail(KVC_ERR_INVALID_ARG, "sigma is not 4-byte aligned");
  if (!bits_out) return fail(KVC_ERR_INVALID_ARG, "bits_out is NULL");
  if (result_dev && !aligned(result_dev, 8)) return fail(KVC_ERR_INVALID_ARG, "result is not 8-byte aligned");
  if (stage == KVC_ALLOC_K_CHANNELS && !bits_v) return fail(KVC_ERR_INVALID_ARG, "K stage needs bits_v");
  if (stage != KVC_ALLOC_TOPK) {
    // avg <= 2^16 keeps floor(avg * E) below 2^62 for every valid layer (E < 2^44).
    if (!std::isfinite(avg_bits_per_elem) || avg_bits_per_elem < 0.0 || avg_bits_per_elem > 65536.0)
      return fail(KVC_ERR_INVALID_ARG, "avg_bits_per_elem must be in [0, 65536]");
  } else {
    if (!(keep_fraction >= 0.0 && keep_fraction <= 1.0))
      return fail(KVC_ERR_INVALID_ARG, "keep_fraction must be in [0, 1]");
    if (keep_bits != 2 && keep_bits != 4 && keep_bits != 8 && keep_bits != 16)
      return fail(KVC_ERR_INVALID_ARG, "keep_bits must be 2, 4, 8 or 16");
  }
  KVC_TRY(need_ws(ws, ws_bytes, alloc_ws_bytes(L, stage)));
  KVC_TRY(need_device());
  return finish(launch_allocate(L, stage, weight, sigma, bits_v, avg_bits_per_elem, keep_fraction,
                                keep_bits, bits_out, result_dev, (char*)ws, (hipStream_t)hip_stream),
                "kvc_allocate_bits launch");
}

kvc_status kvc_keep_threshold(const kvc_layer_desc* desc, const float* scores, float threshold,
                              int64_t window, uint8_t keep_bits, uint8_t* bits_out,
                              int64_t* kept_dev, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_ptr(scores, 4, "scores"));
  if (!bits_out) return fail(KVC_ERR_INVALID_ARG, "bits_out is NULL");
  if (kept_dev && !aligned(kept_dev, 8)) return fail(KVC_ERR_INVALID_ARG, "kept is not 8-byte aligned");
  if (std::isnan(threshold)) return fail(KVC_ERR_INVALID_ARG, "threshold is NaN");
  if (window < 0) return fail(KVC_ERR_INVALID_ARG, "window must be >= 0");
  if (keep_bits != 2 && keep_bits != 4 && keep_bits != 8 && keep_bits != 16)
    return fail(KVC_ERR_INVALID_ARG, "keep_bits must be 2, 4, 8 or 16");
  KVC_TRY(need_device());
  return finish(launch_keep_threshold(L, scores, threshold, window, keep_bits, bits_out, kept_dev,
                                      (hipStream_t)hip_stream),
                "kvc_keep_threshold launch");
}

kvc_status kvc_packed_capacity(const kvc_layer_desc* desc, int32_t group_size,
                               size_t bytes_per_buffer[KVC_PK_NBUF]) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  if (group_size != 32) return fail(KVC_ERR_UNSUPPORTED, "group_size %d (only 32)", group_size);
  if (!bytes_per_buffer) return fail(KVC_ERR_INVALID_ARG, "bytes_per_buffer is NULL");
  packed_capacity(L, bytes_per_buffer);
  return ok();
}

static kvc_status check_cache(const kvc_packed_cache* c) {
  if (!c) return fail(KVC_ERR_INVALID_ARG, "packed cache is NULL");
  KVC_TRY(need_ptr(c->header, 8, "cache.header"));
  KVC_TRY(need_ptr(c->v_idx, 4, "cache.v_idx"));
  KVC_TRY(need_ptr(c->v_words, 16, "cache.v_words"));
  KVC_TRY(need_ptr(c->v_par, 8, "cache.v_par"));
  KVC_TRY(need_ptr(c->k_keep, 4, "cache.k_keep"));
  KVC_TRY(need_ptr(c->k_vloc, 4, "cache.k_vloc"));
  KVC_TRY(need_ptr(c->k_words, 16, "cache.k_words"));
  KVC_TRY(need_ptr(c->k_par, 8, "cache.k_par"));
  KVC_TRY(need_ptr(c->k_width, 1, "cache.k_width"));
  return KVC_OK;
}

kvc_status kvc_quantize_pack(const kvc_layer_desc* desc, const void* k, const void* v,
                             const uint8_t* bits_v, const uint8_t* bits_k, int32_t group_size,
                             const kvc_packed_cache* out, void* ws, size_t ws_bytes,
                             void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  if (group_size != 32) return fail(KVC_ERR_UNSUPPORTED, "group_size %d (only 32)", group_size);
  KVC_TRY(need_bf16(k, "k"));
  KVC_TRY(need_bf16(v, "v"));
  if (!bits_v || !bits_k) return fail(KVC_ERR_INVALID_ARG, "bits_v / bits_k is NULL");
  KVC_TRY(check_cache(out));
  KVC_TRY(need_ws(ws, ws_bytes, pack_ws_bytes(L)));
  KVC_TRY(need_device());
  return finish(launch_pack(L, (const uint16_t*)k, (const uint16_t*)v, bits_v, bits_k, *out,
                            (char*)ws, (hipStream_t)hip_stream),
                "kvc_quantize_pack launch");
}

kvc_status kvc_compressed_attend(const kvc_layer_desc* desc, const void* q,
                                 const kvc_packed_cache* cache, float* out, float* lse,
                                 void* ws, size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(check_cache(cache));
  KVC_TRY(need_ptr(out, 4, "out"));
  KVC_TRY(need_ptr(lse, 4, "lse"));
  KVC_TRY(need_ws(ws, ws_bytes, attend_ws_bytes(L)));
  KVC_TRY(need_device());
  return finish(launch_attend(L, (const uint16_t*)q, *cache, out, lse, (char*)ws, (hipStream_t)hip_stream),
                "kvc_compressed_attend launch");
}

kvc_status kvc_compressed_attend_append(const kvc_layer_desc* desc, const void* q,
                                        const kvc_packed_cache* cache, const void* k_new,
                                        const void* v_new, int64_t n_new, float* out, float* lse,
                                        void* ws, size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(check_cache(cache));
  KVC_TRY(need_ptr(out, 4, "out"));
  KVC_TRY(need_ptr(lse, 4, "lse"));
  if (n_new < 0) return fail(KVC_ERR_INVALID_ARG, "n_new must be >= 0");
  if (n_new > 0) {
    KVC_TRY(need_bf16(k_new, "k_new"));
    KVC_TRY(need_bf16(v_new, "v_new"));
  }
  KVC_TRY(need_ws(ws, ws_bytes, attend_ws_bytes(L)));
  KVC_TRY(need_device());
  return finish(launch_attend(L, (const uint16_t*)q, *cache, out, lse, (char*)ws, (hipStream_t)hip_stream,
                              (const uint16_t*)k_new, (const uint16_t*)v_new, n_new),
                "kvc_compressed_attend_append launch");
}

kvc_status kvc_fidelity_terms(const kvc_layer_desc* desc, const float* y_hat, const float* lse_hat,
                              const float* y, const float* lse, double* terms, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L));
  KVC_TRY(need_ptr(y_hat, 16, "y_hat"));
  KVC_TRY(need_ptr(y, 16, "y"));
  KVC_TRY(need_ptr(lse_hat, 4, "lse_hat"));
  KVC_TRY(need_ptr(lse, 4, "lse"));
  KVC_TRY(need_ptr(terms, 8, "terms"));
  KVC_TRY(need_device());
  return finish(launch_fidelity_terms(L, y_hat, lse_hat, y, lse, terms, (hipStream_t)hip_stream),
                "kvc_fidelity_terms launch");
}

kvc_status kvc_pilot_budgets(const double* mse, int32_t n, int64_t total, int64_t floor_each,
                             int64_t* budgets) {
  if (!mse || !budgets) return fail(KVC_ERR_INVALID_ARG, "mse / budgets is NULL");
  if (n < 1) return fail(KVC_ERR_INVALID_ARG, "n must be >= 1");
  if (total < 0 || floor_each < 0) return fail(KVC_ERR_INVALID_ARG, "total and floor_each must be >= 0");
  if (total >= (int64_t(1) << 53)) return fail(KVC_ERR_UNSUPPORTED, "total >= 2^53");
  for (int32_t i = 0; i < n; ++i)
    if (!std::isfinite(mse[i]) || mse[i] < 0.0)
      return fail(KVC_ERR_INVALID_ARG, "mse[%d] must be finite and >= 0", (int)i);
  if (floor_each > total / n) return fail(KVC_ERR_INVALID_ARG, "total is below n * floor_each");
  const int64_t rest = total - (int64_t)n * floor_each;
  std::vector<double> r(n), share(n), frac(n);
  double tot = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    r[i] = std::sqrt(mse[i]);
    tot += r[i];
  }
  for (int32_t i = 0; i < n; ++i) share[i] = tot == 0.0 ? (double)rest / (double)n : (double)rest * (r[i] / tot);
  int64_t used = 0;
  for (int32_t i = 0; i < n; ++i) {
    const double b = std::floor(share[i]);
    budgets[i] = (int64_t)b;
    frac[i] = share[i] - b;
    used += budgets[i];
  }
  int64_t left = rest - used;
  std::vector<int32_t> order;
  order.reserve(n);
  if (left >= 0) {
    for (int32_t i = 0; i < n; ++i) order.push_back(i);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return frac[a] > frac[b]; });
    for (int64_t j = 0; j < left && j < n; ++j) budgets[order[j]] += 1;
  } else {
    // rounding left the floors above the rest: take units back from the smallest fractions
    for (int32_t i = n - 1; i >= 0; --i)
      if (budgets[i] > 0) order.push_back(i);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return frac[a] < frac[b]; });
    for (int64_t j = 0; j < -left && j < (int64_t)order.size(); ++j) budgets[order[j]] -= 1;
  }
  for (int32_t i = 0; i < n; ++i) budgets[i] += floor_each;
  return ok();
}

kvc_status kvc_ridge_value_fit(const kvc_layer_desc* desc, int64_t n_compressed, const void* q, const void* k,
                               const void* v_r, const float* y, double lambda, float* v_c, void* ws,
                               size_t ws_bytes, void* hip_stream) {
  Layer L;
  KVC_TRY(make_layer(desc, &L, true));
  if (n_compressed < 1 || n_compressed > L.n)
    return fail(KVC_ERR_INVALID_ARG, "n_compressed %lld outside [1, n_keys]", (long long)n_compressed);
  if (n_compressed > kMaxRidgePairs) return fail(KVC_ERR_UNSUPPORTED, "n_compressed > %d", kMaxRidgePairs);
  if (!std::isfinite(lambda) || lambda < 0.0) return fail(KVC_ERR_INVALID_ARG, "lambda must be finite and >= 0");
  if ((int64_t)L.G * L.nq > (int64_t(1) << 22)) return fail(KVC_ERR_UNSUPPORTED, "G * Nq > 2^22 rows");
  KVC_TRY(need_bf16(q, "q"));
  KVC_TRY(need_bf16(k, "k"));
  if (n_compressed < L.n) KVC_TRY(need_bf16(v_r, "v_r"));
  KVC_TRY(need_ptr(y, 16, "y"));
  KVC_TRY(need_ptr(v_c, 16, "v_c"));
  KVC_TRY(need_ws(ws, ws_bytes, ridge_ws_bytes(L, n_compressed)));
  KVC_TRY(need_device());
  return finish(launch_ridge_fit(L, n_compressed, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v_r, y,
                                 lambda, v_c, (char*)ws, (hipStream_t)hip_stream),
                "kvc_ridge_value_fit launch");
}

kvc_status kvc_get_device_status(const void* ws, int32_t* code, void* hip_stream) {
  if (!ws || !code) return fail(KVC_ERR_INVALID_ARG, "ws / code is NULL");
  KVC_TRY(need_device());
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipMemcpyAsync(code, ws, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(status)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return ok();
}

const char* kvc_status_string(kvc_status status) {
  switch (status) {
    case KVC_OK: return "KVC_OK";
    case KVC_ERR_INVALID_ARG: return "KVC_ERR_INVALID_ARG";
    case KVC_ERR_UNSUPPORTED: return "KVC_ERR_UNSUPPORTED";
    case KVC_ERR_WORKSPACE: return "KVC_ERR_WORKSPACE";
    case KVC_ERR_NO_DEVICE: return "KVC_ERR_NO_DEVICE";
    case KVC_ERR_HIP: return "KVC_ERR_HIP";
    case KVC_ERR_DEVICE_DATA: return "KVC_ERR_DEVICE_DATA";
    default: return "KVC_ERR_UNKNOWN";
  }
}

const char* kvc_last_error(void) { return g_last_error.c_str(); }

const char* kvc_version(void) { return "kvc 0.1.0 gfx950"; }

}  // extern "C"
