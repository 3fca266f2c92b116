// Host-side internal interface between the C ABI layer (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// Validated view of a kvc_layer_desc.
struct Layer {
  int hq, hkv, d, G, causal;
  int64_t n, nq;
  double scale;     // softmax scale (float64; 1/sqrt(d) unless the caller fixed one)
  float c_log2;     // float32(scale * log2(e)): logits in the base-2 domain
};

// Bump allocator over the caller's workspace.  Offset 0 holds the device status word.
struct WsPlan {
  size_t off = 256;
  size_t take(size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  }
};

// ---- scorer ------------------------------------------------------------------------------
// Both passes split the layer into work items (KV head g, 256-row tile rt, key chunk ch,
// query head of the group hl); a block of 4 waves handles one item.
struct ScorePlan {
  int nRT;          // 256-row tiles
  int KC;           // keys per chunk (multiple of 64)
  int maxCh;        // chunks of the longest row tile
  int64_t W;        // work items H_kv * nRT * maxCh * G (some are empty)
  int64_t Npad;     // N rounded up to 256
};
ScorePlan score_plan(const Layer& L);
size_t lse_ws_bytes(const Layer& L);
size_t score_ws_bytes(const Layer& L, int mode, int hidden_dim);
hipError_t launch_row_lse(const Layer& L, const uint16_t* q, const uint16_t* k, float* lse,
                          char* ws, hipStream_t s, int tag = 0);
// The allocation-free row LSE: the library's static scratch (kLseScratchBytes per device) stands in
// for the workspace.  row_lse_scratch() gives its address on the current device.
constexpr size_t kLseScratchBytes = size_t(16) << 20;
hipError_t row_lse_scratch(char** out);
hipError_t launch_score(const Layer& L, int mode, const uint16_t* q, const uint16_t* k,
                        const float* lse, const uint16_t* hidden, const uint16_t* w_o,
                        const uint16_t* v, int hidden_dim, float* scores, char* ws,
                        hipStream_t s);

// ---- channel weights --------------------------------------------------------------------
size_t chanw_ws_bytes(const Layer& L);
hipError_t launch_channel_weights(const Layer& L, const uint16_t* q, const uint16_t* k,
                                  float* w_c, char* ws, hipStream_t s);

// ---- allocation -------------------------------------------------------------------------
size_t alloc_ws_bytes(const Layer& L, int stage);
hipError_t launch_allocate(const Layer& L, int stage, const float* weight, const float* sigma,
                           const uint8_t* bits_v, double avg_bits, double keep_fraction,
                           int keep_bits, uint8_t* bits_out, kvc_alloc_result* result,
                           char* ws, hipStream_t s);

// ---- threshold-and-window keep ---------------------------------------------------------
hipError_t launch_keep_threshold(const Layer& L, const float* scores, float threshold, int64_t window,
                                 int keep_bits, uint8_t* bits_out, int64_t* kept, hipStream_t s);

// ---- fidelity terms ---------------------------------------------------------------------
hipError_t launch_fidelity_terms(const Layer& L, const float* y_hat, const float* lse_hat, const float* y,
                                 const float* lse, double* terms, hipStream_t s);

// ---- quantise / pack --------------------------------------------------------------------
void packed_capacity(const Layer& L, size_t bytes[KVC_PK_NBUF]);
size_t pack_ws_bytes(const Layer& L);
hipError_t launch_pack(const Layer& L, const uint16_t* k, const uint16_t* v,
                       const uint8_t* bits_v, const uint8_t* bits_k,
                       const kvc_packed_cache& out, char* ws, hipStream_t s);

// ---- compressed attend ------------------------------------------------------------------
size_t attend_ws_bytes(const Layer& L);
// Decode-shaped attends (at most 16 query rows per KV head): a logits and a values kernel (decode.hip).
int decode_nsplit(const Layer& L);
size_t decode_ws_bytes(const Layer& L);   // the logits (by V row) and the logits blocks' maxima
hipError_t launch_attend_decode(const Layer& L, const uint16_t* q, const kvc_packed_cache& cache, float* part,
                                int nsplit, int pstride, int64_t shift, int32_t* status, char* dws, hipStream_t s);
hipError_t launch_attend(const Layer& L, const uint16_t* q, const kvc_packed_cache& cache,
                         float* out, float* lse, char* ws, hipStream_t s, const uint16_t* k_new = nullptr,
                         const uint16_t* v_new = nullptr, int64_t n_new = 0);

// ---- ridge value fit ----------------------------------------------------------------------
size_t ridge_ws_bytes(const Layer& L, int64_t nc);
hipError_t launch_ridge_fit(const Layer& L, int64_t nc, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v_r, const float* y, double lambda, float* v_c, char* ws,
                            hipStream_t s);

// ---- misc ------------------------------------------------------------------------------
hipError_t launch_reset_status(char* ws, hipStream_t s);

}  // namespace kvc
