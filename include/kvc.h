/*
 * kvc.h -- C ABI of libkvc: KV-cache scoring and compression for one attention layer on an
 * AMD Instinct MI355X (gfx950).
 *
 * The library scores every cached KV unit by the attention it receives and compresses the
 * cache to a mixed-width, partly evicted form:
 *
 *   kvc_row_lse            row log-sum-exp of the causal, scaled logits        (pass 1)
 *   kvc_row_lse_noalloc    the same with the library's static scratch (no workspace)
 *   kvc_score_tokens       per-token scores, RDKV sum or KVzip+ max            (pass 2)
 *   kvc_channel_weights    RDKV K-channel weights
 *   kvc_allocate_bits      Lagrangian width allocation over {0,2,4,8,16}, or top-k keep
 *   kvc_quantize_pack      group quantisation and packing into the width zones
 *   kvc_compressed_attend  attention output and LSE over a packed cache
 *   kvc_compressed_attend_append  the same, over the packed cache and a bf16 buffer of new tokens
 *   kvc_keep_threshold     KVzap threshold keep plus a recent-token window
 *   kvc_fidelity_terms     per-head output and LSE errors of a compressed attend (KVSculpt loss)
 *   kvc_pilot_budgets      per-head budgets in proportion to sqrt(pilot MSE) (host only)
 *   kvc_ridge_value_fit    KVSculpt's closed-form ridge fit of compressed values to given keys
 *
 * Sources (summary pages of the papers; section numbers are the pages' own):
 *   "RDKV - rate-distortion bit allocation for joint eviction and quantization of the KV
 *    cache": §2.1 distortion weights and objective, §2.2 three-stage allocation, §2.3 packed
 *    zones with fused dequantisation.
 *   "KVzap - fast, adaptive and faithful KV cache pruning": §2.1 KVzip+ score, §2.2 one score
 *    per KV head, §2.3 fixed-budget keep of KVzip.
 *   "KVSculpt: KV Cache Compression as Distillation": §2 loss terms (output error and LSE
 *    error) that the fidelity attend measures, §2's closed-form value solve and its adaptive
 *    per-head budget.
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory: the caller owns all memory.  Every pointer argument named as data (q, k, v, lse,
 *   scores, weights, bits, packed buffers, ws, result) is DEVICE memory on the current HIP
 *   device; descriptors and kvc_packed_cache structs are HOST memory holding device
 *   pointers.  The library never allocates device memory and keeps no per-call state.
 *   Outputs must not alias inputs.  Data pointers must be 16-byte aligned.
 * Layouts (row-major, bf16 = IEEE bfloat16 bit patterns):
 *   Q      bf16 [H_q][Nq][d]     K, V  bf16 [H_kv][N][d]
 *   lse    f32  [H_q][Nq]        scores f32 [H_kv][N]      w_c f32 [H_kv][d]
 *   bits_v u8   [H_kv][N]        bits_k u8  [H_kv][d]
 *   query head h reads KV head h / (H_q / H_kv).  Query row i sits at position N - Nq + i
 *   (the rows are the last Nq positions); with causal = 1 it sees key t iff t <= N - Nq + i.
 * Streams: every call only enqueues work on `hip_stream` (a hipStream_t; NULL = the default
 *   stream) and returns; there is no hidden synchronisation.
 * Errors: argument errors are detected on the host and returned before anything is
 *   enqueued.  KVC_ERR_HIP means a HIP runtime call failed; kvc_last_error() gives the
 *   detail (thread-local).  Data errors only visible on the device (a width outside
 *   {0,2,4,8,16}, a packed cache that does not match the descriptor) are recorded in the
 *   status word at the start of `ws`; read it with kvc_get_device_status().
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, misalignment, bad enum value      */
  KVC_ERR_UNSUPPORTED = 2,   /* valid request outside what is built (head_dim, group size) */
  KVC_ERR_WORKSPACE = 3,     /* ws_bytes smaller than kvc_workspace_size()                  */
  KVC_ERR_NO_DEVICE = 4,     /* no HIP device, or the current device is not gfx950          */
  KVC_ERR_HIP = 5,           /* a HIP runtime call failed (detail in kvc_last_error())      */
  KVC_ERR_DEVICE_DATA = 6,   /* device-side data error (see kvc_get_device_status())        */
  KVC_STATUS_INT32_MIN_ = -0x7FFFFFFF - 1,  /* (not statuses) these two give the enum the range */
  KVC_STATUS_INT32_MAX_ = 0x7FFFFFFF        /* of int32_t                                        */
} kvc_status;

/* One attention layer.  Limits: H_q % H_kv == 0, 1 <= H_kv, H_q / H_kv <= 16,
 * head_dim in {64, 128}, 1 <= Nq <= N < 2^29.  softmax_scale == 0 means 1/sqrt(head_dim). */
typedef struct {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t causal;            /* 1: row i sees keys t <= N - Nq + i; 0: every row sees all N */
  int64_t n_keys;            /* N  */
  int64_t n_queries;         /* Nq */
  float softmax_scale;
  int32_t reserved;          /* must be 0 */
} kvc_layer_desc;

/* Operation ids for kvc_workspace_size(). */
enum {
  KVC_OP_ROW_LSE = 0,
  KVC_OP_SCORE_TOKENS = 1,
  KVC_OP_CHANNEL_WEIGHTS = 2,
  KVC_OP_ALLOCATE_BITS = 3,
  KVC_OP_QUANTIZE_PACK = 4,
  KVC_OP_COMPRESSED_ATTEND = 5,
  KVC_OP_RIDGE_FIT = 6
};

/* Bytes of device workspace `op` needs for `desc` (`mode` = score mode, allocation stage, or
 * for KVC_OP_RIDGE_FIT the number of compressed pairs n_c; ignored otherwise).  Returns 0 for an invalid descriptor.  A larger workspace is fine. */
size_t kvc_workspace_size(int32_t op, const kvc_layer_desc* desc, int32_t mode);

/* Pass 1.  lse[h][i] = ln sum_{t visible} exp(scale * q_{h,i} . k_{g(h),t}) (natural log, the
 * scale included): the attention mass KVSculpt's loss matches (KVSculpt §2) and the
 * normaliser of RDKV's attention probabilities (RDKV §2.1).  bf16 matrix-core products with
 * float32 accumulation.  Workspace: kvc_workspace_size(KVC_OP_ROW_LSE, desc, 0) bytes. */
kvc_status kvc_row_lse(const kvc_layer_desc* desc, const void* q, const void* k, float* lse,
                       void* ws, size_t ws_bytes, void* hip_stream);

/* kvc_row_lse for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and the same result,
 * with no workspace argument.  Its scratch (pass 1's per-chunk partials) is a static device
 * array inside the library, 16 MiB per device, held from the first call on a device until the
 * process ends; the call itself allocates nothing.  Layers whose kvc_workspace_size(
 * KVC_OP_ROW_LSE, desc, 0) exceeds 16 MiB are rejected with KVC_ERR_UNSUPPORTED (the decode
 * cache of 32 query heads x 512 rows x 131072 keys needs 8 MiB).  Every call on one device
 * shares that scratch, so calls that overlap on one device (concurrent streams or host threads)
 * race and must be ordered by the caller; nothing in it needs clearing between calls.
 * Errors: as kvc_row_lse, plus KVC_ERR_UNSUPPORTED for a layer beyond the scratch. */
kvc_status kvc_row_lse_noalloc(const kvc_layer_desc* desc, const void* q, const void* k, float* lse,
                               void* hip_stream);

/* The enums of this header span the range of int32_t (their last two members), so any int32
 * value is a valid argument of the enum type, and one outside the listed modes is refused with
 * KVC_ERR_INVALID_ARG. */
typedef enum {
  KVC_SCORE_SUM = 0,
  KVC_SCORE_MAX = 1,
  KVC_SCORE_INT32_MIN_ = -0x7FFFFFFF - 1,
  KVC_SCORE_INT32_MAX_ = 0x7FFFFFFF
} kvc_score_mode;

/* Extra inputs of the KVzip+ score (KVzap §2.1); required iff mode == KVC_SCORE_MAX. */
typedef struct {
  const void* hidden;        /* bf16 [Nq][D_h]: hidden state h_j of each query row          */
  const void* w_o;           /* bf16 [D_h][H_q*d]: output projection, Linear weight (out x in) */
  const void* v;             /* bf16 [H_kv][N][d] */
  int32_t hidden_dim;        /* D_h, a positive multiple of 8 */
  int32_t reserved;          /* must be 0 */
} kvc_kvzip_args;

/* Pass 2.  With a = exp(scale q.k - lse) (lse from kvc_row_lse):
 *   SUM: scores[g][t] = sum over the group's query heads h and visible rows i of a_{h,i,t}
 *        (RDKV §2.1 token distortion weight);
 *   MAX: scores[g][t] = max over the group's heads h of
 *        ( max over visible rows j of a_{h,j,t} * ||hidden_j|| ) / ||W_O^(h) v_{g,t}||,
 *        W_O^(h) = columns [h*d, (h+1)*d) of W_O (KVzap §2.1, one score per KV head §2.2);
 *        a zero value norm gives +inf (0 if the numerator is 0).
 * Column reductions run in a fixed order: results are bitwise reproducible. */
kvc_status kvc_score_tokens(const kvc_layer_desc* desc, kvc_score_mode mode, const void* q,
                            const void* k, const float* lse, const kvc_kvzip_args* zip,
                            float* scores, void* ws, size_t ws_bytes, void* hip_stream);

/* RDKV §2.1 channel weight: w_c[g][c] = scale * ||Q_g[:,c]||_2 * ||K_g[:,c]||_2, Q_g stacking
 * every row of every query head of group g, K_g the whole cache of head g (computed once on the
 * full cache, RDKV §2.2 stage 1).  Sums of squares are accumulated in float64. */
kvc_status kvc_channel_weights(const kvc_layer_desc* desc, const void* q, const void* k,
                               float* w_c, void* ws, size_t ws_bytes, void* hip_stream);

typedef enum {
  KVC_ALLOC_V_TOKENS = 0,    /* RDKV stage 2: units (g,t), size d                            */
  KVC_ALLOC_K_CHANNELS = 1,  /* RDKV stage 3: units (g,c), size R_g = #tokens with bits_v > 0 */
  KVC_ALLOC_TOPK = 2,        /* KVzip fixed budget: keep floor(rho*N) best tokens per head    */
  KVC_ALLOC_INT32_MIN_ = -0x7FFFFFFF - 1,
  KVC_ALLOC_INT32_MAX_ = 0x7FFFFFFF
} kvc_alloc_stage;

/* Allocation result, written to DEVICE memory by kvc_allocate_bits. */
typedef struct {
  double lambda;             /* lambda* (V/K stages); the kept score threshold (TOPK)         */
  int64_t budget_bits;       /* B = floor(avg * elements covered) (V/K); kept*d*keep_bits (TOPK) */
  int64_t used_bits;         /* sum_u size_u * b_u                                             */
  double distortion;         /* sum_u c_u 2^-b_u (V/K); 0 (TOPK)                               */
} kvc_alloc_result;

/* RDKV §2.1-§2.2: minimise sum_u c_u 2^-b_u subject to sum_u size_u b_u <= B over widths
 * {0,2,4,8,16}, c_u = float32(weight_u * sigma_u) (sigma NULL: c_u = weight_u), by reverse
 * water-filling with one multiplier per call.  Exact rule: the key of step k of unit u is
 * (c_u * num_k) / (size_u * den_k) in float64 with theta_k = num_k/den_k = 3/8, 3/32, 15/1024,
 * 255/524288; lambda* is the smallest key (or 0) whose rate of steps with key > lambda* fits
 * B; every step with key > lambda* is taken, then steps with key == lambda* in ascending unit
 * index (unit = g*N + t or g*d + c) until the first that does not fit.  Units with c_u <= 0,
 * NaN, or size 0 get width 0.  B = floor(avg_bits_per_elem * E), E = H_kv*N*d (V stage) or
 * d * sum_g R_g (K stage, counted on the device from bits_v).
 * TOPK (KVzap §2.3 describes KVzip's fixed keep): per KV head keep the floor(keep_fraction*N)
 * highest scores at width keep_bits (ties to the lower index), others 0.
 * weight: f32 [H_kv][N] (V, TOPK) or [H_kv][d] (K).  sigma: same shape or NULL (ignored by
 * TOPK).  bits_v: u8 [H_kv][N], K stage only (else NULL).  bits_out: u8, same shape as
 * weight.  result_dev: device kvc_alloc_result, may be NULL.
 * Errors: avg_bits_per_elem < 0 or not finite, keep_fraction outside [0,1], keep_bits not in
 * {2,4,8,16}.  A width outside {0,2,4,8,16} in bits_v sets the device status. */
kvc_status kvc_allocate_bits(const kvc_layer_desc* desc, kvc_alloc_stage stage,
                             const float* weight, const float* sigma, const uint8_t* bits_v,
                             double avg_bits_per_elem, double keep_fraction, uint8_t keep_bits,
                             uint8_t* bits_out, kvc_alloc_result* result_dev, void* ws,
                             size_t ws_bytes, void* hip_stream);

/* KVzap §2.3 adaptive keep: per KV head, token t keeps width keep_bits when
 * scores[g][t] >= threshold (a float32 compare; a NaN score never passes) or when it is one
 * of the head's last `window` tokens (t >= N - window; the pages keep w = 128); every other
 * token gets width 0.  The pages threshold predicted log-scores against tau and log is
 * increasing, so a caller holding tau passes threshold = float32(exp(tau)).  The ratio kept
 * follows the scores, unlike the fixed top-k stage of kvc_allocate_bits.
 * scores: f32 [H_kv][N] (device).  bits_out: u8 [H_kv][N] (device; the widths the pack step
 * takes as bits_v).  kept_dev: i64 [H_kv] (device), tokens kept per head, or NULL.  No
 * workspace; asynchronous on hip_stream.  Uses desc's n_kv_heads and n_keys only.
 * Errors: NULL scores or bits_out, misaligned scores or kept_dev, NaN threshold, window < 0,
 * keep_bits not in {2,4,8,16}. */
kvc_status kvc_keep_threshold(const kvc_layer_desc* desc, const float* scores, float threshold,
                              int64_t window, uint8_t keep_bits, uint8_t* bits_out,
                              int64_t* kept_dev, void* hip_stream);

/* ---- Packed cache ------------------------------------------------------------------------
 * RDKV §2.3 stores retained rows grouped by width so each width has one dequantisation
 * path.  This library's layout (its own format; a token is retained iff bits_v > 0; zone z
 * holds width {2,4,8,16}[z]; group = 32 elements):
 *   header  i64 [16 + 24*H_kv].  [0..3] H_kv, d, N, 32; [4..9] totals of v_idx, v_words,
 *           v_par pairs, k_keep, k_words, k_par pairs.  Per head g at 16 + 24*g:
 *           [0..3] tokens per zone, [4] R_g, [5..8] v_idx offset per zone, [9..12] v_words
 *           offset per zone, [13..16] v_par offset per zone (pairs), [17] k_keep/k_vloc
 *           offset, [18] k_words offset, [19] k_par offset (pairs), [20] words per K group
 *           (sum_c bits_k), [21] quantised K channels (width 2/4/8), [22] K groups
 *           ceil(R_g/32), [23] 0.  Heads are concatenated in order, zones in width order.
 *   v_idx   i32  token ids of each (head, zone), ascending
 *   v_words u32  per listed token: d/32 groups x b words
 *   v_par   f32  (scale, zero) per listed token and group, zones 2/4/8 only
 *   k_keep  i32  retained tokens of each head, ascending
 *   k_vloc  i32  per retained token: zone << 29 | position within its V zone
 *   k_words u32  per head, per group j of 32 retained tokens, per channel c ascending with
 *                bits_k[c] > 0: bits_k[c] words (a short last group is padded with code 0)
 *   k_par   f32  (scale, zero) per (group j, channel c with bits_k[c] in {2,4,8})
 *   k_width u8   [H_kv][d] copy of bits_k
 * Quantiser per group x at width b in {2,4,8}: z = min x, s = float32(float64(max - min) /
 * (2^b - 1)), code = clamp(round_half_even(float64(x - z) / s), 0, 2^b - 1), every code 0
 * when s == 0; element e uses bits [e*b, e*b + b) of the group's little-endian u32 stream;
 * b = 16 stores the raw bf16 bits.  V groups run over the d channels of one token, K groups
 * over 32 consecutive retained tokens of one channel. */
enum {
  KVC_PK_HEADER = 0, KVC_PK_V_IDX, KVC_PK_V_WORDS, KVC_PK_V_PAR, KVC_PK_K_KEEP,
  KVC_PK_K_VLOC, KVC_PK_K_WORDS, KVC_PK_K_PAR, KVC_PK_K_WIDTH, KVC_PK_NBUF
};
#define KVC_HDR_GLOBAL 16
#define KVC_HDR_PER_HEAD 24

typedef struct {
  int64_t* header;
  int32_t* v_idx;
  uint32_t* v_words;
  float* v_par;
  int32_t* k_keep;
  int32_t* k_vloc;
  uint32_t* k_words;
  float* k_par;
  uint8_t* k_width;
} kvc_packed_cache;

/* Worst-case bytes of each packed buffer (indexed by KVC_PK_*) for `desc`. */
kvc_status kvc_packed_capacity(const kvc_layer_desc* desc, int32_t group_size,
                               size_t bytes_per_buffer[KVC_PK_NBUF]);

/* Quantise and pack K and V at the widths bits_v (per token) and bits_k (per channel),
 * RDKV §2.2 stages 2-3 and §2.3 zones.  `out` is a host struct of device buffers of at least
 * kvc_packed_capacity() bytes.  Only retained units are read.  group_size must be 32. */
kvc_status kvc_quantize_pack(const kvc_layer_desc* desc, const void* k, const void* v,
                             const uint8_t* bits_v, const uint8_t* bits_k, int32_t group_size,
                             const kvc_packed_cache* out, void* ws, size_t ws_bytes,
                             void* hip_stream);

/* Attention of Q (the last Nq = desc->n_queries rows of the sequence, [H_q][Nq][d]) over the
 * retained tokens of a packed cache, dequantised on the fly (x = zero + scale*code; width 0
 * channels are 0; width 16 the stored bf16 value): out f32 [H_q][Nq][d] and lse f32 [H_q][Nq]
 * (RDKV §2.3 decode over packed zones; the two outputs whose errors form KVSculpt's loss,
 * §2).  A row with no visible retained token gets lse = -inf and out = 0.  The packed cache's
 * header must match desc (H_kv, d, N); a mismatch sets the device status.
 * Precision: with more than 16 query rows per KV head, logits use keys to 2^-17 relative (bf16
 * hi + lo) with float32 accumulation, and the value products take fp16 operands: the
 * probabilities, and V_hat scaled per KV head by a power of two that puts the head's largest
 * |V_hat| in [2^14, 2^15), so any finite bf16 V keeps 11 significant bits (values below 2^-24 of
 * the head's largest round to that absolute step).  With at most 16 rows (decode) the codes and
 * raw bf16 values enter exactly, q * scale and p * scale_v as bf16 hi + lo pairs (2^-17
 * relative), zero terms exactly or in float32, all accumulated in float32.  Workspace: the
 * decode path also holds every retained token's logits (4 * H_kv * N * 16 bytes at most); with
 * G * ceil(Nq / 32) > 24 query row tiles per KV head every group of 32 retained tokens is decoded
 * once into the workspace (192 * d bytes for each of the H_kv * ceil(N / 32) possible groups). */
kvc_status kvc_compressed_attend(const kvc_layer_desc* desc, const void* q,
                                 const kvc_packed_cache* cache, float* out, float* lse,
                                 void* ws, size_t ws_bytes, void* hip_stream);

/* kvc_compressed_attend over the packed cache followed by an append buffer: the n_new tokens
 * generated since compression, kept as raw bf16 beside the packed zones (RDKV §2.3), at
 * positions N .. N+n_new-1.  The query rows are the last Nq of the N + n_new positions (row i
 * at N + n_new - Nq + i; with the causal flag it sees the new tokens up to its own position).
 * The buffer's keys and values are attended exactly; its log-sum-exp part is merged with the
 * packed cache's.  k_new, v_new: bf16 [H_kv][n_new][d] (device, 16-byte aligned; NULL allowed
 * when n_new == 0, which gives kvc_compressed_attend).  ws: as kvc_compressed_attend
 * (KVC_OP_COMPRESSED_ATTEND sizes both).  Errors: n_new < 0, a NULL or misaligned buffer when
 * n_new > 0, and every error of kvc_compressed_attend. */
kvc_status kvc_compressed_attend_append(const kvc_layer_desc* desc, const void* q,
                                        const kvc_packed_cache* cache, const void* k_new,
                                        const void* v_new, int64_t n_new, float* out, float* lse,
                                        void* ws, size_t ws_bytes, void* hip_stream);

/* The two terms of KVSculpt's distillation loss (KVSculpt §2), split by query head: for head h,
 * terms[h][0] = sum over rows i and channels c of (y_hat - y)^2 and terms[h][1] = sum over rows
 * of (lse_hat - lse)^2, both accumulated in float64 from the float32 inputs.  A row whose two
 * LSE values are equal adds 0 (this covers a row that sees no token in either attend, both
 * -inf); -inf against a finite value adds +inf.  The summation order is fixed (a strided
 * split over 256 lanes, then a fixed tree), so repeated calls give identical bits.
 * y_hat, y: f32 [H_q][Nq][d] (device, 16-byte aligned), the outputs of kvc_compressed_attend
 * over the compressed and the uncompressed cache.  lse_hat, lse: f32 [H_q][Nq] (device).
 * terms: f64 [H_q][2] (device).  No workspace; asynchronous on hip_stream.  Uses desc's
 * n_q_heads, head_dim and n_queries.  Errors: a NULL or misaligned pointer. */
kvc_status kvc_fidelity_terms(const kvc_layer_desc* desc, const float* y_hat, const float* lse_hat,
                              const float* y, const float* lse, double* terms, void* hip_stream);

/* KVSculpt §2 adaptive budget: after a pilot at a uniform budget, head i's share of `total` is
 * proportional to sqrt(mse[i]).  Each head first gets floor_each; the rest R = total -
 * n*floor_each is split as R * sqrt(mse[i]) / sum_j sqrt(mse[j]) (float64, the sum taken in
 * index order), rounded down, and the units left go one each to the largest fractional parts,
 * ties to the lower index.  All MSE zero gives equal shares.  If rounding ever made the floors
 * exceed R, the excess is taken back from the smallest fractional parts among heads holding a
 * unit, ties to the higher index.  The budgets always add up to `total`.
 * mse: f64 [n] and budgets: i64 [n] are HOST memory (this call runs on the host and touches
 * no device).  Errors: NULL pointer, n < 1, total or floor_each < 0, total >= 2^53, an MSE that
 * is negative or not finite, total < n * floor_each. */
kvc_status kvc_pilot_budgets(const double* mse, int32_t n, int64_t total, int64_t floor_each,
                             int64_t* budgets);

/* KVSculpt §2 value step (also §4's Select+Fit): the cache is n_c free pairs (K_c, V_c)
 * followed by the m = n_keys - n_c most recent tokens kept as they are (K_r, V_r).  With the
 * keys fixed the attention weights A = softmax(scale Q [K_c; K_r]^T) do not depend on the
 * values, and this call returns the V_c minimising ||A_c V_c + A_r V_r - Y||_F^2 +
 * lambda ||V_c||_F^2, i.e. the solution of (A_c^T A_c + lambda I) V_c = A_c^T (Y - A_r V_r).
 * The G query heads of a KV head share its V_c: their rows are stacked into one problem.
 * desc: n_keys = n_c + m, n_queries = Nq training query rows per query head (the layer's
 * causal convention applies, bottom-right over the n_keys keys; causal = 0 for queries that
 * see every key, and then Nq may exceed n_keys).  q: bf16 [H_q][Nq][d]; k: bf16 [H_kv][n_keys][d], compressed keys first;
 * v_r: bf16 [H_kv][m][d] (NULL allowed when m = 0); y: f32 [H_q][Nq][d] target outputs
 * (16-byte aligned); v_c: f32 [H_kv][n_c][d] (output).  A is float32 (exp of float32 logits
 * from bf16 products); the normal equations are summed and solved (blocked Cholesky) in
 * float64, in a fixed order.  Workspace: kvc_workspace_size(KVC_OP_RIDGE_FIT, desc, n_c).
 * Errors: n_c outside [1, n_keys], n_c > 8192, lambda < 0 or not finite, G * Nq > 2^22 rows, a
 * NULL or misaligned pointer.  A normal matrix that is not positive definite (lambda = 0 with
 * too few independent rows) sets KVC_DEV_NOT_SPD in the status word. */
kvc_status kvc_ridge_value_fit(const kvc_layer_desc* desc, int64_t n_compressed, const void* q, const void* k,
                               const void* v_r, const float* y, double lambda, float* v_c, void* ws,
                               size_t ws_bytes, void* hip_stream);

/* Device status codes (bit set). */
#define KVC_DEV_BAD_WIDTH 1
#define KVC_DEV_BAD_CACHE 2
#define KVC_DEV_NOT_SPD 4      /* kvc_ridge_value_fit: the normal matrix is not positive definite */

/* Copy the device status word at the start of `ws` to *code (synchronises `hip_stream`). */
kvc_status kvc_get_device_status(const void* ws, int32_t* code, void* hip_stream);

const char* kvc_status_string(kvc_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* kvc_last_error(void);

/* Library version, e.g. "kvc 0.1.0 gfx950". */
const char* kvc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
