// Scorer: pass 1 (row log-sum-exp) and pass 2 (per-token column reductions of the attention
// probabilities), plus the KVzip+ norm helpers.
//
// Pass 1 computes l_{h,i} = ln sum_{t visible} exp(s q.k) (KVSculpt summary §2, LSE term; the
// normaliser of RDKV's attention probabilities, RDKV summary §2.1).  Pass 2 recomputes
// a = exp(s q.k - l) and reduces it over query rows per key: the RDKV token weight (sum,
// RDKV summary §2.1) or the KVzip+ numerator max_j a_{j,t} ||h_j|| (KVzap summary §2.1).
// Both passes run QK^T on 32x32x16 bf16 matrix cores with fp32 accumulation; logits are
// handled in the base-2 domain (x = s*log2(e) * q.k) so each probability is one exp2.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kThreads = 256;   // 4 waves per block in both passes
constexpr int kPad = 8;         // bf16 elements of padding per LDS row (16 bytes)

template <int D>
__device__ __forceinline__ void load_rows_to_regs(uint4 (&r)[D / 32], const uint16_t* base,
                                                  int64_t row0, int64_t nrows_valid,
                                                  int64_t row_limit) {
  // 64 rows x D bf16 = 64*D/8 chunks of 16 bytes; 256 threads -> D/32 chunks each.
  constexpr int kChunksPerRow = D / 8;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    int chunk = threadIdx.x + j * kThreads;
    int rr = chunk / kChunksPerRow;
    int cc = chunk % kChunksPerRow;
    int64_t row = row0 + rr;
    if (rr < nrows_valid && row < row_limit) {
      r[j] = *reinterpret_cast<const uint4*>(base + row * D + cc * 8);
    } else {
      r[j] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_regs_to_lds(const uint4 (&r)[D / 32], uint16_t* lds) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int RS = D + kPad;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    int chunk = threadIdx.x + j * kThreads;
    int rr = chunk / kChunksPerRow;
    int cc = chunk % kChunksPerRow;
    *reinterpret_cast<uint4*>(lds + rr * RS + cc * 8) = r[j];
  }
}

// ---------------------------------------------------------------------------------------
// Pass 1.  Block = (256 query rows, q head h); wave w owns rows [64w, 64w+64) of the tile.
// K streams through LDS in 64-key tiles (double buffered); Q^T stays in registers.
// D[m = key][n = row]: a lane holds one row and 16 keys per 32x32 block, so the online
// max / sum-exp updates are in-lane plus one exchange with the lane 32 apart.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads)
lse_pass1(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
          float* __restrict__ lse, int G, int64_t N, int64_t Nq, int causal, float c) {
  constexpr int RS = D + kPad;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][64 * RS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const int h = blockIdx.y;
  const int g = h / G;
  const int64_t off = N - Nq;
  const int64_t i_block = (int64_t)blockIdx.x * 256;
  const int64_t i_wave = i_block + 64 * wave;

  const uint16_t* kh = k + (int64_t)g * N * D;

  // Q^T operand for this wave's 64 rows (2 column blocks of 32 rows).
  bf16x8 qb[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    int64_t row = i_wave + 32 * nb + lo;
    bool ok = row < Nq;
    const uint16_t* qp = q + ((int64_t)h * Nq + (ok ? row : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + ks * 16 + 8 * hi) : make_uint4(0, 0, 0, 0);
      qb[nb][ks] = as_bf16x8(v);
    }
  }

  const int64_t last_row_block = (i_block + 256 < Nq ? i_block + 256 : Nq) - 1;
  const int64_t kend = causal ? (off + last_row_block + 1 < N ? off + last_row_block + 1 : N) : N;
  int64_t kend_wave = 0;
  if (i_wave < Nq) {
    int64_t lr = (i_wave + 63 < Nq ? i_wave + 63 : Nq - 1);
    kend_wave = causal ? (off + lr + 1 < N ? off + lr + 1 : N) : N;
  }
  const int ntiles = (int)((kend + 63) / 64);

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  uint4 pre[D / 32];
  load_rows_to_regs<D>(pre, kh, 0, 64, N);
  store_regs_to_lds<D>(pre, kt[0]);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int64_t t0 = (int64_t)j * 64;
    if (j + 1 < ntiles) load_rows_to_regs<D>(pre, kh, t0 + 64, 64, N);
    const uint16_t* kl = kt[j & 1];
    if (t0 < kend_wave) {
      f32x16 acc[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(kl + (mb * 32 + lo) * RS + ks * 16 + 8 * hi));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(a, qb[nb][ks], acc[mb][nb]);
        }
      }
      const bool full = (!causal || t0 + 63 <= off + i_wave) && (t0 + 64 <= N);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int64_t pos = off + i_wave + 32 * nb + lo;
        float x[2][16];
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float v = acc[mb][nb][i] * c;
            if (!full) {
              int64_t t = t0 + 32 * mb + acc_row(i, hi);
              if (t >= N || (causal && t > pos)) v = -INFINITY;
            }
            x[mb][i] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = fmaxf(tmax, swap_half(tmax));
        const float mnew = fmaxf(m_run[nb], tmax);
        if (mnew > -INFINITY) {
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            s0 += fast_exp2(x[0][i] - mnew) + fast_exp2(x[0][i + 1] - mnew);
            s1 += fast_exp2(x[1][i] - mnew) + fast_exp2(x[1][i + 1] - mnew);
          }
          l_run[nb] = l_run[nb] * fast_exp2(m_run[nb] - mnew) + (s0 + s1);
          m_run[nb] = mnew;
        }
      }
    }
    if (j + 1 < ntiles) store_regs_to_lds<D>(pre, kt[(j + 1) & 1]);
    __syncthreads();
  }

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float lt = l_run[nb] + swap_half(l_run[nb]);
    int64_t row = i_wave + 32 * nb + lo;
    if (hi == 0 && row < Nq) {
      float out = (m_run[nb] > -INFINITY) ? (m_run[nb] + log2f(lt)) * kLn2 : -INFINITY;
      lse[(int64_t)h * Nq + row] = out;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Pass 2.  Block = (256-key tile, query-row chunk, KV head g); wave w owns keys
// [t0 + 64w, t0 + 64w + 64) whose K^T operand stays in registers.  The block walks the
// group's query heads and the chunk's rows in 64-row sub-tiles staged through LDS together
// with each row's base-2 offset (lse*log2e, minus log2||h|| in MAX mode).
// D[m = row][n = key]: a lane holds one key and 16 rows per 32x32 block, so the column
// reduction is in-lane plus one exchange with the lane 32 apart.  Each block writes its
// partial column sums (or maxima per query head) to the workspace; a second kernel
// reduces the chunks in a fixed order, so results are bitwise reproducible.
// ---------------------------------------------------------------------------------------
template <int D, bool MAXMODE>
__global__ void __launch_bounds__(kThreads)
score_pass2(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const float* __restrict__ lse, const float* __restrict__ hlog2,
            float* __restrict__ partial, int G, int64_t N, int64_t Nq, int causal, float c,
            int QC, int maxC, int64_t Npad) {
  constexpr int RS = D + kPad;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t qt[2][64 * RS];
  __shared__ float lt[2][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const int tile = blockIdx.x;
  const int chunk = blockIdx.y;
  const int g = blockIdx.z;
  const int64_t off = N - Nq;
  const int64_t t0 = (int64_t)tile * kScoreTileKeys;
  const int64_t kw0 = t0 + 64 * wave;

  int64_t i_first = 0;
  if (causal) {
    int64_t f = t0 - off;
    i_first = f > 0 ? (f & ~int64_t(63)) : 0;
  }
  const int64_t r_begin = i_first + (int64_t)chunk * QC;
  if (r_begin >= Nq) return;   // uniform for the block
  const int64_t r_end = (r_begin + QC < Nq) ? r_begin + QC : Nq;
  const int nsub = (int)((r_end - r_begin + 63) / 64);
  const int total_it = G * nsub;

  // K^T operand: this wave's 64 keys (2 column blocks of 32 keys).
  const uint16_t* kh = k + (int64_t)g * N * D;
  bf16x8 kb[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    int64_t t = kw0 + 32 * nb + lo;
    const uint16_t* kp = kh + (t < N ? t : N - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[nb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kp + ks * 16 + 8 * hi));
  }

  float colacc[2];
  colacc[0] = colacc[1] = MAXMODE ? -INFINITY : 0.f;

  auto row_offset = [&](int hh, int64_t row) -> float {
    if (row >= Nq) return INFINITY;
    float l2 = lse[(int64_t)hh * Nq + row] * kLog2e;
    if (MAXMODE) l2 -= hlog2[row];
    return l2;
  };

  // stage iteration 0
  uint4 pre[D / 32];
  float lpre = 0.f;
  {
    const int hh = g * G;
    load_rows_to_regs<D>(pre, q + (int64_t)hh * Nq * D, r_begin, 64, Nq);
    if (threadIdx.x < 64) lpre = row_offset(hh, r_begin + threadIdx.x);
    store_regs_to_lds<D>(pre, qt[0]);
    if (threadIdx.x < 64) lt[0][threadIdx.x] = lpre;
  }
  __syncthreads();

  for (int it = 0; it < total_it; ++it) {
    const int hl = it / nsub;
    const int sub = it % nsub;
    const int64_t r = r_begin + (int64_t)sub * 64;
    const int buf = it & 1;
    if (it + 1 < total_it) {
      const int hl2 = (it + 1) / nsub;
      const int64_t r2 = r_begin + (int64_t)((it + 1) % nsub) * 64;
      const int hh2 = g * G + hl2;
      load_rows_to_regs<D>(pre, q + (int64_t)hh2 * Nq * D, r2, 64, Nq);
      if (threadIdx.x < 64) lpre = row_offset(hh2, r2 + threadIdx.x);
    }
    const int64_t pp = off + r;       // position of the sub-tile's first row
    const bool any = !causal || kw0 <= pp + 63;
    if (any) {
      const uint16_t* ql = qt[buf];
      f32x16 acc[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(ql + (mb * 32 + lo) * RS + ks * 16 + 8 * hi));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(a, kb[nb][ks], acc[mb][nb]);
        }
      }
      float lv[2][16];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) lv[mb][i] = lt[buf][32 * mb + acc_row(i, hi)];
      const bool full = !causal || kw0 + 63 <= pp;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int64_t t = kw0 + 32 * nb + lo;
        if (MAXMODE) {
          float mx = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float x = fmaf(acc[mb][nb][i], c, -lv[mb][i]);
              if (!full && t > pp + 32 * mb + acc_row(i, hi)) x = -INFINITY;
              mx = fmaxf(mx, x);
            }
          colacc[nb] = fmaxf(colacc[nb], mx);
        } else {
          float s[2];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            float e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float x = fmaf(acc[mb][nb][i], c, -lv[mb][i]);
              if (!full && t > pp + 32 * mb + acc_row(i, hi)) x = -INFINITY;
              e[i] = fast_exp2(x);
            }
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
              for (int i = 0; i < w; ++i) e[i] += e[i + w];
            s[mb] = e[0];
          }
          colacc[nb] += s[0] + s[1];
        }
      }
    }
    if (MAXMODE && sub == nsub - 1) {
      // finished query head hl: write its column maxima
      const int hh = g * G + hl;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float m = fmaxf(colacc[nb], swap_half(colacc[nb]));
        if (hi == 0) partial[((int64_t)hh * maxC + chunk) * Npad + kw0 + 32 * nb + lo] = m;
        colacc[nb] = -INFINITY;
      }
    }
    if (it + 1 < total_it) {
      store_regs_to_lds<D>(pre, qt[buf ^ 1]);
      if (threadIdx.x < 64) lt[buf ^ 1][threadIdx.x] = lpre;
    }
    __syncthreads();
  }

  if (!MAXMODE) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float s = colacc[nb] + swap_half(colacc[nb]);
      if (hi == 0) partial[((int64_t)g * maxC + chunk) * Npad + kw0 + 32 * nb + lo] = s;
    }
  }
}

__device__ __forceinline__ int chunks_of_tile(int64_t t0, int64_t N, int64_t Nq, int causal, int QC) {
  int64_t i_first = 0;
  if (causal) {
    int64_t f = t0 - (N - Nq);
    i_first = f > 0 ? (f & ~int64_t(63)) : 0;
  }
  if (i_first >= Nq) return 0;
  return (int)((Nq - i_first + QC - 1) / QC);
}

// w[g][t] = sum over chunks (ascending) of the partial column sums.
__global__ void score_reduce_sum(const float* __restrict__ partial, float* __restrict__ scores,
                                 int64_t N, int64_t Nq, int causal, int QC, int maxC,
                                 int64_t Npad, int Hkv) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Hkv * N) return;
  int g = (int)(idx / N);
  int64_t t = idx % N;
  int nc = chunks_of_tile((t / kScoreTileKeys) * kScoreTileKeys, N, Nq, causal, QC);
  float s = 0.f;
  for (int ch = 0; ch < nc; ++ch) s += partial[((int64_t)g * maxC + ch) * Npad + t];
  scores[idx] = s;
}

// s+[g][t] = max over the group's heads h of exp2(max over chunks of partial) / ||W_O^h v||.
__global__ void score_reduce_max(const float* __restrict__ partial, const float* __restrict__ won,
                                 float* __restrict__ scores, int64_t N, int64_t Nq, int causal,
                                 int QC, int maxC, int64_t Npad, int Hkv, int G) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Hkv * N) return;
  int g = (int)(idx / N);
  int64_t t = idx % N;
  int nc = chunks_of_tile((t / kScoreTileKeys) * kScoreTileKeys, N, Nq, causal, QC);
  float best = 0.f;
  for (int hl = 0; hl < G; ++hl) {
    int hh = g * G + hl;
    float m = -INFINITY;
    for (int ch = 0; ch < nc; ++ch) m = fmaxf(m, partial[((int64_t)hh * maxC + ch) * Npad + t]);
    float num = exp2f(m);
    float den = won[(int64_t)hh * N + t];
    float r = (num == 0.f && den == 0.f) ? 0.f : num / den;
    best = fmaxf(best, r);
  }
  scores[idx] = best;
}

// log2 ||h_j||_2 per query row (float64 accumulation of the squares).
__global__ void __launch_bounds__(256)
hidden_log2_norm(const uint16_t* __restrict__ hidden, float* __restrict__ hlog2, int Dh) {
  const int64_t row = blockIdx.x;
  const uint16_t* hp = hidden + row * Dh;
  double ss = 0.0;
  for (int i = threadIdx.x; i < Dh; i += blockDim.x) {
    double v = (double)bf16_bits_to_f32(hp[i]);
    ss += v * v;
  }
  __shared__ double red[256];
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) hlog2[row] = (float)(0.5 * log2(red[0]));
}

// Partial Gram matrices of each head's W_O slice: gp[h][s][c1][c2] = sum over rows r of
// split s of W[r][h*d + c1] * W[r][h*d + c2]  (products of bf16 are exact in fp32).
template <int D>
__global__ void __launch_bounds__(256)
wo_gram_partial(const uint16_t* __restrict__ w_o, float* __restrict__ gp, int Hq, int Dh,
                int rows_per_split) {
  constexpr int RB = 32;   // rows staged per step
  __shared__ float ws[RB][D + 1];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int r0 = s * rows_per_split;
  const int r1 = (r0 + rows_per_split < Dh) ? r0 + rows_per_split : Dh;
  constexpr int T = D / 16;     // entries per thread per dimension
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float acc[T][T];
#pragma unroll
  for (int a = 0; a < T; ++a)
#pragma unroll
    for (int b = 0; b < T; ++b) acc[a][b] = 0.f;
  const int64_t ld = (int64_t)Hq * D;
  for (int rb = r0; rb < r1; rb += RB) {
    __syncthreads();
    for (int e = threadIdx.x; e < RB * D; e += 256) {
      int rr = e / D, cc = e % D;
      int r = rb + rr;
      ws[rr][cc] = (r < r1) ? bf16_bits_to_f32(w_o[(int64_t)r * ld + (int64_t)h * D + cc]) : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < RB; ++rr) {
      float x[T], y[T];
#pragma unroll
      for (int a = 0; a < T; ++a) x[a] = ws[rr][ty * T + a];
#pragma unroll
      for (int b = 0; b < T; ++b) y[b] = ws[rr][tx * T + b];
#pragma unroll
      for (int a = 0; a < T; ++a)
#pragma unroll
        for (int b = 0; b < T; ++b) acc[a][b] = fmaf(x[a], y[b], acc[a][b]);
    }
  }
  float* out = gp + ((int64_t)h * gridDim.y + s) * D * D;
#pragma unroll
  for (int a = 0; a < T; ++a)
#pragma unroll
    for (int b = 0; b < T; ++b) out[(ty * T + a) * D + tx * T + b] = acc[a][b];
}

// Sum the Gram partials over splits in order: gram[h] = sum_s gp[h][s].
__global__ void wo_gram_reduce(const float* __restrict__ gp, float* __restrict__ gram, int Hq,
                               int splits, int DD) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Hq * DD) return;
  int h = (int)(idx / DD);
  int e = (int)(idx % DD);
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += gp[((int64_t)h * splits + sp) * DD + e];
  gram[idx] = s;
}

// ||W_O^h v_t||_2 = sqrt(v_t^T (W_O^h^T W_O^h) v_t): one token per thread, the Gram matrix of
// head h in LDS (every lane reads the same entry: broadcast).
template <int D>
__global__ void __launch_bounds__(256)
value_out_norm(const uint16_t* __restrict__ v, const float* __restrict__ gram,
               float* __restrict__ won, int G, int64_t N) {
  __shared__ float gm[D * D];
  const int h = blockIdx.y;
  const int g = h / G;
  for (int e = threadIdx.x; e < D * D; e += 256) gm[e] = gram[(int64_t)h * D * D + e];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N) return;
  const uint16_t* vp = v + ((int64_t)g * N + t) * D;
  float x[D];
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) {
    uint4 w = *reinterpret_cast<const uint4*>(vp + c8 * 8);
    uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[c8 * 8 + 2 * j] = bf16_bits_to_f32(ww[j] & 0xFFFFu);
      x[c8 * 8 + 2 * j + 1] = bf16_bits_to_f32(ww[j] >> 16);
    }
  }
  float qf = 0.f;
  for (int c1 = 0; c1 < D; ++c1) {
    float y = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < D; ++c2) y = fmaf(gm[c1 * D + c2], x[c2], y);
    qf = fmaf(x[c1], y, qf);
  }
  won[(int64_t)h * N + t] = sqrtf(fmaxf(qf, 0.f));
}

}  // namespace

int score_chunk_rows(const Layer& L) {
  // Split a tile's query rows so that no tile has more than 16 chunks; at least 256 rows.
  int64_t rows = (L.nq + 15) / 16;
  int64_t qc = ((rows + 255) / 256) * 256;
  if (qc < 256) qc = 256;
  return (int)qc;
}

int score_max_chunks(const Layer& L) {
  int QC = score_chunk_rows(L);
  return (int)((L.nq + QC - 1) / QC);
}

static int64_t npad_of(const Layer& L) {
  return ((L.n + kScoreTileKeys - 1) / kScoreTileKeys) * kScoreTileKeys;
}

static constexpr int kGramSplits = 14;

size_t score_ws_bytes(const Layer& L, int mode, int hidden_dim) {
  (void)hidden_dim;
  WsPlan p;
  int64_t units = (mode == KVC_SCORE_MAX) ? L.hq : L.hkv;
  p.take((size_t)units * score_max_chunks(L) * npad_of(L) * sizeof(float));
  if (mode == KVC_SCORE_MAX) {
    p.take((size_t)L.nq * sizeof(float));                                  // log2 ||h||
    p.take((size_t)L.hq * kGramSplits * L.d * L.d * sizeof(float));        // gram partials
    p.take((size_t)L.hq * L.d * L.d * sizeof(float));                      // gram
    p.take((size_t)L.hq * L.n * sizeof(float));                            // ||W_O^h v||
  }
  return p.off;
}

hipError_t launch_row_lse(const Layer& L, const uint16_t* q, const uint16_t* k, float* lse,
                          hipStream_t s) {
  dim3 grid((unsigned)((L.nq + 255) / 256), (unsigned)L.hq);
  if (L.d == 128)
    lse_pass1<128><<<grid, kThreads, 0, s>>>(q, k, lse, L.G, L.n, L.nq, L.causal, L.c_log2);
  else
    lse_pass1<64><<<grid, kThreads, 0, s>>>(q, k, lse, L.G, L.n, L.nq, L.causal, L.c_log2);
  return hipGetLastError();
}

hipError_t launch_score(const Layer& L, int mode, const uint16_t* q, const uint16_t* k,
                        const float* lse, const uint16_t* hidden, const uint16_t* w_o,
                        const uint16_t* v, int hidden_dim, float* scores, char* ws,
                        hipStream_t s) {
  const int QC = score_chunk_rows(L);
  const int maxC = score_max_chunks(L);
  const int64_t Npad = npad_of(L);
  const int ntiles = (int)(Npad / kScoreTileKeys);
  WsPlan p;
  const bool mx = (mode == KVC_SCORE_MAX);
  int64_t units = mx ? L.hq : L.hkv;
  float* partial = reinterpret_cast<float*>(ws + p.take((size_t)units * maxC * Npad * sizeof(float)));
  float* hlog2 = nullptr;
  float* won = nullptr;
  if (mx) {
    hlog2 = reinterpret_cast<float*>(ws + p.take((size_t)L.nq * sizeof(float)));
    float* gp = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * kGramSplits * L.d * L.d * sizeof(float)));
    float* gram = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * L.d * L.d * sizeof(float)));
    won = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * L.n * sizeof(float)));
    hidden_log2_norm<<<(unsigned)L.nq, 256, 0, s>>>(hidden, hlog2, hidden_dim);
    int rps = (hidden_dim + kGramSplits - 1) / kGramSplits;
    dim3 gg((unsigned)L.hq, kGramSplits);
    if (L.d == 128)
      wo_gram_partial<128><<<gg, 256, 0, s>>>(w_o, gp, L.hq, hidden_dim, rps);
    else
      wo_gram_partial<64><<<gg, 256, 0, s>>>(w_o, gp, L.hq, hidden_dim, rps);
    int64_t ng = (int64_t)L.hq * L.d * L.d;
    wo_gram_reduce<<<(unsigned)((ng + 255) / 256), 256, 0, s>>>(gp, gram, L.hq, kGramSplits, L.d * L.d);
    dim3 gv((unsigned)((L.n + 255) / 256), (unsigned)L.hq);
    if (L.d == 128)
      value_out_norm<128><<<gv, 256, 0, s>>>(v, gram, won, L.G, L.n);
    else
      value_out_norm<64><<<gv, 256, 0, s>>>(v, gram, won, L.G, L.n);
  }
  dim3 grid((unsigned)ntiles, (unsigned)maxC, (unsigned)L.hkv);
  if (L.d == 128) {
    if (mx)
      score_pass2<128, true><<<grid, kThreads, 0, s>>>(q, k, lse, hlog2, partial, L.G, L.n, L.nq, L.causal, L.c_log2, QC, maxC, Npad);
    else
      score_pass2<128, false><<<grid, kThreads, 0, s>>>(q, k, lse, nullptr, partial, L.G, L.n, L.nq, L.causal, L.c_log2, QC, maxC, Npad);
  } else {
    if (mx)
      score_pass2<64, true><<<grid, kThreads, 0, s>>>(q, k, lse, hlog2, partial, L.G, L.n, L.nq, L.causal, L.c_log2, QC, maxC, Npad);
    else
      score_pass2<64, false><<<grid, kThreads, 0, s>>>(q, k, lse, nullptr, partial, L.G, L.n, L.nq, L.causal, L.c_log2, QC, maxC, Npad);
  }
  int64_t total = (int64_t)L.hkv * L.n;
  unsigned rb = (unsigned)((total + 255) / 256);
  if (mx)
    score_reduce_max<<<rb, 256, 0, s>>>(partial, won, scores, L.n, L.nq, L.causal, QC, maxC, Npad, L.hkv, L.G);
  else
    score_reduce_sum<<<rb, 256, 0, s>>>(partial, scores, L.n, L.nq, L.causal, QC, maxC, Npad, L.hkv);
  return hipGetLastError();
}

}  // namespace kvc
