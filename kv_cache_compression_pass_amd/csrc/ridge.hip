// KVSculpt's value solve (KVSculpt summary §2, value step; §4 "Select+Fit"): with the
// compressed keys fixed, the values V_c that minimise ||A_c V_c + A_r V_r - Y||_F^2 +
// lambda ||V_c||_F^2 solve (A_c^T A_c + lambda I) V_c = A_c^T (Y - A_r V_r).  The rows of the
// G query heads of a KV head are stacked (they share the head's V_c).
//
// Kernels, one stream, per KV head g (R = G * Nq stacked rows, n = n_c + m keys):
//   row LSE        the scorer's pass 1 over the n keys                          (score.hip)
//   ridge_probs    P[r][t] = exp(s q_r . k_t - l_r), fp32, 64 x 64 tiles, bf16 matrix-core products
//   ridge_resid    T = Y - P_r V_r (fp32), 64 x 64 tiles over (rows, channels), bf16 matrix cores
//   ridge_gram     M = P_c^T P_c and B = P_c^T T on the fp64 matrix cores (each product of two
//                  fp32 values is exact in fp64), the row sum split in kSplit fixed parts
//   ridge_sum      M += lambda I (identity on the padding), the parts added in fixed order
//   ridge_chol     blocked Cholesky (32-wide blocks), one launch per block column kb: every tile
//                  (i, j) of the trailing matrix computes L_ik = A_ik L_kk^-T itself, subtracts
//                  L_ik L_jk^T, and the tile (kb+1, kb+1) then factors itself and inverts its L
//                  (look-ahead); in the same launch the forward solve moves one block: Y_k =
//                  L_kk^-1 B_k, and B_i -= L_ik Y_k for every i > k
//   ridge_back2    the backward solve, one launch per pair of block rows from the last: X_k =
//                  L_kk^-T Y_k, then the row above and its X_{k-1}, then Y_i -= L_ki^T X_k +
//                  L_{k-1},i^T X_{k-1} for every i < k - 1; the X rows are V_c's rows
//                  (ridge_back takes a lone row 0 when the number of block rows is odd)
// Every sum has a fixed order, so results are deterministic.  The matrix is padded to a
// multiple of 64 with an identity block, which leaves the solution unchanged.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kT = 64;          // tile edge of the probability, residual and Gram kernels
constexpr int kNB = 32;         // block edge of the Cholesky factorisation and the solves
constexpr int kSplit = 5;       // parts of the row sum in the Gram products

struct RidgeDims {
  int hq, hkv, d, G, causal;
  int64_t n, nq, nc, m, R, npad;
  int nt;         // 64-wide tiles of npad (Gram)
  int nb;         // 32-wide blocks of npad (Cholesky, solves)
};

RidgeDims dims_of(const Layer& L, int64_t nc) {
  RidgeDims r{};
  r.hq = L.hq;
  r.hkv = L.hkv;
  r.d = L.d;
  r.G = L.G;
  r.causal = L.causal;
  r.n = L.n;
  r.nq = L.nq;
  r.nc = nc;
  r.m = L.n - nc;
  r.R = (int64_t)L.G * L.nq;
  r.npad = (nc + kT - 1) / kT * kT;
  r.nt = (int)(r.npad / kT);
  r.nb = (int)(r.npad / kNB);
  return r;
}

struct RidgeWs {
  char* lse_ws;   // the row-LSE kernels' own scratch
  float* lse;     // [Hq][Nq]
  float* P;       // [Hkv][R][n]
  float* T;       // [Hkv][R][d]
  double* Mp;     // [kSplit][Hkv][npad][npad]  (lower tiles)
  double* Bp;     // [kSplit][Hkv][npad][d]
  double* M;      // [Hkv][npad][npad]          (lower tiles; updated in place)
  double* Lm;     // [Hkv][npad][npad]          (lower tiles of L)
  double* Li;     // [Hkv][nb][32][32]          inverse of each diagonal block of L
  double* Bm;     // [Hkv][npad][d]             right side, updated by the forward solve
  double* Yf;     // [Hkv][npad][d]             forward result, updated by the backward solve
};

RidgeWs carve(const Layer& L, const RidgeDims& r, char* ws, size_t* total) {
  WsPlan p;
  const size_t o_lse_ws = p.take(lse_ws_bytes(L));
  const size_t o_lse = p.take(sizeof(float) * r.hq * r.nq);
  const size_t o_P = p.take(sizeof(float) * r.hkv * r.R * r.n);
  const size_t o_T = p.take(sizeof(float) * r.hkv * r.R * r.d);
  const size_t o_Mp = p.take(sizeof(double) * kSplit * r.hkv * r.npad * r.npad);
  const size_t o_Bp = p.take(sizeof(double) * kSplit * r.hkv * r.npad * r.d);
  const size_t o_M = p.take(sizeof(double) * r.hkv * r.npad * r.npad);
  const size_t o_L = p.take(sizeof(double) * r.hkv * r.npad * r.npad);
  const size_t o_Li = p.take(sizeof(double) * r.hkv * r.nb * kNB * kNB);
  const size_t o_Bm = p.take(sizeof(double) * r.hkv * r.npad * r.d);
  const size_t o_Y = p.take(sizeof(double) * r.hkv * r.npad * r.d);
  if (total) *total = p.off;
  RidgeWs w{};
  if (ws) {
    w.lse_ws = ws + o_lse_ws;
    w.lse = reinterpret_cast<float*>(ws + o_lse);
    w.P = reinterpret_cast<float*>(ws + o_P);
    w.T = reinterpret_cast<float*>(ws + o_T);
    w.Mp = reinterpret_cast<double*>(ws + o_Mp);
    w.Bp = reinterpret_cast<double*>(ws + o_Bp);
    w.M = reinterpret_cast<double*>(ws + o_M);
    w.Lm = reinterpret_cast<double*>(ws + o_L);
    w.Li = reinterpret_cast<double*>(ws + o_Li);
    w.Bm = reinterpret_cast<double*>(ws + o_Bm);
    w.Yf = reinterpret_cast<double*>(ws + o_Y);
  }
  return w;
}


// A[r][t] = exp(s q_r . k_t - l_r) on the bf16 matrix cores (each product exact, fp32 sums,
// like the scorer's pass 1).  Block = 64 rows x 64 keys; wave w takes the 32 x 32 quarter
// (w / 2, w % 2) with the query rows as the A operand and the keys as the B operand, so a
// lane's accumulator holds one key column of 16 rows and the 32 lanes of a row store 32
// consecutive keys.  The rows' LSE (base 2) and last visible key are laid out once in LDS.
template <int D>
__global__ void __launch_bounds__(256)
ridge_probs(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ lse,
            float* __restrict__ P, RidgeDims r, float c_log2) {
  constexpr int KS = D / 16;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float l2s[kT];
  __shared__ int64_t lasts[kT];
  const int g = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t r0 = (int64_t)blockIdx.y * kT;
  if (threadIdx.x < kT) {
    const int64_t rr = r0 + threadIdx.x;
    float l2 = -__builtin_inff();
    int64_t last = -1;
    if (rr < r.R) {
      const int64_t h = (int64_t)g * r.G + rr / r.nq, qi = rr % r.nq;
      const float l = lse[h * r.nq + qi];
      if (l > -__builtin_inff()) {
        l2 = l * kLog2e;
        last = r.causal ? r.n - r.nq + qi : r.n - 1;      // last visible key
      }
    }
    l2s[threadIdx.x] = l2;
    lasts[threadIdx.x] = last;
  }
  const int rw = (wave >> 1) * 32;                          // the wave's rows and keys in the tile
  const int64_t tcol = (int64_t)blockIdx.x * kT + (wave & 1) * 32 + lo;   // this lane's key
  const int64_t rr = r0 + rw + lo;                          // this lane's A-operand row
  const uint16_t* qp = nullptr;
  if (rr < r.R) {
    const int64_t h = (int64_t)g * r.G + rr / r.nq, qi = rr % r.nq;
    qp = q + (h * r.nq + qi) * D;
  }
  const uint16_t* kp = tcol < r.n ? k + ((int64_t)g * r.n + tcol) * D : nullptr;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 a = qp ? *reinterpret_cast<const uint4*>(qp + ks * 16 + 8 * hi) : make_uint4(0, 0, 0, 0);
    const uint4 b = kp ? *reinterpret_cast<const uint4*>(kp + ks * 16 + 8 * hi) : make_uint4(0, 0, 0, 0);
    acc = mfma32(as_bf16x8(a), as_bf16x8(b), acc);
  }
  __syncthreads();
  if (tcol >= r.n) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rl = rw + acc_row(i, hi);
    const int64_t row = r0 + rl;
    if (row >= r.R) continue;
    const bool vis = tcol <= lasts[rl];
    P[((int64_t)g * r.R + row) * r.n + tcol] = vis ? exp2f(fmaf(acc[i], c_log2, -l2s[rl])) : 0.f;
  }
}

// T = Y - A_r V_r (fp32) on the bf16 matrix cores: A_r's fp32 weights enter as a bf16 hi + lo
// pair (exact to about 2^-17 of each weight) and V_r is bf16, so each product pair is exact and
// the sums are fp32.  Block = 64 rows x 64 channels; wave w takes the 32 x 32 quarter (w / 2,
// w % 2).  Per chunk of 64 retained keys the block stages V_r^T in LDS (channel-major, so a
// lane's 8 consecutive keys are one 16-byte read) from registers loaded during the previous
// chunk; a lane's weights of the chunk are requested before the chunk's barriers.
template <int D>
__global__ void __launch_bounds__(256)
ridge_resid(const float* __restrict__ P, const uint16_t* __restrict__ v_r, const float* __restrict__ y,
            float* __restrict__ T, RidgeDims r) {
  __shared__ __attribute__((aligned(16))) uint16_t vT[kT][kT + 8];   // [channel][key]
  const int g = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t r0 = (int64_t)blockIdx.y * kT;
  const int c0 = blockIdx.x * kT;
  const int rw = (wave >> 1) * 32, cw = (wave & 1) * 32;
  const int64_t arow = r0 + rw + lo;                        // this lane's A-operand row
  const float* prow = arow < r.R ? P + ((int64_t)g * r.R + arow) * r.n + r.nc : nullptr;
  f32x16 acc, acc_lo;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = acc_lo[i] = 0.f;
  // V_r of the next chunk waits in registers while the current one is multiplied
  constexpr int kVPer = kT * kT / 256;                      // 16 values per thread
  uint16_t vn[kVPer];
  auto load_v = [&](int64_t s0) {
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int e = threadIdx.x + 256 * u;                  // V_r rows: consecutive threads, channels
      const int64_t tt = s0 + e / kT;
      vn[u] = tt < r.m ? v_r[((int64_t)g * r.m + tt) * D + c0 + e % kT] : (uint16_t)0;
    }
  };
  load_v(0);
  for (int64_t s0 = 0; s0 < r.m; s0 += kT) {
    float pv[kT / 16][8];                                   // this lane's weights of the chunk
#pragma unroll
    for (int ks = 0; ks < kT / 16; ++ks) {
      const int64_t t0 = s0 + ks * 16 + 8 * hi;
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[ks][u] = (prow && t0 + u < r.m) ? prow[t0 + u] : 0.f;
    }
    __syncthreads();                                        // the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int e = threadIdx.x + 256 * u;
      vT[e % kT][e / kT] = vn[u];
    }
    if (s0 + kT < r.m) load_v(s0 + kT);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kT / 16; ++ks) {
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float p0 = pv[ks][2 * u], p1 = pv[ks][2 * u + 1];
        const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
        const __bf16 l0 = (__bf16)(p0 - (float)h0), l1 = (__bf16)(p1 - (float)h1);
        ph[u] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        pl[u] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(&vT[cw + lo][ks * 16 + 8 * hi]));
      acc = mfma32(as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3])), b, acc);
      acc_lo = mfma32(as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3])), b, acc_lo);
    }
  }
  // acc[i]: row rw + acc_row(i, hi), channel cw + lo
  const int ch = c0 + cw + lo;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t rr = r0 + rw + acc_row(i, hi);
    if (rr >= r.R) continue;
    const int64_t h = (int64_t)g * r.G + rr / r.nq, qi = rr % r.nq;
    T[((int64_t)g * r.R + rr) * D + ch] = y[(h * r.nq + qi) * D + ch] - (acc[i] + acc_lo[i]);
  }
}

// Gram products over the rows of part s: tile (a-tile, b-tile) of M = P_c^T P_c (lower tiles),
// or tile (a-tile, channel tile) of B = P_c^T T.  fp32 inputs staged in LDS as fp64, products and
// sums on the fp64 matrix cores (v_mfma_f64_16x16x4f64: A[i][k] from lane i + 16k, B[k][j] from
// lane j + 16k, D[i][j] in lane j + 16 (i % 4), register i / 4).  Wave w owns the 16 tile rows
// 16w .. 16w+15 and all 64 columns (four 16 x 16 accumulators); each step of 4 staged rows is
// one A fragment, four B fragments and four MFMAs per wave, in a fixed order.  Four waves per
// SIMD (at most 128 registers: the step loop is unrolled twice, not eight times) and five row
// parts make about four blocks per compute unit, so the whole grid runs in one round.
typedef double v4d __attribute__((ext_vector_type(4)));

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
ridge_gram(const float* __restrict__ P, const float* __restrict__ T, double* __restrict__ Mp,
           double* __restrict__ Bp, RidgeDims r) {
  __shared__ double xs[32][kT + 1];
  __shared__ double zs[32][kT + 1];
  const int s = blockIdx.y, g = blockIdx.z;
  const int nt = r.nt;
  const int nlow = nt * (nt + 1) / 2;
  int tile = blockIdx.x;
  bool isB;
  int ia, ib;
  if (tile < nlow) {
    isB = false;
    ia = 0;
    while ((ia + 1) * (ia + 2) / 2 <= tile) ++ia;      // tile = ia (ia + 1) / 2 + ib
    ib = tile - ia * (ia + 1) / 2;
  } else {
    isB = true;
    tile -= nlow;
    ia = tile / (D / kT);
    ib = tile % (D / kT);
  }
  const int64_t a0 = (int64_t)ia * kT, b0 = (int64_t)ib * kT;
  const int64_t rs = (r.R + kSplit - 1) / kSplit;
  const int64_t rbeg = s * rs, rend = (s + 1) * rs < r.R ? (s + 1) * rs : r.R;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  v4d acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = (v4d){0.0, 0.0, 0.0, 0.0};
  const float* Pg = P + (int64_t)g * r.R * r.n;
  const float* Tg = T + (int64_t)g * r.R * D;
  // the next chunk's values are loaded into registers while the matrix cores work on this one
  constexpr int kPer = 32 * kT / 256;               // values per thread per chunk and array
  float px[kPer], pz[kPer];
  auto fetch = [&](int64_t q0) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      const int rr = e / kT, col = e % kT;
      const int64_t row = q0 + rr;
      const bool rv = row < rend;
      const int64_t a = a0 + col, b = b0 + col;
      px[u] = (rv && a < r.nc) ? Pg[row * r.n + a] : 0.f;
      pz[u] = rv ? (isB ? Tg[row * D + b] : (b < r.nc ? Pg[row * r.n + b] : 0.f)) : 0.f;
    }
  };
  if (rbeg < rend) fetch(rbeg);
  for (int64_t q0 = rbeg; q0 < rend; q0 += 32) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + 256 * u;
      xs[e / kT][e % kT] = (double)px[u];
      zs[e / kT][e % kT] = (double)pz[u];
    }
    __syncthreads();
    if (q0 + 32 < rend) fetch(q0 + 32);
#pragma unroll 2
    for (int k0 = 0; k0 < 32; k0 += 4) {
      const double av = xs[k0 + lk][16 * w + li];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double bv = zs[k0 + lk][16 * q + li];
        acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[q], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  double* dst;
  int64_t ld;
  if (!isB) {
    dst = Mp + ((int64_t)s * r.hkv + g) * r.npad * r.npad + a0 * r.npad + b0;
    ld = r.npad;
  } else {
    dst = Bp + ((int64_t)s * r.hkv + g) * r.npad * D + a0 * D + b0;
    ld = D;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int reg = 0; reg < 4; ++reg) {
      const int i = 16 * w + 4 * reg + lk, j = 16 * q + li;
      dst[(int64_t)i * ld + j] = acc[q][reg];
    }
}

// M = sum of the parts + lambda I (1 on the padded diagonal) over the lower tiles; B likewise.
__global__ void __launch_bounds__(256)
ridge_sum(const double* __restrict__ Mp, const double* __restrict__ Bp, double* __restrict__ M,
          double* __restrict__ Bm, RidgeDims r, double lambda) {
  const int g = blockIdx.y;
  const int64_t nn = r.npad * r.npad, nbm = r.npad * r.d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < nn + nbm; e += (int64_t)gridDim.x * 256) {
    if (e < nn) {
      const int64_t a = e / r.npad, b = e % r.npad;
      if (b / kT > a / kT) continue;                     // upper tiles: never read
      double v = 0.0;
      for (int s = 0; s < kSplit; ++s) v += Mp[((int64_t)s * r.hkv + g) * nn + e];
      if (a == b) v += a < r.nc ? lambda : 1.0;
      M[(int64_t)g * nn + e] = v;
    } else {
      const int64_t f = e - nn;
      double v = 0.0;
      for (int s = 0; s < kSplit; ++s) v += Bp[((int64_t)s * r.hkv + g) * nbm + f];
      Bm[(int64_t)g * nbm + f] = v;
    }
  }
}

// 1 / sqrt(a): the hardware estimate and two Newton steps y <- y (3 - a y^2) / 2.
__device__ __forceinline__ double rsqrt_newton(double a) {
  const double h = 0.5 * a;
  double y = __builtin_amdgcn_rsq(a);
  y = y * fma(-h * y, y, 1.5);
  y = y * fma(-h * y, y, 1.5);
  return y;
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Step J of the factorisation below (a template, so that every register index is a constant).
template <int J>
__device__ __forceinline__ void potrf_step(double (&r)[kNB], double& rd, bool& bad, double (*B)[kNB], int row,
                                           bool fac) {
  const double m = r[J] * rd;
  r[J] = m;
  if constexpr (J + 1 < kNB) {
    if (fac) B[J][row] = m;                                       // L(row, J), read back as L(e, J)
    const double piv = readlane_f64(fma(-m, m, r[J + 1]), J + 1); // lane J+1: a_{J+1,J+1} - L(J+1, J)^2
    __builtin_amdgcn_wave_barrier();
    constexpr int e0 = ((J + 1) & 1) ? J + 2 : J + 1;
    constexpr int np = (kNB - e0) / 2;
    double b1 = 0.0;
    if constexpr ((J + 1) & 1) b1 = B[J][J + 1];
    double2 b[np > 0 ? np : 1];
#pragma unroll
    for (int p = 0; p < np; ++p) b[p] = *reinterpret_cast<const double2*>(&B[J][e0 + 2 * p]);
    bad |= !(piv > 0.0);
    rd = rsqrt_newton(piv);
    if constexpr ((J + 1) & 1) r[J + 1] = fma(-m, b1, r[J + 1]);
#pragma unroll
    for (int p = 0; p < np; ++p) {
      r[e0 + 2 * p] = fma(-m, b[p].x, r[e0 + 2 * p]);
      r[e0 + 2 * p + 1] = fma(-m, b[p].y, r[e0 + 2 * p + 1]);
    }
#pragma unroll
    for (int e = J + 1; e < kNB; ++e) asm volatile("" : "+v"(r[e]));
    potrf_step<J + 1>(r, rd, bad, B, row, fac);
  }
}

// Cholesky of the 32 x 32 tile in LDS (lower part) and the inverse of its factor, by the first
// wave of the block alone, with every row in registers (no block barrier in the 32 steps).
// Lane i < 32 holds row i of A; lane 32 + c holds column c of the identity, which becomes column
// c of L^-1 (the elimination form L X = I: row j of X is row j of the reduced right side over
// L_jj, then every later row drops L_ej times it).  Step j: with rd_j = 1 / sqrt(pivot_j), every
// lane scales its element j by rd_j (lane i: L(i, j); lane 32 + c: L^-1(j, c)) and subtracts that
// element times L(e, j) from its elements e > j.  The column L(., j) is passed through LDS (one
// row of B per step).  The next pivot, lane j+1's element j+1 after the update, is formed by lane
// j+1 from its own element j and read with readlane, so the chain of pivots never waits on LDS.
// Elements above the diagonal of A's rows end with values nobody reads; the elements of the
// inverse's columns above the diagonal keep their zeros (their multipliers are zeros of L^-1).
// Writes L (lower, zeros above) to Ld (row stride ld) and L^-1 to Li (32 x 32).  A pivot that
// is not positive sets the status bit.  The caller has written the tile and passed a barrier;
// B is 31 x 32 doubles of LDS with 16-byte aligned rows.
__device__ __forceinline__ void potrf_tile(const double (*A)[kNB + 1], double (*B)[kNB], double* __restrict__ Ld,
                                           int64_t ld, double* __restrict__ Li, int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 31;
  const bool fac = lane < 32;
  double r[kNB];
#pragma unroll
  for (int e = 0; e < kNB; ++e) {
    const double a = A[row][e];
    r[e] = fac ? a : (e == row ? 1.0 : 0.0);
  }
  const double piv = readlane_f64(r[0], 0);
  bool bad = !(piv > 0.0);
  double rd = rsqrt_newton(piv);
  potrf_step<0>(r, rd, bad, B, row, fac);
  if (bad && lane == 0) atomicOr(status, KVC_DEV_NOT_SPD);
  if (fac) {
#pragma unroll
    for (int c = 0; c < kNB; ++c) Ld[row * ld + c] = c <= row ? r[c] : 0.0;
  } else {
#pragma unroll
    for (int i = 0; i < kNB; ++i) Li[i * kNB + row] = i >= row ? r[i] : 0.0;
  }
}

// 32 x 32 products with 256 threads as 16 x 16, each 2 x 2 outputs:
//   mm_abT: C[r][c] = sum_p A[r][p] B[c][p];   mm_ab: C[r][c] = sum_p A[r][p] B[p][c];
//   mm_aTb: C[r][c] = sum_p A[p][r] B[p][c].
typedef double Tile[kNB][kNB + 1];
__device__ __forceinline__ void mm_abT(const Tile& A, const Tile& B, double (&c)[2][2]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll 8
  for (int p = 0; p < kNB; ++p) {
    const double a0 = A[2 * ty][p], a1 = A[2 * ty + 1][p], b0 = B[2 * tx][p], b1 = B[2 * tx + 1][p];
    c[0][0] = fma(a0, b0, c[0][0]);
    c[0][1] = fma(a0, b1, c[0][1]);
    c[1][0] = fma(a1, b0, c[1][0]);
    c[1][1] = fma(a1, b1, c[1][1]);
  }
}
__device__ __forceinline__ void mm_ab(const Tile& A, const Tile& B, double (&c)[2][2]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll 8
  for (int p = 0; p < kNB; ++p) {
    const double a0 = A[2 * ty][p], a1 = A[2 * ty + 1][p], b0 = B[p][2 * tx], b1 = B[p][2 * tx + 1];
    c[0][0] = fma(a0, b0, c[0][0]);
    c[0][1] = fma(a0, b1, c[0][1]);
    c[1][0] = fma(a1, b0, c[1][0]);
    c[1][1] = fma(a1, b1, c[1][1]);
  }
}
__device__ __forceinline__ void mm_aTb(const Tile& A, const Tile& B, double (&c)[2][2]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll 8
  for (int p = 0; p < kNB; ++p) {
    const double a0 = A[p][2 * ty], a1 = A[p][2 * ty + 1], b0 = B[p][2 * tx], b1 = B[p][2 * tx + 1];
    c[0][0] = fma(a0, b0, c[0][0]);
    c[0][1] = fma(a0, b1, c[0][1]);
    c[1][0] = fma(a1, b0, c[1][0]);
    c[1][1] = fma(a1, b1, c[1][1]);
  }
}
__device__ __forceinline__ void tile_load(Tile& T, const double* __restrict__ src, int64_t ld) {
  for (int e = threadIdx.x; e < kNB * kNB; e += 256) T[e / kNB][e % kNB] = src[(e / kNB) * ld + e % kNB];
}
__device__ __forceinline__ void tile_put(Tile& T, const double (&c)[2][2]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  T[2 * ty][2 * tx] = c[0][0];
  T[2 * ty][2 * tx + 1] = c[0][1];
  T[2 * ty + 1][2 * tx] = c[1][0];
  T[2 * ty + 1][2 * tx + 1] = c[1][1];
}
__device__ __forceinline__ void zero2(double (&c)[2][2]) { c[0][0] = c[0][1] = c[1][0] = c[1][1] = 0.0; }

// One block column kb of the blocked Cholesky and one block of the forward solve (kb = -1:
// factor tile (0, 0) only).  Blocks [0, ntile) cover the trailing tiles (ib, jb),
// kb < jb <= ib < nb; the next blocks the right-side tiles (ib, column block cb), ib > kb.
__global__ void __launch_bounds__(256)
ridge_chol(double* __restrict__ M, double* __restrict__ Lm, double* __restrict__ Li, double* __restrict__ Bm,
           double* __restrict__ Yf, RidgeDims r, int kb, int32_t* __restrict__ status) {
  __shared__ Tile Ls, Xj, Xk;
  __shared__ __attribute__((aligned(16))) Tile Xi;                // also the factorisation's column rows
  double (*const Bc)[kNB] = reinterpret_cast<double (*)[kNB]>(&Xi[0][0]);
  const int g = blockIdx.y;
  const int64_t np = r.npad, D = r.d;
  double* Mg = M + (int64_t)g * np * np;
  double* Lg = Lm + (int64_t)g * np * np;
  double* Lig = Li + (int64_t)g * r.nb * kNB * kNB;
  if (kb < 0) {
    tile_load(Ls, Mg, np);
    __syncthreads();
    if (threadIdx.x < 64) potrf_tile(Ls, Bc, Lg, np, Lig, status);
    return;
  }
  const int rem = r.nb - 1 - kb;
  const int ntile = rem * (rem + 1) / 2;
  const int64_t k0 = (int64_t)kb * kNB;
  double c[2][2];
  tile_load(Ls, Lig + k0 * kNB, kNB);                             // L_kk^-1
  if ((int)blockIdx.x >= ntile) {
    // forward solve: Y_k = L_kk^-1 B_k, B_ib -= L_ib,k Y_k
    const int t = blockIdx.x - ntile;
    const int ib = kb + 1 + t / (int)(D / kNB), cb = t % (int)(D / kNB);
    double* Bg = Bm + (int64_t)g * np * D;
    tile_load(Xj, Mg + (int64_t)ib * kNB * np + k0, np);          // A_ib,k
    tile_load(Xi, Bg + k0 * D + (int64_t)cb * kNB, D);            // B_k
    __syncthreads();
    zero2(c);
    mm_ab(Ls, Xi, c);                                             // Y_k = L_kk^-1 B_k
    double y[2][2] = {{c[0][0], c[0][1]}, {c[1][0], c[1][1]}};
    zero2(c);
    mm_abT(Xj, Ls, c);                                            // L_ib,k = A_ib,k L_kk^-T
    __syncthreads();
    tile_put(Xi, y);
    tile_put(Xj, c);
    __syncthreads();
    if (ib == kb + 1) {
      const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
      double* Yt = Yf + (int64_t)g * np * D + k0 * D + (int64_t)cb * kNB;
      Yt[(2 * ty) * D + 2 * tx] = y[0][0];
      Yt[(2 * ty) * D + 2 * tx + 1] = y[0][1];
      Yt[(2 * ty + 1) * D + 2 * tx] = y[1][0];
      Yt[(2 * ty + 1) * D + 2 * tx + 1] = y[1][1];
    }
    double* Bt = Bg + (int64_t)ib * kNB * D + (int64_t)cb * kNB;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    c[0][0] = -Bt[(2 * ty) * D + 2 * tx];
    c[0][1] = -Bt[(2 * ty) * D + 2 * tx + 1];
    c[1][0] = -Bt[(2 * ty + 1) * D + 2 * tx];
    c[1][1] = -Bt[(2 * ty + 1) * D + 2 * tx + 1];
    mm_ab(Xj, Xi, c);                                             // L_ib,k Y_k - B_ib
    Bt[(2 * ty) * D + 2 * tx] = -c[0][0];
    Bt[(2 * ty) * D + 2 * tx + 1] = -c[0][1];
    Bt[(2 * ty + 1) * D + 2 * tx] = -c[1][0];
    Bt[(2 * ty + 1) * D + 2 * tx + 1] = -c[1][1];
    return;
  }
  // trailing tile index -> (ib, jb): t = u (u + 1) / 2 + v, ib = kb + 1 + u, jb = kb + 1 + v
  const int t = blockIdx.x;
  int u = 0;
  while ((u + 1) * (u + 2) / 2 <= t) ++u;
  const int v = t - u * (u + 1) / 2;
  const int ib = kb + 1 + u, jb = kb + 1 + v;
  // every global read of the block is issued before the first barrier
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double* tileA = Mg + (int64_t)ib * kNB * np + (int64_t)jb * kNB;
  c[0][0] = -tileA[(2 * ty) * np + 2 * tx];
  c[0][1] = -tileA[(2 * ty) * np + 2 * tx + 1];
  c[1][0] = -tileA[(2 * ty + 1) * np + 2 * tx];
  c[1][1] = -tileA[(2 * ty + 1) * np + 2 * tx + 1];
  tile_load(Xj, Mg + (int64_t)ib * kNB * np + k0, np);            // A_ib,k
  const bool diag = ib == jb;                                     // then X_j = X_i
  if (!diag) tile_load(Xk, Mg + (int64_t)jb * kNB * np + k0, np); // A_jb,k
  __syncthreads();
  double xi[2][2];
  zero2(xi);
  mm_abT(Xj, Ls, xi);                                             // X_i = A_ib,k L_kk^-T
  double xj[2][2] = {{xi[0][0], xi[0][1]}, {xi[1][0], xi[1][1]}};
  if (!diag) {
    zero2(xj);
    mm_abT(Xk, Ls, xj);                                           // X_j = A_jb,k L_kk^-T
  }
  __syncthreads();
  tile_put(Xi, xi);
  tile_put(Xj, xj);
  __syncthreads();
  // A_ib,jb -= X_i X_j^T
  mm_abT(Xi, Xj, c);
  c[0][0] = -c[0][0];
  c[0][1] = -c[0][1];
  c[1][0] = -c[1][0];
  c[1][1] = -c[1][1];
  tileA[(2 * ty) * np + 2 * tx] = c[0][0];
  tileA[(2 * ty) * np + 2 * tx + 1] = c[0][1];
  tileA[(2 * ty + 1) * np + 2 * tx] = c[1][0];
  tileA[(2 * ty + 1) * np + 2 * tx + 1] = c[1][1];
  if (jb == kb + 1) {                                             // this tile publishes L_ib,k
    double* Lt = Lg + (int64_t)ib * kNB * np + k0;
    for (int e = threadIdx.x; e < kNB * kNB; e += 256) Lt[(e / kNB) * np + e % kNB] = Xi[e / kNB][e % kNB];
  }
  if (ib == kb + 1 && jb == kb + 1) {                             // look-ahead: factor the next diagonal tile
    __syncthreads();
    tile_put(Ls, c);
    __syncthreads();
    if (threadIdx.x < 64)
      potrf_tile(Ls, Bc, Lg + (int64_t)ib * kNB * np + (int64_t)ib * kNB, np, Lig + (int64_t)ib * kNB * kNB, status);
  }
}

// Backward solve, block row kb (from the last): every block computes X_k = L_kk^-T Y_k
// (Y_{nb-1} = L^-1 B_{nb-1}, the last forward step, for the first launch); block (ib, cb),
// ib < kb, then does Y_ib -= L_k,ib^T X_k.  Block ib = 0 (the only one when kb = 0) writes
// X_k's rows below n_c to V_c.
__global__ void __launch_bounds__(256)
ridge_back(const double* __restrict__ Lm, const double* __restrict__ Li, const double* __restrict__ Bm,
           double* __restrict__ Yf, float* __restrict__ v_c, RidgeDims r, int kb) {
  __shared__ Tile Ls, Ys, Lt;
  const int g = blockIdx.y;
  const int64_t np = r.npad, D = r.d;
  const int nib = kb > 0 ? kb : 1;
  const int ib = blockIdx.x % nib, cb = blockIdx.x / nib;
  const int64_t k0 = (int64_t)kb * kNB;
  const double* Lig = Li + (int64_t)g * r.nb * kNB * kNB;
  double* Yg = Yf + (int64_t)g * np * D;
  tile_load(Ls, Lig + k0 * kNB, kNB);
  double c[2][2];
  if (kb == r.nb - 1) {
    tile_load(Ys, Bm + (int64_t)g * np * D + k0 * D + (int64_t)cb * kNB, D);
    __syncthreads();
    zero2(c);
    mm_ab(Ls, Ys, c);                                             // Y_k = L_kk^-1 B_k
    __syncthreads();
    tile_put(Ys, c);
  } else {
    tile_load(Ys, Yg + k0 * D + (int64_t)cb * kNB, D);
  }
  __syncthreads();
  zero2(c);
  mm_aTb(Ls, Ys, c);                                              // X_k = L_kk^-T Y_k
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  if (ib == 0) {
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j) {
        const int64_t a = k0 + 2 * ty + i;
        if (a < r.nc) v_c[((int64_t)g * r.nc + a) * D + (int64_t)cb * kNB + 2 * tx + j] = (float)c[i][j];
      }
  }
  if (kb == 0) return;
  __syncthreads();
  tile_put(Ys, c);                                                // Ys = X_k
  tile_load(Lt, Lm + (int64_t)g * np * np + k0 * np + (int64_t)ib * kNB, np);   // L_k,ib
  __syncthreads();
  double* Yt = Yg + (int64_t)ib * kNB * D + (int64_t)cb * kNB;
  c[0][0] = -Yt[(2 * ty) * D + 2 * tx];
  c[0][1] = -Yt[(2 * ty) * D + 2 * tx + 1];
  c[1][0] = -Yt[(2 * ty + 1) * D + 2 * tx];
  c[1][1] = -Yt[(2 * ty + 1) * D + 2 * tx + 1];
  mm_aTb(Lt, Ys, c);                                              // L_k,ib^T X_k - Y_ib
  Yt[(2 * ty) * D + 2 * tx] = -c[0][0];
  Yt[(2 * ty) * D + 2 * tx + 1] = -c[0][1];
  Yt[(2 * ty + 1) * D + 2 * tx] = -c[1][0];
  Yt[(2 * ty + 1) * D + 2 * tx + 1] = -c[1][1];
}

// Backward solve, block rows kb and kb - 1 in one launch (kb >= 1): every block computes X_k =
// L_kk^-T Y_k (Y_{nb-1} = L^-1 B_{nb-1} at kb = nb - 1), the row above Y_{k-1} - L_k,k-1^T X_k
// and X_{k-1} = L_{k-1,k-1}^-T of that, the same values in every block; block (ib, cb), ib <
// kb - 1, then does Y_ib -= L_k,ib^T X_k + L_{k-1},ib^T X_{k-1} (one product chain, so the
// sums round as two single-row steps would).  Block ib = 0 (the only one when kb = 1) writes
// both rows of X below n_c to V_c.  Every global read of a block is issued before its first
// barrier.
__global__ void __launch_bounds__(256)
ridge_back2(const double* __restrict__ Lm, const double* __restrict__ Li, const double* __restrict__ Bm,
            double* __restrict__ Yf, float* __restrict__ v_c, RidgeDims r, int kb) {
  __shared__ Tile Ls, Ys, Lk1, Y1, Ls1, La, Lb;
  const int g = blockIdx.y;
  const int64_t np = r.npad, D = r.d;
  const int k1 = kb - 1;
  const int nib = k1 > 0 ? k1 : 1;
  const int ib = blockIdx.x % nib, cb = blockIdx.x / nib;
  const int64_t k0 = (int64_t)kb * kNB, j0 = (int64_t)k1 * kNB;
  const double* Lig = Li + (int64_t)g * r.nb * kNB * kNB;
  const double* Lg = Lm + (int64_t)g * np * np;
  double* Yg = Yf + (int64_t)g * np * D;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const bool last = kb == r.nb - 1;
  tile_load(Ls, Lig + k0 * kNB, kNB);                             // L_kk^-1
  tile_load(Ys, (last ? Bm + (int64_t)g * np * D : Yg) + k0 * D + (int64_t)cb * kNB, D);   // B_k or Y_k
  tile_load(Lk1, Lg + k0 * np + j0, np);                          // L_k,k-1
  tile_load(Y1, Yg + j0 * D + (int64_t)cb * kNB, D);              // Y_{k-1}
  tile_load(Ls1, Lig + j0 * kNB, kNB);                            // L_{k-1,k-1}^-1
  double* Yt = Yg + (int64_t)ib * kNB * D + (int64_t)cb * kNB;
  double yb[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  if (k1 > 0) {
    tile_load(La, Lg + k0 * np + (int64_t)ib * kNB, np);          // L_k,ib
    tile_load(Lb, Lg + j0 * np + (int64_t)ib * kNB, np);          // L_{k-1},ib
    yb[0][0] = Yt[(2 * ty) * D + 2 * tx];
    yb[0][1] = Yt[(2 * ty) * D + 2 * tx + 1];
    yb[1][0] = Yt[(2 * ty + 1) * D + 2 * tx];
    yb[1][1] = Yt[(2 * ty + 1) * D + 2 * tx + 1];
  }
  __syncthreads();
  double c[2][2];
  if (last) {
    zero2(c);
    mm_ab(Ls, Ys, c);                                             // Y_k = L_kk^-1 B_k
    __syncthreads();
    tile_put(Ys, c);
    __syncthreads();
  }
  double xk[2][2];
  zero2(xk);
  mm_aTb(Ls, Ys, xk);                                             // X_k = L_kk^-T Y_k
  // Y_{k-1} - L_k,k-1^T X_k, as the single-row step forms it: -(L^T X - Y)
  c[0][0] = -Y1[2 * ty][2 * tx];
  c[0][1] = -Y1[2 * ty][2 * tx + 1];
  c[1][0] = -Y1[2 * ty + 1][2 * tx];
  c[1][1] = -Y1[2 * ty + 1][2 * tx + 1];
  __syncthreads();
  tile_put(Ys, xk);                                               // Ys = X_k
  __syncthreads();
  mm_aTb(Lk1, Ys, c);
  c[0][0] = -c[0][0];
  c[0][1] = -c[0][1];
  c[1][0] = -c[1][0];
  c[1][1] = -c[1][1];
  __syncthreads();
  tile_put(Y1, c);                                                // Y1 = the updated Y_{k-1}
  __syncthreads();
  double xk1[2][2];
  zero2(xk1);
  mm_aTb(Ls1, Y1, xk1);                                           // X_{k-1}
  if (ib == 0) {
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j) {
        const int64_t a = k0 + 2 * ty + i, b = j0 + 2 * ty + i;
        if (a < r.nc) v_c[((int64_t)g * r.nc + a) * D + (int64_t)cb * kNB + 2 * tx + j] = (float)xk[i][j];
        if (b < r.nc) v_c[((int64_t)g * r.nc + b) * D + (int64_t)cb * kNB + 2 * tx + j] = (float)xk1[i][j];
      }
  }
  if (k1 == 0) return;
  __syncthreads();
  tile_put(Y1, xk1);                                              // Y1 = X_{k-1}
  __syncthreads();
  c[0][0] = -yb[0][0];
  c[0][1] = -yb[0][1];
  c[1][0] = -yb[1][0];
  c[1][1] = -yb[1][1];
  mm_aTb(La, Ys, c);                                              // L_k,ib^T X_k - Y_ib
  mm_aTb(Lb, Y1, c);                                              //   + L_{k-1},ib^T X_{k-1}
  Yt[(2 * ty) * D + 2 * tx] = -c[0][0];
  Yt[(2 * ty) * D + 2 * tx + 1] = -c[0][1];
  Yt[(2 * ty + 1) * D + 2 * tx] = -c[1][0];
  Yt[(2 * ty + 1) * D + 2 * tx + 1] = -c[1][1];
}

__global__ void ridge_reset_status(int32_t* status) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *status = 0;
}

}  // namespace

size_t ridge_ws_bytes(const Layer& L, int64_t nc) {
  size_t total = 0;
  carve(L, dims_of(L, nc), nullptr, &total);
  return total;
}

hipError_t launch_ridge_fit(const Layer& L, int64_t nc, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v_r, const float* y, double lambda, float* v_c, char* ws,
                            hipStream_t s) {
  const RidgeDims r = dims_of(L, nc);
  RidgeWs w = carve(L, r, ws, nullptr);
  int32_t* status = reinterpret_cast<int32_t*>(ws);
  ridge_reset_status<<<1, 64, 0, s>>>(status);
  hipError_t e = launch_row_lse(L, q, k, w.lse, w.lse_ws, s, 1);
  if (e != hipSuccess) return e;
  const dim3 gp((unsigned)((r.n + kT - 1) / kT), (unsigned)((r.R + kT - 1) / kT), (unsigned)r.hkv);
  const dim3 gr((unsigned)(r.d / kT), (unsigned)((r.R + kT - 1) / kT), (unsigned)r.hkv);
  const int nlow = r.nt * (r.nt + 1) / 2;
  const dim3 gg((unsigned)(nlow + r.nt * (r.d / kT)), (unsigned)kSplit, (unsigned)r.hkv);
  if (r.d == 128) {
    ridge_probs<128><<<gp, 256, 0, s>>>(q, k, w.lse, w.P, r, L.c_log2);
    ridge_resid<128><<<gr, 256, 0, s>>>(w.P, v_r, y, w.T, r);
    ridge_gram<128><<<gg, 256, 0, s>>>(w.P, w.T, w.Mp, w.Bp, r);
  } else {
    ridge_probs<64><<<gp, 256, 0, s>>>(q, k, w.lse, w.P, r, L.c_log2);
    ridge_resid<64><<<gr, 256, 0, s>>>(w.P, v_r, y, w.T, r);
    ridge_gram<64><<<gg, 256, 0, s>>>(w.P, w.T, w.Mp, w.Bp, r);
  }
  const int64_t nsum = r.npad * r.npad + r.npad * r.d;
  unsigned bs = (unsigned)((nsum + 255) / 256);
  if (bs > 4096) bs = 4096;
  ridge_sum<<<dim3(bs, (unsigned)r.hkv), 256, 0, s>>>(w.Mp, w.Bp, w.M, w.Bm, r, lambda);
  ridge_chol<<<dim3(1, (unsigned)r.hkv), 256, 0, s>>>(w.M, w.Lm, w.Li, w.Bm, w.Yf, r, -1, status);
  const int ncb = r.d / kNB;
  for (int kb = 0; kb + 1 < r.nb; ++kb) {
    const int rem = r.nb - 1 - kb;
    const unsigned nblk = (unsigned)(rem * (rem + 1) / 2 + rem * ncb);
    ridge_chol<<<dim3(nblk, (unsigned)r.hkv), 256, 0, s>>>(w.M, w.Lm, w.Li, w.Bm, w.Yf, r, kb, status);
  }
  int kb = r.nb - 1;
  for (; kb >= 1; kb -= 2) {                                      // block rows kb and kb - 1
    const unsigned nblk = (unsigned)((kb - 1 > 0 ? kb - 1 : 1) * ncb);
    ridge_back2<<<dim3(nblk, (unsigned)r.hkv), 256, 0, s>>>(w.Lm, w.Li, w.Bm, w.Yf, v_c, r, kb);
  }
  if (kb == 0)                                                    // an odd count: row 0 alone
    ridge_back<<<dim3((unsigned)ncb, (unsigned)r.hkv), 256, 0, s>>>(w.Lm, w.Li, w.Bm, w.Yf, v_c, r, 0);
  return hipGetLastError();
}

}  // namespace kvc
