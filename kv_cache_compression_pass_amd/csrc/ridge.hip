// KVSculpt's value solve (KVSculpt summary §2, value step; §4 "Select+Fit"): with the
// compressed keys fixed, the values V_c that minimise ||A_c V_c + A_r V_r - Y||_F^2 +
// lambda ||V_c||_F^2 solve (A_c^T A_c + lambda I) V_c = A_c^T (Y - A_r V_r).  The rows of the
// G query heads of a KV head are stacked (they share the head's V_c).
//
// Kernels, one stream, per KV head g (R = G * Nq stacked rows, n = n_c + m keys):
//   row LSE        the scorer's pass 1 over the n keys                          (score.hip)
//   ridge_probs    P[r][t] = exp(s q_r . k_t - l_r), fp32, 64 x 64 tiles, VALU dot products
//   ridge_resid    T = Y - P_r V_r (fp32), 64 x 64 tiles over (rows, channels)
//   ridge_gram     M = P_c^T P_c and B = P_c^T T, fp64 sums of fp32 products (exact), the row
//                  sum split in kSplit fixed parts
//   ridge_sum      M += lambda I (identity on the padding), the parts added in fixed order
//   ridge_chol     blocked Cholesky, one launch per block column kb: every tile (i, j) of the
//                  trailing matrix computes L_ik = A_ik L_kk^-T itself, subtracts L_ik L_jk^T,
//                  and the tile (kb+1, kb+1) then factors itself and inverts its L (look-ahead)
//   ridge_solve    forward and backward substitution by blocks, one block per 16 columns
// Every sum has a fixed order, so results are deterministic.  The matrix is padded to a
// multiple of 64 with an identity block, which leaves the solution unchanged.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kT = 64;          // tile edge
constexpr int kSplit = 4;       // parts of the row sum in the Gram products
constexpr int kSolveCols = 16;  // right-hand-side columns per solve block

struct RidgeDims {
  int hq, hkv, d, G, causal;
  int64_t n, nq, nc, m, R, npad;
  int nb;
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
  r.nb = (int)(r.npad / kT);
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
  double* Li;     // [Hkv][nb][64][64]          inverse of each diagonal block of L
  double* Bm;     // [Hkv][npad][d]
  double* Yf;     // [Hkv][npad][d]             forward-substitution result
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
  const size_t o_Li = p.take(sizeof(double) * r.hkv * r.nb * kT * kT);
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

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// P[g][r][t] = exp(s q_r . k_t - l_r) (0 where masked).  Block: 64 rows x 64 keys of head g,
// 256 threads as 16 x 16, each 4 rows x 4 keys; Q and K tiles staged transposed in LDS as fp32.
template <int D>
__global__ void __launch_bounds__(256)
ridge_probs(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ lse,
            float* __restrict__ P, RidgeDims r, float c_log2) {
  __shared__ float qT[D][kT];
  __shared__ float kT_[D][kT];
  const int g = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kT, t0 = (int64_t)blockIdx.x * kT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int e = tid; e < kT * (D / 8); e += 256) {
    const int row = e / (D / 8), c8 = e % (D / 8);
    const int64_t rr = r0 + row;
    uint4 qv = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
    if (rr < r.R) {
      const int64_t h = (int64_t)g * r.G + rr / r.nq, i = rr % r.nq;
      qv = *reinterpret_cast<const uint4*>(q + (h * r.nq + i) * D + c8 * 8);
    }
    const int64_t tt = t0 + row;
    if (tt < r.n) kv = *reinterpret_cast<const uint4*>(k + ((int64_t)g * r.n + tt) * D + c8 * 8);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w}, kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qT[c8 * 8 + 2 * u][row] = __uint_as_float(qw[u] << 16);
      qT[c8 * 8 + 2 * u + 1][row] = __uint_as_float(qw[u] & 0xFFFF0000u);
      kT_[c8 * 8 + 2 * u][row] = __uint_as_float(kw[u] << 16);
      kT_[c8 * 8 + 2 * u + 1][row] = __uint_as_float(kw[u] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll 4
  for (int c = 0; c < D; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(&qT[c][ty * 4]);
    const float4 b = *reinterpret_cast<const float4*>(&kT_[c][tx * 4]);
    const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rr = r0 + ty * 4 + i;
    if (rr >= r.R) continue;
    const int64_t h = (int64_t)g * r.G + rr / r.nq, qi = rr % r.nq;
    const float l = lse[h * r.nq + qi];
    const float l2 = l * kLog2e;
    const int64_t last = r.causal ? r.n - r.nq + qi : r.n - 1;      // last visible key
    float* prow = P + ((int64_t)g * r.R + rr) * r.n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tt = t0 + tx * 4 + j;
      if (tt >= r.n) continue;
      const bool vis = tt <= last && l > -__builtin_inff();
      prow[tt] = vis ? exp2f(fmaf(acc[i][j], c_log2, -l2)) : 0.f;
    }
  }
}

// T[g][r][c] = Y[h][i][c] - sum_{t < m} P[g][r][n_c + t] V_r[g][t][c].  Block: 64 rows x 64
// channels; the t sum in chunks of 32 staged in LDS.
template <int D>
__global__ void __launch_bounds__(256)
ridge_resid(const float* __restrict__ P, const uint16_t* __restrict__ v_r, const float* __restrict__ y,
            float* __restrict__ T, RidgeDims r) {
  __shared__ float pT[32][kT];
  __shared__ float vS[32][kT];
  const int g = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kT;
  const int c0 = blockIdx.x * kT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int64_t s0 = 0; s0 < r.m; s0 += 32) {
    for (int e = tid; e < 32 * kT; e += 256) {
      const int row = e / 32, tt = e % 32;               // P: consecutive threads, consecutive keys
      const int64_t rr = r0 + row, t = s0 + tt;
      pT[tt][row] = (rr < r.R && t < r.m) ? P[((int64_t)g * r.R + rr) * r.n + r.nc + t] : 0.f;
      const int vt = e / kT, vc = e % kT;                // V: consecutive threads, consecutive channels
      const int64_t t2 = s0 + vt;
      vS[vt][vc] = (t2 < r.m) ? bf16f(v_r[((int64_t)g * r.m + t2) * D + c0 + vc]) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int tt = 0; tt < 32; ++tt) {
      const float4 a = *reinterpret_cast<const float4*>(&pT[tt][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&vS[tt][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rr = r0 + ty * 4 + i;
    if (rr >= r.R) continue;
    const int64_t h = (int64_t)g * r.G + rr / r.nq, qi = rr % r.nq;
    const float4 yv = *reinterpret_cast<const float4*>(y + (h * r.nq + qi) * D + c0 + tx * 4);
    *reinterpret_cast<float4*>(T + ((int64_t)g * r.R + rr) * D + c0 + tx * 4) =
        make_float4(yv.x - acc[i][0], yv.y - acc[i][1], yv.z - acc[i][2], yv.w - acc[i][3]);
  }
}

// Gram products over the rows of part s: tile (a-tile, b-tile) of M = P_c^T P_c (lower tiles),
// or tile (a-tile, channel tile) of B = P_c^T T.  fp32 inputs, fp64 products and sums.
template <int D>
__global__ void __launch_bounds__(256)
ridge_gram(const float* __restrict__ P, const float* __restrict__ T, double* __restrict__ Mp,
           double* __restrict__ Bp, RidgeDims r) {
  __shared__ double xs[32][kT];
  __shared__ double zs[32][kT];
  const int s = blockIdx.y, g = blockIdx.z;
  const int nt = r.nb;
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
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  const float* Pg = P + (int64_t)g * r.R * r.n;
  const float* Tg = T + (int64_t)g * r.R * D;
  for (int64_t q0 = rbeg; q0 < rend; q0 += 32) {
    for (int e = tid; e < 32 * kT; e += 256) {
      const int rr = e / kT, col = e % kT;
      const int64_t row = q0 + rr;
      const bool rv = row < rend;
      const int64_t a = a0 + col;
      xs[rr][col] = (rv && a < r.nc) ? (double)Pg[row * r.n + a] : 0.0;
      const int64_t b = b0 + col;
      double z = 0.0;
      if (rv) z = isB ? (double)Tg[row * D + b] : (b < r.nc ? (double)Pg[row * r.n + b] : 0.0);
      zs[rr][col] = z;
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < 32; ++rr) {
      double av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = xs[rr][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = zs[rr][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (!isB) {
    double* dst = Mp + ((int64_t)s * r.hkv + g) * r.npad * r.npad;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(a0 + ty * 4 + i) * r.npad + b0 + tx * 4 + j] = acc[i][j];
  } else {
    double* dst = Bp + ((int64_t)s * r.hkv + g) * r.npad * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(a0 + ty * 4 + i) * D + b0 + tx * 4 + j] = acc[i][j];
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

// Cholesky of the 64 x 64 tile in LDS (lower part) by wave 0, then the inverse of that L;
// writes L (lower, zeros above) to Ld (row stride ld) and L^-1 to Li (64 x 64).  A pivot that
// is not positive sets the status bit.
__device__ void potrf_tile(double (*A)[kT + 1], double (*X)[kT + 1], double* __restrict__ Ld, int64_t ld,
                           double* __restrict__ Li, int32_t* __restrict__ status) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int i = tid;
    bool bad = false;
    for (int j = 0; j < kT; ++j) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      const double piv = A[j][j];
      bad |= !(piv > 0.0);
      const double dj = sqrt(piv);
      if (i == j) A[j][j] = dj;
      if (i > j) A[i][j] = A[i][j] / dj;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      if (i > j) {
        const double lij = A[i][j];
        for (int c = j + 1; c <= i; ++c) A[i][c] -= lij * A[c][j];
      }
    }
    if (bad && i == 0) atomicOr(status, KVC_DEV_NOT_SPD);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    // column i of L^-1 by forward substitution: X[r][i] for r >= i
    for (int rr = 0; rr < kT; ++rr) {
      double v;
      if (rr < i) {
        v = 0.0;
      } else {
        v = rr == i ? 1.0 : 0.0;
        for (int p = i; p < rr; ++p) v -= A[rr][p] * X[p][i];
        v /= A[rr][rr];
      }
      X[rr][i] = v;
    }
  }
  __syncthreads();
  for (int e = tid; e < kT * kT; e += blockDim.x) {
    const int rr = e / kT, c = e % kT;
    Ld[rr * ld + c] = c <= rr ? A[rr][c] : 0.0;
    Li[e] = X[rr][c];
  }
}

// One block column kb of the blocked Cholesky (kb = -1: factor tile (0, 0) only).  Block
// (tile index) covers tile (ib, jb), kb < jb <= ib < nb, of head g.
__global__ void __launch_bounds__(256)
ridge_chol(double* __restrict__ M, double* __restrict__ Lm, double* __restrict__ Li, RidgeDims r, int kb,
           int32_t* __restrict__ status) {
  __shared__ double Ls[kT][kT + 1];     // L_kk^-1, then the tile to factor
  __shared__ double Xi[kT][kT + 1];
  __shared__ double Xj[kT][kT + 1];
  const int g = blockIdx.y, tid = threadIdx.x;
  const int64_t np = r.npad;
  double* Mg = M + (int64_t)g * np * np;
  double* Lg = Lm + (int64_t)g * np * np;
  double* Lig = Li + (int64_t)g * r.nb * kT * kT;
  if (kb < 0) {
    for (int e = tid; e < kT * kT; e += 256) Ls[e / kT][e % kT] = Mg[(e / kT) * np + e % kT];
    __syncthreads();
    potrf_tile(Ls, Xi, Lg, np, Lig, status);
    return;
  }
  // tile index -> (ib, jb) with kb < jb <= ib < nb: t = u (u + 1) / 2 + v, ib = kb + 1 + u, jb = kb + 1 + v
  const int t = blockIdx.x;
  int u = 0;
  while ((u + 1) * (u + 2) / 2 <= t) ++u;
  const int v = t - u * (u + 1) / 2;
  const int ib = kb + 1 + u, jb = kb + 1 + v;
  for (int e = tid; e < kT * kT; e += 256) {
    const int rr = e / kT, c = e % kT;
    Ls[rr][c] = Lig[(int64_t)kb * kT * kT + e];
    Xj[rr][c] = Mg[((int64_t)ib * kT + rr) * np + (int64_t)kb * kT + c];      // A_ib,kb
  }
  __syncthreads();
  const int tx = tid & 15, ty = tid >> 4;
  // X_i = A_ib,kb L_kk^-T: X[r][c] = sum_{p <= c} A[r][p] Linv[c][p]
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int p = 0; p < kT; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = Xj[ty * 4 + i][p];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fma(a, Ls[tx * 4 + j][p], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Xi[ty * 4 + i][tx * 4 + j] = acc[i][j];
  __syncthreads();
  if (jb != ib) {
    for (int e = tid; e < kT * kT; e += 256)
      Xj[e / kT][e % kT] = Mg[((int64_t)jb * kT + e / kT) * np + (int64_t)kb * kT + e % kT];   // A_jb,kb
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int p = 0; p < kT; ++p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = Xj[ty * 4 + i][p];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a, Ls[tx * 4 + j][p], acc[i][j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) Xj[ty * 4 + i][tx * 4 + j] = acc[i][j];
    __syncthreads();
  } else {
    for (int e = tid; e < kT * kT; e += 256) Xj[e / kT][e % kT] = Xi[e / kT][e % kT];
    __syncthreads();
  }
  // A_ib,jb -= X_i X_j^T
  double* tileA = Mg + (int64_t)ib * kT * np + (int64_t)jb * kT;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = tileA[(ty * 4 + i) * np + tx * 4 + j];
  for (int p = 0; p < kT; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = Xi[ty * 4 + i][p];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fma(-a, Xj[tx * 4 + j][p], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tileA[(ty * 4 + i) * np + tx * 4 + j] = acc[i][j];
  if (jb == kb + 1) {                                  // this tile publishes L_ib,kb
    double* Lt = Lg + (int64_t)ib * kT * np + (int64_t)kb * kT;
    for (int e = tid; e < kT * kT; e += 256) Lt[(e / kT) * np + e % kT] = Xi[e / kT][e % kT];
  }
  if (ib == kb + 1 && jb == kb + 1) {                 // look-ahead: factor the next diagonal tile
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) Ls[ty * 4 + i][tx * 4 + j] = acc[i][j];
    __syncthreads();
    potrf_tile(Ls, Xi, Lg + (int64_t)ib * kT * np + (int64_t)ib * kT, np, Lig + (int64_t)ib * kT * kT, status);
  }
}

// Solve L L^T X = B for kSolveCols columns of head g: forward Y_k = L_kk^-1 (B_k - sum_{j<k}
// L_kj Y_j), backward X_k = L_kk^-T (Y_k - sum_{j>k} L_jk^T X_j); writes V_c = X[:n_c] (fp32).
__global__ void __launch_bounds__(256)
ridge_solve(const double* __restrict__ Lm, const double* __restrict__ Li, const double* __restrict__ Bm,
            double* __restrict__ Yf, float* __restrict__ v_c, RidgeDims r) {
  __shared__ double acc_s[kT][kSolveCols];
  const int g = blockIdx.y, c0 = blockIdx.x * kSolveCols;
  const int tid = threadIdx.x, row = tid >> 2, cq = (tid & 3) * 4;
  const int64_t np = r.npad, D = r.d;
  const double* Lg = Lm + (int64_t)g * np * np;
  const double* Lig = Li + (int64_t)g * r.nb * kT * kT;
  const double* Bg = Bm + (int64_t)g * np * D;
  double* Yg = Yf + (int64_t)g * np * D;
  for (int kb = 0; kb < r.nb; ++kb) {
    const int64_t a = (int64_t)kb * kT + row;
    double acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = Bg[a * D + c0 + cq + j];
    for (int64_t p = 0; p < (int64_t)kb * kT; ++p) {
      const double l = Lg[a * np + p];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fma(-l, Yg[p * D + c0 + cq + j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc_s[row][cq + j] = acc[j];
    __syncthreads();
    const double* Lik = Lig + (int64_t)kb * kT * kT;
    double y[4] = {0.0, 0.0, 0.0, 0.0};
    for (int p = 0; p <= row; ++p) {
      const double l = Lik[row * kT + p];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = fma(l, acc_s[p][cq + j], y[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) Yg[a * D + c0 + cq + j] = y[j];
    __syncthreads();
  }
  for (int kb = r.nb - 1; kb >= 0; --kb) {
    const int64_t a = (int64_t)kb * kT + row;
    double acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = Yg[a * D + c0 + cq + j];
    for (int64_t p = (int64_t)(kb + 1) * kT; p < np; ++p) {
      const double l = Lg[p * np + a];                 // (L^T)[a][p] = L[p][a]
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fma(-l, Yg[p * D + c0 + cq + j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc_s[row][cq + j] = acc[j];
    __syncthreads();
    const double* Lik = Lig + (int64_t)kb * kT * kT;
    double x[4] = {0.0, 0.0, 0.0, 0.0};
    for (int p = row; p < kT; ++p) {
      const double l = Lik[p * kT + row];              // (L_kk^-T)[row][p] = L_kk^-1[p][row]
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = fma(l, acc_s[p][cq + j], x[j]);
    }
    __syncthreads();                                   // every thread has read Y_k's rows
#pragma unroll
    for (int j = 0; j < 4; ++j) Yg[a * D + c0 + cq + j] = x[j];   // X_k replaces Y_k
    if (a < r.nc) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v_c[((int64_t)g * r.nc + a) * D + c0 + cq + j] = (float)x[j];
    }
    __syncthreads();
  }
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
  hipError_t e = launch_row_lse(L, q, k, w.lse, w.lse_ws, s);
  if (e != hipSuccess) return e;
  const dim3 gp((unsigned)((r.n + kT - 1) / kT), (unsigned)((r.R + kT - 1) / kT), (unsigned)r.hkv);
  const dim3 gr((unsigned)(r.d / kT), (unsigned)((r.R + kT - 1) / kT), (unsigned)r.hkv);
  const int nlow = r.nb * (r.nb + 1) / 2;
  const dim3 gg((unsigned)(nlow + r.nb * (r.d / kT)), (unsigned)kSplit, (unsigned)r.hkv);
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
  ridge_chol<<<dim3(1, (unsigned)r.hkv), 256, 0, s>>>(w.M, w.Lm, w.Li, r, -1, status);
  for (int kb = 0; kb + 1 < r.nb; ++kb) {
    const int rem = r.nb - 1 - kb;
    ridge_chol<<<dim3((unsigned)(rem * (rem + 1) / 2), (unsigned)r.hkv), 256, 0, s>>>(w.M, w.Lm, w.Li, r, kb,
                                                                                        status);
  }
  ridge_solve<<<dim3((unsigned)(r.d / kSolveCols), (unsigned)r.hkv), 256, 0, s>>>(w.Lm, w.Li, w.Bm, w.Yf, v_c, r);
  return hipGetLastError();
}

}  // namespace kvc
