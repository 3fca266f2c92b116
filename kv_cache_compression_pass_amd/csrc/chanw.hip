// RDKV K-channel weights w_c[g][c] = s * ||Q_g[:,c]|| * ||K_g[:,c]|| (RDKV summary §2.1: the
// spectral norm of the logit change from zeroing channel c; computed once on the full cache,
// §2.2 stage 1).  An HBM-streaming column reduction: each block sums the squares of a range of
// rows in float64 (bf16 squares are exact), partials are reduced in a fixed order.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kRowsPerBlock = 512;

// grid: x = row block, y = source (0: the G*Nq stacked query rows of group g, 1: the N keys
// of head g), z = g.  part[g][src][block][c].
template <int D>
__global__ void __launch_bounds__(256)
chanw_partial(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              double* __restrict__ part, int G, int64_t N, int64_t Nq, int nblk) {
  constexpr int TPR = D / 8;              // threads per row (8 channels each)
  constexpr int RPP = 256 / TPR;          // rows per pass
  const int g = blockIdx.z;
  const int src = blockIdx.y;
  const int64_t rows = src == 0 ? (int64_t)G * Nq : N;
  const uint16_t* base = src == 0 ? q + (int64_t)g * G * Nq * D : k + (int64_t)g * N * D;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;
  if (r0 >= rows) return;
  const int64_t r1 = (r0 + kRowsPerBlock < rows) ? r0 + kRowsPerBlock : rows;
  const int cg = threadIdx.x % TPR;
  const int rl = threadIdx.x / TPR;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
#pragma unroll 4
  for (int64_t r = r0 + rl; r < r1; r += RPP) {
    uint4 w = *reinterpret_cast<const uint4*>(base + r * D + cg * 8);
    uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = bf16_bits_to_f32(ww[j] & 0xFFFFu);
      float b = bf16_bits_to_f32(ww[j] >> 16);
      acc[2 * j] += (double)(a * a);       // bf16*bf16 is exact in fp32
      acc[2 * j + 1] += (double)(b * b);
    }
  }
  __shared__ double red[256][9];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[threadIdx.x][j] = acc[j];
  __syncthreads();
  // fixed-order tree over the RPP row lanes of each channel group
  for (int w = RPP / 2; w >= 1; w >>= 1) {
    if (rl < w) {
#pragma unroll
      for (int j = 0; j < 8; ++j) red[threadIdx.x][j] += red[threadIdx.x + w * TPR][j];
    }
    __syncthreads();
  }
  if (rl == 0) {
    double* out = part + (((int64_t)g * 2 + src) * nblk + blockIdx.x) * D + cg * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = red[threadIdx.x][j];
  }
}

// One block per KV head.  Four threads share each (src, c): thread q sums the q-th quarter of
// the partials in ascending block order, eight independent loads at a time, and the four
// sums are combined as (s0 + s1) + (s2 + s3): a fixed order.
__global__ void __launch_bounds__(1024)
chanw_finish(const double* __restrict__ part, float* __restrict__ w_c, int D, int G, int64_t N,
             int64_t Nq, int nblk, double scale) {
  __shared__ double sums[2][4][128];
  const int g = blockIdx.x;
  const int c = threadIdx.x % D;
  const int q = (threadIdx.x / D) & 3;
  const int src = threadIdx.x / (4 * D);
  if (src < 2) {
    const int64_t rows = src == 0 ? (int64_t)G * Nq : N;
    const int nb = (int)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
    const int b0 = (int)((int64_t)nb * q / 4), b1 = (int)((int64_t)nb * (q + 1) / 4);
    const double* p = part + (((int64_t)g * 2 + src) * nblk) * D + c;
    double a[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += p[(int64_t)(b + u) * D];
    }
    for (; b < b1; ++b) a[0] += p[(int64_t)b * D];
    sums[src][q][c] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  }
  __syncthreads();
  if ((int)threadIdx.x < D) {
    const int cc = threadIdx.x;
    const double sq = (sums[0][0][cc] + sums[0][1][cc]) + (sums[0][2][cc] + sums[0][3][cc]);
    const double sk = (sums[1][0][cc] + sums[1][1][cc]) + (sums[1][2][cc] + sums[1][3][cc]);
    w_c[(int64_t)g * D + cc] = (float)(scale * sqrt(sq) * sqrt(sk));
  }
}

int nblk_of(const Layer& L) {
  int64_t rq = (int64_t)L.G * L.nq, rk = L.n;
  int64_t r = rq > rk ? rq : rk;
  return (int)((r + kRowsPerBlock - 1) / kRowsPerBlock);
}

}  // namespace

size_t chanw_ws_bytes(const Layer& L) {
  WsPlan p;
  p.take((size_t)L.hkv * 2 * nblk_of(L) * L.d * sizeof(double));
  return p.off;
}

hipError_t launch_channel_weights(const Layer& L, const uint16_t* q, const uint16_t* k,
                                  float* w_c, char* ws, hipStream_t s) {
  WsPlan p;
  const int nblk = nblk_of(L);
  double* part = reinterpret_cast<double*>(ws + p.take((size_t)L.hkv * 2 * nblk * L.d * sizeof(double)));
  dim3 grid((unsigned)nblk, 2, (unsigned)L.hkv);
  if (L.d == 128)
    chanw_partial<128><<<grid, 256, 0, s>>>(q, k, part, L.G, L.n, L.nq, nblk);
  else
    chanw_partial<64><<<grid, 256, 0, s>>>(q, k, part, L.G, L.n, L.nq, nblk);
  chanw_finish<<<(unsigned)L.hkv, 1024, 0, s>>>(part, w_c, L.d, L.G, L.n, L.nq, nblk, L.scale);
  return hipGetLastError();
}

}  // namespace kvc
