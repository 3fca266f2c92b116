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

// One block per KV head: thread (src, c) sums its partials in ascending block order.
__global__ void __launch_bounds__(256)
chanw_finish(const double* __restrict__ part, float* __restrict__ w_c, int D, int G, int64_t N,
             int64_t Nq, int nblk, double scale) {
  __shared__ double sums[2][128];
  const int g = blockIdx.x;
  const int src = threadIdx.x / D;
  const int c = threadIdx.x % D;
  if (src < 2) {
    const int64_t rows = src == 0 ? (int64_t)G * Nq : N;
    const int nb = (int)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
    const double* p = part + (((int64_t)g * 2 + src) * nblk) * D + c;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int b = 0;
    for (; b + 4 <= nb; b += 4) {
      s0 += p[(int64_t)b * D];
      s1 += p[(int64_t)(b + 1) * D];
      s2 += p[(int64_t)(b + 2) * D];
      s3 += p[(int64_t)(b + 3) * D];
    }
    for (; b < nb; ++b) s0 += p[(int64_t)b * D];
    sums[src][c] = (s0 + s1) + (s2 + s3);
  }
  __syncthreads();
  if (threadIdx.x < D)
    w_c[(int64_t)g * D + threadIdx.x] = (float)(scale * sqrt(sums[0][threadIdx.x]) * sqrt(sums[1][threadIdx.x]));
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
  chanw_finish<<<(unsigned)L.hkv, 256, 0, s>>>(part, w_c, L.d, L.G, L.n, L.nq, nblk, L.scale);
  return hipGetLastError();
}

}  // namespace kvc
