// The two terms of KVSculpt's loss (KVSculpt summary §2) per query head: the squared
// Frobenius error of the attention output and of the row log-sum-exp, compressed against full.
// One block per query head: each thread adds a strided subset in float64 in index order, then
// a fixed tree over the block, so the result does not depend on scheduling.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kFidThreads = 256;

__device__ __forceinline__ double block_sum_fixed(double v, double* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int w = kFidThreads / 2; w >= 1; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kFidThreads)
fidelity_terms_kernel(const float* __restrict__ y_hat, const float* __restrict__ lse_hat,
                      const float* __restrict__ y, const float* __restrict__ lse, double* __restrict__ terms,
                      int64_t Nq, int d) {
  __shared__ double sh[kFidThreads];
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = Nq * d;                        // a multiple of 4 (d is 64 or 128)
  const float4* a = reinterpret_cast<const float4*>(y_hat + (int64_t)h * n);
  const float4* b = reinterpret_cast<const float4*>(y + (int64_t)h * n);
  double sy = 0.0;
  for (int64_t i = t; i < n / 4; i += kFidThreads) {
    const float4 p = a[i], r = b[i];
    const double e0 = (double)p.x - (double)r.x, e1 = (double)p.y - (double)r.y;
    const double e2 = (double)p.z - (double)r.z, e3 = (double)p.w - (double)r.w;
    sy += e0 * e0;
    sy += e1 * e1;
    sy += e2 * e2;
    sy += e3 * e3;
  }
  double sl = 0.0;
  for (int64_t i = t; i < Nq; i += kFidThreads) {
    const float p = lse_hat[(int64_t)h * Nq + i], r = lse[(int64_t)h * Nq + i];
    if (!(p == r)) {                               // equal values (both -inf included) add nothing
      const double e = (double)p - (double)r;
      sl += e * e;
    }
  }
  const double ty = block_sum_fixed(sy, sh);
  const double tl = block_sum_fixed(sl, sh);
  if (t == 0) {
    terms[2 * h] = ty;
    terms[2 * h + 1] = tl;
  }
}

}  // namespace

hipError_t launch_fidelity_terms(const Layer& L, const float* y_hat, const float* lse_hat, const float* y,
                                 const float* lse, double* terms, hipStream_t s) {
  fidelity_terms_kernel<<<(unsigned)L.hq, kFidThreads, 0, s>>>(y_hat, lse_hat, y, lse, terms, L.nq, L.d);
  return hipGetLastError();
}

}  // namespace kvc
