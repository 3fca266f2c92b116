// Adaptive keep by threshold and sliding window (KVzap summary §2.3): per KV head, token t
// keeps width keep_bits when its score is at or above the threshold (float32 compare) or when
// t >= N - window; every other token gets width 0.  One pass over the scores; HBM-bound
// (4 bytes read and 1 written per token).
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kKeepPerThread = 16;
constexpr int kKeepBlock = 256 * kKeepPerThread;   // tokens per block

__global__ void __launch_bounds__(256) keep_clear(int64_t* __restrict__ kept, int Hkv) {
  for (int g = threadIdx.x; g < Hkv; g += 256) kept[g] = 0;
}

__device__ __forceinline__ uint32_t keep_byte(float s, float thr, int64_t t, int64_t wstart, uint32_t kb) {
  return (s >= thr || t >= wstart) ? kb : 0u;
}

// Block (chunk, g): tokens [chunk * 4096, +4096) of head g, 16 consecutive tokens per thread.
// The kept count of the block is added to kept[g] (integers: order-free).
__global__ void __launch_bounds__(256)
keep_threshold(const float* __restrict__ scores, float thr, int64_t N, int64_t wstart, uint32_t kb,
               uint8_t* __restrict__ bits, int64_t* __restrict__ kept) {
  __shared__ int wsum[4];
  const int g = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kKeepBlock + (int64_t)threadIdx.x * kKeepPerThread;
  const float* src = scores + (int64_t)g * N + t0;
  uint8_t* dst = bits + (int64_t)g * N + t0;
  int cnt = 0;
  if (t0 + kKeepPerThread <= N && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 x = reinterpret_cast<const float4*>(src)[i];
      const int64_t t = t0 + 4 * i;
      const uint32_t b0 = keep_byte(x.x, thr, t, wstart, kb), b1 = keep_byte(x.y, thr, t + 1, wstart, kb);
      const uint32_t b2 = keep_byte(x.z, thr, t + 2, wstart, kb), b3 = keep_byte(x.w, thr, t + 3, wstart, kb);
      cnt += (b0 != 0) + (b1 != 0) + (b2 != 0) + (b3 != 0);
      w[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    for (int j = 0; j < kKeepPerThread; ++j) {
      const int64_t t = t0 + j;
      if (t < N) {
        const uint32_t b = keep_byte(src[j], thr, t, wstart, kb);
        dst[j] = (uint8_t)b;
        cnt += (b != 0);
      }
    }
  }
  if (kept == nullptr) return;                 // uniform
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(&kept[g]), (unsigned long long)tot);
  }
}

}  // namespace

hipError_t launch_keep_threshold(const Layer& L, const float* scores, float threshold, int64_t window,
                                 int keep_bits, uint8_t* bits_out, int64_t* kept, hipStream_t s) {
  if (kept) keep_clear<<<1, 256, 0, s>>>(kept, L.hkv);
  const int64_t nblk = (L.n + kKeepBlock - 1) / kKeepBlock;
  const int64_t wstart = window >= L.n ? 0 : L.n - window;
  keep_threshold<<<dim3((unsigned)nblk, (unsigned)L.hkv), 256, 0, s>>>(scores, threshold, L.n, wstart,
                                                                       (uint32_t)keep_bits, bits_out, kept);
  return hipGetLastError();
}

}  // namespace kvc
