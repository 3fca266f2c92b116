// Bit allocation over the widths {0,2,4,8,16} (RDKV summary §2.1 objective, §2.2 reverse
// water-filling, stages 2 and 3) and the fixed-budget top-k keep (KVzap summary §2.3).
//
// Exact rule.  Unit u has cost c_u = float32(w_u * sigma_u) and size s_u (d for a V token,
// R_g for a K channel).  Step k (width b_k -> b_{k+1}) has the key
// key = (c_u * num_k) / (s_u * den_k) in float64 (theta_k = num_k/den_k = 3/8, 3/32, 15/1024,
// 255/524288) and rate s_u * (b_{k+1} - b_k).  lambda* is the key at which the cumulative rate
// of the keys in descending order first exceeds B (0 if every step fits); every step with a
// larger key is taken; steps with key == lambda* are granted in ascending unit index while the
// cumulative rate fits, stopping at the first that does not.
//
// GPU plan: positive float64 keys order like their bit patterns, so lambda* is found by a
// weighted MSB-first radix select over the 64-bit patterns (11-bit digits; integer
// histograms of step rates, so the selection is exact and independent of summation order).
// Each bin also records its smallest and largest key: once the chosen bin holds a single key
// value, that value is lambda* and the remaining passes do nothing.  The tie rule is an
// ordered exclusive scan over units.  Top-k runs the same select per KV head on
// order-preserving 32-bit score keys with weight 1.
//
// Two launch shapes:
//  * small stages (<= 2048 units, e.g. the K-channel stage): one block does everything in LDS;
//  * larger stages: per pass a histogram kernel (block-private LDS bins flushed with integer
//    atomics) and a one-block select kernel; then per-block tie sums, and the assignment, each
//    of whose blocks adds up the tie sums of the blocks before it (at most kMaxBlocks).
//    Kernel boundaries order every step; no cross-block fences are needed.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kHistUpt = 4;           // multi-block V/K histograms: units per thread of a 1024-thread block
constexpr int kMaxBlocks = 512;       // multi-block path: units per thread (1..16) chosen so that
                                       // the blocks of all segments stay within this
constexpr int kSmallUnits = 2048;      // single-block path: up to 8192 keys in LDS
constexpr int kMaxSeg = 1024;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

__constant__ uint32_t kThetaNum[4] = {3u, 3u, 15u, 255u};
__constant__ uint32_t kThetaDen[4] = {8u, 32u, 1024u, 524288u};
__constant__ uint32_t kLevels[5] = {0u, 2u, 4u, 8u, 16u};

struct SelState {
  uint64_t prefix;      // selected key bits so far (the full key once done)
  int64_t brem;         // budget left for keys above the prefix
  int64_t budget;       // B (V/K); kept tokens per head (top-k)
  int32_t all_fit;      // every positive key fits: lambda* = 0, no ties
  int32_t none;         // top-k with k == 0
  int32_t done;         // lambda* known
  int32_t pad;
};

struct AllocWs {
  int32_t* status;
  SelState* st;         // [nseg]
  int64_t* hist;        // [nseg][kBins]  (the current pass)
  uint64_t* pmin;       // [nseg]  smallest key of the current prefix set (this pass)
  uint64_t* pmax;       // [nseg]  largest
  int32_t* rpart;       // [Hkv][ncb]  retained tokens per 4096-token block (K stage)
  int32_t* rbad;        // [Hkv][ncb]  invalid token widths seen in the block
  int64_t* rcount;      // [Hkv]      R_g (K stage)
  int64_t* bsum;        // [nseg][nblk]
  int64_t* used_part;   // [nseg][nblk]
  double* dist_part;    // [nseg][nblk]
};

// Digit of pass p: bits [lo, hi) counted from the top of an nb-bit key.
struct Digit {
  int lo, hi;
  uint64_t himask;      // bits at or above hi
};
__host__ __device__ __forceinline__ Digit digit_of(int pass, int nb) {
  Digit d;
  d.hi = nb - kDigitBits * pass;
  d.lo = d.hi - kDigitBits > 0 ? d.hi - kDigitBits : 0;
  d.himask = (d.hi >= 64) ? 0ull : (~0ull << d.hi);
  return d;
}
__host__ __device__ __forceinline__ int passes_of(int nb) { return (nb + kDigitBits - 1) / kDigitBits; }

__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The four step keys of a unit of cost c and size s.  The passes recompute them from the weights
// (the same float64 operations each time, so the same bits): cheaper than storing and re-reading
// 32 bytes per unit.
__device__ __forceinline__ void unit_keys(float c, int64_t s, uint64_t (&kk)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) kk[k] = 0;
  if (c > 0.f && s > 0) {
    const double cd = (double)c, sd = (double)s;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      kk[k] = (uint64_t)__double_as_longlong((cd * (double)kThetaNum[k]) / (sd * (double)kThetaDen[k]));
  }
}

__device__ __forceinline__ int64_t step_rate(int64_t s, int k) {
  return s * (int64_t)(kLevels[k + 1] - kLevels[k]);
}

// Steps with key > lam (all positive keys when everything fits) and the rate of the step
// tied at lam (0 if none).
__device__ __forceinline__ int64_t steps_and_tie(const uint64_t (&kk)[4], int64_t s, uint64_t lam,
                                                 bool all_fit, int* n) {
  int c = 0;
  int64_t tie = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (kk[k] == 0) continue;
    if (all_fit || kk[k] > lam) ++c;
    else if (kk[k] == lam) tie = step_rate(s, k);
  }
  *n = c;
  return all_fit ? 0 : tie;
}

// Block-wide inclusive scan (wave shuffles, then wave totals through LDS; integer: exact).
// Every thread of the block calls it.  wave_tot holds >= blockDim.x / 64 entries.
__device__ __forceinline__ int64_t block_scan_incl(int64_t v, int64_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int64_t off = 0;
  for (int w = 0; w < wave; ++w) off += wave_tot[w];
  __syncthreads();
  return v + off;
}

// Choose this pass's digit of one segment from its kBins-bin histogram.  NT threads (the
// whole block; it holds barriers), each owning kBins/NT consecutive bins in descending digit
// order.
template <int NT>
__device__ void select_digit(SelState* st, const int64_t* hist, const uint64_t* hmin,
                             const uint64_t* hmax, int pass, int nb, int64_t* wave_tot) {
  const SelState s = *st;
  constexpr int PER = kBins / NT;
  const int i = threadIdx.x;
  int64_t hv[PER];
  int64_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    hv[j] = hist[kBins - 1 - (PER * i + j)];
    mine += hv[j];
  }
  const int64_t incl_t = block_scan_incl(mine, wave_tot);
  if (s.done || s.none) return;               // uniform
  int64_t run = incl_t - mine;                 // cumulative weight of higher digits
  const bool last = (i == NT - 1);
  if (pass == 0 && last && incl_t <= s.brem) {
    st->all_fit = 1;                           // every positive step fits: lambda* = 0
    st->done = 1;
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t excl = run;
    run += hv[j];
    if (excl <= s.brem && run > s.brem) {      // exactly one bin overall
      const int digit = kBins - 1 - (PER * i + j);
      const Digit dg = digit_of(pass, nb);
      const uint64_t mn = hmin[digit], mx = hmax[digit];
      SelState n = s;
      n.brem = s.brem - excl;
      n.prefix = s.prefix | ((uint64_t)digit << dg.lo);
      if (mn == mx) {          // a single key value left in the bin: it is lambda*
        n.prefix = mn;
        n.done = 1;
      } else if (dg.lo == 0) {
        n.done = 1;
      }
      *st = n;
    }
  }
}

// The multi-block path's digit choice.  Instead of per-bin extremes it has the smallest and
// largest key of the current prefix set (the keys of the bin chosen by the previous pass, all
// positive keys on pass 0): when they are equal that value is lambda* (the same value and budget
// the per-bin test finds one pass earlier).
template <int NT>
__device__ void select_digit_set(SelState* st, const int64_t* hist, uint64_t pmin, uint64_t pmax, int pass,
                                 int nb, int64_t* wave_tot) {
  const SelState s = *st;
  constexpr int PER = kBins / NT;
  const int i = threadIdx.x;
  int64_t hv[PER];
  int64_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    hv[j] = hist[kBins - 1 - (PER * i + j)];
    mine += hv[j];
  }
  const int64_t incl_t = block_scan_incl(mine, wave_tot);
  int64_t total = 0;                           // the block's wave totals stay in wave_tot
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) total += wave_tot[w];
  if (s.done || s.none) return;               // uniform
  if (pass == 0 && total <= s.brem) {          // every positive step fits: lambda* = 0
    if (i == 0) {
      st->all_fit = 1;
      st->done = 1;
    }
    return;
  }
  if (pmin == pmax) {                          // a single key value in the prefix set: lambda*
    if (i == 0) {
      SelState n = s;
      n.prefix = pmin;
      n.done = 1;
      *st = n;
    }
    return;
  }
  int64_t run = incl_t - mine;                 // cumulative weight of higher digits
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t excl = run;
    run += hv[j];
    if (excl <= s.brem && run > s.brem) {      // exactly one bin overall
      const int digit = kBins - 1 - (PER * i + j);
      const Digit dg = digit_of(pass, nb);
      SelState n = s;
      n.brem = s.brem - excl;
      n.prefix = s.prefix | ((uint64_t)digit << dg.lo);
      if (dg.lo == 0) n.done = 1;
      *st = n;
    }
  }
}

constexpr int kCountBlock = 4096;      // tokens per block of alloc_count (256 threads x 16)

// K stage: retained tokens (bits_v > 0) of each head, per 4096-token block, and invalid widths.
__global__ void __launch_bounds__(256)
alloc_count(const uint8_t* __restrict__ bits_v, int64_t N, int ncb, int32_t* __restrict__ rpart,
            int32_t* __restrict__ rbad) {
  __shared__ int32_t wsum[4], wbad[4];
  const int blk = blockIdx.x, g = blockIdx.y;
  const int64_t t0 = (int64_t)blk * kCountBlock + threadIdx.x * 16;
  const uint8_t* src = bits_v + (int64_t)g * N + t0;
  int cnt = 0;
  bool bad = false;
  if (t0 + 15 < N && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    const uint4 w = *reinterpret_cast<const uint4*>(src);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t b = (ww[i] >> (8 * j)) & 0xFFu;
        cnt += (b > 0);
        bad |= !valid_width(b);
      }
  } else {
    for (int j = 0; j < 16; ++j) {
      if (t0 + j < N) {
        const uint32_t b = src[j];
        cnt += (b > 0);
        bad |= !valid_width(b);
      }
    }
  }
  int bi = bad ? 1 : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    cnt += __shfl_xor(cnt, o, 64);
    bi |= __shfl_xor(bi, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    wsum[wave] = cnt;
    wbad[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    rpart[(int64_t)g * ncb + blk] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    rbad[(int64_t)g * ncb + blk] = wbad[0] | wbad[1] | wbad[2] | wbad[3];
  }
}

// R_g = sum of the head's block counts (integer: order-free), computed by a whole block of NT
// threads into rc[Hkv] (LDS, zeroed by the caller); returns whether any width was invalid.
template <typename T>
__device__ __forceinline__ void sum_counts(const int32_t* rpart, const int32_t* rbad, int Hkv,
                                           int ncb, T* rc, int32_t* bad) {
  for (int64_t i = threadIdx.x; i < (int64_t)Hkv * ncb; i += blockDim.x) {
    const int g = (int)(i / ncb);
    const int32_t v = rpart[i];
    if (v) atomicAdd(&rc[g], (T)v);
    if (rbad[i]) *bad = 1;
  }
}

// ======================= single-block path (V/K stages, <= 2048 units) ===================
__global__ void __launch_bounds__(1024)
alloc_small(const float* __restrict__ weight, const float* __restrict__ sigma,
            const int32_t* __restrict__ rpart, const int32_t* __restrict__ rbad, int ncb,
            int stage, int Hkv, int64_t N, int d, double avg,
            uint8_t* __restrict__ bits_out, kvc_alloc_result* result, int32_t* status) {
  __shared__ uint64_t keys[kSmallUnits * 4];
  __shared__ int64_t hist[kBins];
  __shared__ uint64_t hmin[kBins], hmax[kBins];
  __shared__ int64_t wave_tot[16];
  __shared__ int32_t rc[256];
  __shared__ SelState st;
  __shared__ int32_t bad;
  __shared__ double dbuf[16];
  __shared__ unsigned long long kmin, kmax;
  __shared__ int nbits;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int U = (stage == KVC_ALLOC_V_TOKENS) ? (int)(Hkv * N) : Hkv * d;
  // thread tid owns units 2 tid and 2 tid + 1 (U <= 2048) throughout; their costs are read
  // first, so the load overlaps the count of retained tokens
  float cw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = 2 * tid + j;
    float c = 0.f;
    if (u < U) {
      c = weight[u];
      if (sigma) c = c * sigma[u];
    }
    cw[j] = c;
  }
  if (tid == 0) {
    bad = 0;
    kmin = ~0ull;
    kmax = 0;
  }
  for (int g = tid; g < Hkv; g += 1024) rc[g] = 0;
  __syncthreads();
  if (stage == KVC_ALLOC_K_CHANNELS) sum_counts(rpart, rbad, Hkv, ncb, rc, &bad);
  __syncthreads();
  if (tid == 0) {
    int64_t E;
    if (stage == KVC_ALLOC_V_TOKENS) {
      E = (int64_t)Hkv * N * d;
    } else {
      int64_t r = 0;
      for (int g = 0; g < Hkv; ++g) r += rc[g];
      E = (int64_t)d * r;
    }
    st.prefix = 0;
    st.budget = (int64_t)floor(avg * (double)E);
    st.brem = st.budget;
    st.all_fit = 0;
    st.none = 0;
    st.done = 0;
    st.pad = 0;
    *status = bad ? KVC_DEV_BAD_WIDTH : 0;
  }
  uint64_t tmn = ~0ull, tmx = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = 2 * tid + j;
    if (u >= U) continue;
    const int64_t s = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)d : (int64_t)rc[u / d];
    uint64_t kk[4];
    unit_keys(cw[j], s, kk);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      keys[u * 4 + k] = kk[k];
      if (kk[k] != 0) {
        tmn = kk[k] < tmn ? kk[k] : tmn;
        tmx = kk[k] > tmx ? kk[k] : tmx;
      }
    }
  }
  // The radix select starts at the highest bit in which the positive keys differ: the bits
  // above it are the same for all of them and become the starting prefix, so the first digit
  // already spreads the keys over many bins (few colliding LDS atomics, earlier single-value
  // bins).
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t a = __shfl_xor(tmn, o, 64), b = __shfl_xor(tmx, o, 64);
    tmn = a < tmn ? a : tmn;
    tmx = b > tmx ? b : tmx;
  }
  if (lane == 0) {
    atomicMin(&kmin, (unsigned long long)tmn);
    atomicMax(&kmax, (unsigned long long)tmx);
  }
  __syncthreads();
  if (tid == 0) {
    int nb = 64;
    if (kmax != 0) {
      const uint64_t x = kmin ^ kmax;
      nb = x ? 64 - __clzll((long long)x) : 1;
      if (nb < 64) st.prefix = kmin & (~0ull << nb);
    }
    nbits = nb;
  }
  __syncthreads();
  const int nbk = nbits;
  const int npass = passes_of(nbk);
  for (int pass = 0; pass < npass; ++pass) {
    __syncthreads();
    if (st.done) break;                         // uniform: read after a barrier
    for (int b = tid; b < kBins; b += 1024) {
      hist[b] = 0;
      hmin[b] = ~0ull;
      hmax[b] = 0;
    }
    __syncthreads();
    const Digit dg = digit_of(pass, nbk);
    const uint64_t pre = st.prefix & dg.himask;
    const uint64_t dmask = (1ull << (dg.hi - dg.lo)) - 1;
    for (int e = tid; e < U * 4; e += 1024) {
      const uint64_t key = keys[e];
      if (key != 0 && (key & dg.himask) == pre) {
        const int u = e >> 2, k = e & 3;
        const int64_t s = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)d : (int64_t)rc[u / d];
        const int b = (int)((key >> dg.lo) & dmask);
        atomicAdd((unsigned long long*)&hist[b], (unsigned long long)step_rate(s, k));
        atomicMin((unsigned long long*)&hmin[b], (unsigned long long)key);
        atomicMax((unsigned long long*)&hmax[b], (unsigned long long)key);
      }
    }
    __syncthreads();
    select_digit<1024>(&st, hist, hmin, hmax, pass, nbk, wave_tot);
  }
  __syncthreads();
  const SelState S = st;
  const uint64_t lam = S.all_fit ? 0ull : S.prefix;
  // ordered tie scan: thread i owns units [2i, 2i + 2)
  int64_t tie[2] = {0, 0};
  int n[2] = {0, 0};
  int64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = 2 * tid + j;
    if (u < U) {
      uint64_t kk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) kk[k] = keys[u * 4 + k];
      const int64_t s = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)d : (int64_t)rc[u / d];
      tie[j] = steps_and_tie(kk, s, lam, S.all_fit != 0, &n[j]);
      tsum += tie[j];
    }
  }
  const int64_t incl = block_scan_incl(tsum, wave_tot);
  int64_t run = incl - tsum;
  int64_t used = 0;
  double dist = 0.0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = 2 * tid + j;
    if (u >= U) continue;
    int nn = n[j];
    if (tie[j] > 0) {
      run += tie[j];
      if (run <= S.brem) nn += 1;
    }
    const uint32_t b = kLevels[nn];
    bits_out[u] = (uint8_t)b;
    const int64_t s = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)d : (int64_t)rc[u / d];
    used += s * (int64_t)b;
    dist += ldexp((double)cw[j], -(int)b);
  }
  const int64_t used_tot = block_scan_incl(used, wave_tot);
  // distortion: fixed-order tree within each wave, then the 16 wave sums in order
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double t = __shfl_down(dist, o, 64);
    if (lane < o) dist += t;
  }
  if (lane == 0) dbuf[wave] = dist;
  __syncthreads();
  if (tid == 1023 && result) {
    double dt = 0.0;
    for (int w = 0; w < 16; ++w) dt += dbuf[w];
    kvc_alloc_result r;
    r.lambda = S.all_fit ? 0.0 : __longlong_as_double((long long)S.prefix);
    r.budget_bits = S.budget;
    r.used_bits = used_tot;
    r.distortion = dt;
    *result = r;
  }
}

// ======================= multi-block path =================================================

// Count R_g (K stage), set the budgets, clear the first pass's histogram.  One block.
__global__ void __launch_bounds__(1024)
alloc_begin(AllocWs a, int stage, int nseg, int Hkv, int64_t N, int d, int ncb, double avg,
            double keep_fraction) {
  __shared__ int64_t rsum;
  __shared__ int32_t bad;
  __shared__ unsigned long long rc[256];
  const int tid = threadIdx.x;
  if (tid == 0) {
    rsum = 0;
    bad = 0;
  }
  if (tid < 256) rc[tid] = 0;
  for (int64_t i = tid; i < (int64_t)nseg * kBins; i += 1024) a.hist[i] = 0;
  for (int i = tid; i < nseg; i += 1024) {
    a.pmin[i] = ~0ull;
    a.pmax[i] = 0;
  }
  __syncthreads();
  if (stage == KVC_ALLOC_K_CHANNELS) sum_counts(a.rpart, a.rbad, Hkv, ncb, rc, &bad);
  __syncthreads();
  if (stage == KVC_ALLOC_K_CHANNELS && tid < Hkv) a.rcount[tid] = (int64_t)rc[tid];
  if (tid == 0) {
    *a.status = bad ? KVC_DEV_BAD_WIDTH : 0;
    if (stage == KVC_ALLOC_K_CHANNELS)
      for (int g = 0; g < Hkv; ++g) rsum += (int64_t)rc[g];
  }
  __syncthreads();
  for (int sgi = tid; sgi < nseg; sgi += 1024) {
    SelState s;
    s.prefix = 0;
    s.all_fit = 0;
    s.none = 0;
    s.done = 0;
    s.pad = 0;
    if (stage == KVC_ALLOC_TOPK) {
      const int64_t kk = (int64_t)floor(keep_fraction * (double)N);
      s.budget = kk;
      s.brem = kk - 1;           // the kk-th largest: count above <= kk-1 < count at-or-above
      s.none = (kk == 0);
    } else {
      const int64_t E = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)Hkv * N * d : (int64_t)d * rsum;
      s.budget = (int64_t)floor(avg * (double)E);
      s.brem = s.budget;
    }
    a.st[sgi] = s;
  }
}

__device__ __forceinline__ int64_t unit_size(int stage, int d, int64_t u, const int64_t* rcount) {
  return stage == KVC_ALLOC_V_TOKENS ? (int64_t)d : rcount[u / d];
}

// Cheap bounds on the four step keys of a unit (cost c > 0, size s > 0), as float64 bit patterns:
// the keys in float32 (c * (theta_num / theta_den) * (1 / s), five roundings, within 2^-21.6 of the
// exact quotient), widened to a float64 pattern.  Positive doubles order like their patterns, and
// within 2^-21.6 of a value the pattern moves by less than 2^31.5, so the exact key's pattern lies
// in [ak - kKeyMargin, ak + kKeyMargin].  false when an estimate is not a normal float32 (then only
// the exact keys may decide).
constexpr uint64_t kKeyMargin = 1ull << 33;
__constant__ float kThetaF[4] = {0.375f, 0.09375f, 0.0146484375f, 255.0f / 524288.0f};

__device__ __forceinline__ bool key_bounds(float c, int64_t s, uint64_t (&ak)[4]) {
  const float inv = 1.0f / (float)s;
  bool ok = true;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t b = __float_as_uint((c * kThetaF[k]) * inv);
    const uint32_t e = b >> 23;                // c > 0: the sign bit is clear
    ok = ok && e > 0u && e < 255u;
    ak[k] = ((uint64_t)(e + 896u) << 52) | ((uint64_t)(b & 0x7FFFFFu) << 29);
  }
  return ok;
}

// Whether some step key of the unit may carry the prefix `pre` (pattern bits at and above bit hi).
__device__ __forceinline__ bool may_carry(float c, int64_t s, uint64_t pre, int hi) {
  if (!(c > 0.f) || s <= 0) return false;     // no positive key
  if (hi >= 64) return true;                  // the first pass takes every key
  uint64_t ak[4];
  if (!key_bounds(c, s, ak)) return true;
  const uint64_t end = pre + (1ull << hi);     // the prefix set is [pre, end)
  bool any = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t lo = ak[k] > kKeyMargin ? ak[k] - kKeyMargin : 0ull;
    any = any || (ak[k] + kKeyMargin >= pre && lo < end);
  }
  return any;
}

// The values a thread's UPT units are decided by, all requested before any is used: the cost
// c_u = float32(w_u * sigma_u) (V/K stages; the same product as everywhere else, so the same bits)
// or the score (top-k).  Unit j is ubase + j * ustep of the segment at woff; units past seg_len
// read the segment's last unit (always in bounds) and are never used.  A loop that loaded each
// unit where it is needed waited one memory round trip per unit.
template <int UPT>
__device__ __forceinline__ void load_costs(const float* __restrict__ weight, const float* __restrict__ sigma,
                                           int64_t woff, int64_t ubase, int64_t ustep, int64_t seg_len,
                                           float (&cw)[UPT]) {
  float sg[UPT];
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int64_t u = ubase + j * ustep;
    const int64_t uc = u < seg_len ? u : seg_len - 1;
    cw[j] = weight[woff + uc];
    sg[j] = sigma ? sigma[uc] : 1.0f;
  }
  if (sigma) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) cw[j] = cw[j] * sg[j];
  }
}

// Histogram of one pass over the keys of the current prefix set.  V/K: the 4 step keys of each
// unit, weight = step rate.  Top-k: 32-bit score keys, 1 per token, weight 1, one segment per KV
// head.  The set's smallest and largest keys go out once per block.
template <bool TOPK, int UPT, int NT>
__global__ void __launch_bounds__(NT)
alloc_hist(AllocWs a, const float* __restrict__ weight, const float* __restrict__ sigma,
           int64_t seg_len, int stage, int d, int pass, int nb) {
  __shared__ int64_t h[kBins];
  __shared__ uint64_t wmn[NT / 64], wmx[NT / 64];
  const int seg = blockIdx.y;
  const SelState s = a.st[seg];
  if (s.done || s.none) return;                // uniform for the block
  for (int b = threadIdx.x; b < kBins; b += NT) h[b] = 0;
  __syncthreads();
  uint64_t kmn = ~0ull, kmx = 0;               // extremes of this thread's keys in the prefix set
  int rb[4] = {-1, -1, -1, -1};                // V/K: per step, the bin of the current run and its rates
  int64_t rs[4] = {0, 0, 0, 0};
  const Digit dg = digit_of(pass, nb);
  const uint64_t pre = s.prefix & dg.himask;
  const uint64_t dmask = (1ull << (dg.hi - dg.lo)) - 1;
  const int64_t base = (int64_t)blockIdx.x * (NT * UPT);
  float cw[UPT];
  load_costs<UPT>(weight, TOPK ? nullptr : sigma, TOPK ? (int64_t)seg * seg_len : 0, base + threadIdx.x, NT,
                  seg_len, cw);
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int64_t ul = base + threadIdx.x + j * NT;
    if (ul >= seg_len) continue;
    if (TOPK) {
      const uint64_t key = score_key(cw[j]);
      if ((key & dg.himask) == pre) {
        const int b = (int)((key >> dg.lo) & dmask);
        atomicAdd((unsigned long long*)&h[b], 1ull);
        kmn = key < kmn ? key : kmn;
        kmx = key > kmx ? key : kmx;
      }
    } else {
      // A key's prefix and digit come from its float32 bounds when the whole interval
      // [ak - margin, ak + margin] that holds the exact key shares its bits at and above the digit's
      // lowest bit: on the first passes, whose digit cells (2^53 and 2^42 patterns) are far wider
      // than the margin (2^33), nearly every key.  Only the units with a key across a cell edge, or
      // with estimates that are not normal floats, compute the float64 quotients, and then only
      // where their bounds may reach the prefix set (after the first passes, few units).  A key
      // decided by its bounds enters the set's extremes as its interval, so the extremes then differ
      // and the single-value exit waits for a pass on exact keys: the selection stays exact.
      // Key k of a thread's units often falls in the same bin as the previous one (nearly always on
      // the first passes, where the bins are exponent ranges): each k's rates are summed in
      // registers while the bin repeats, so the LDS atomics, which serialise on a shared address,
      // come once per run.
      const int64_t sz = unit_size(stage, d, ul, a.rcount);
      const float cu = cw[j];
      if (!(cu > 0.f) || sz <= 0) continue;      // no positive key
      uint64_t ak[4], klo[4], khi[4];
      bool by_bounds = key_bounds(cu, sz, ak);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        klo[k] = ak[k] > kKeyMargin ? ak[k] - kKeyMargin : 0ull;
        khi[k] = ak[k] + kKeyMargin;
        by_bounds = by_bounds && (klo[k] >> dg.lo) == (khi[k] >> dg.lo);
      }
      uint64_t kk[4];
      if (by_bounds) {
#pragma unroll
        for (int k = 0; k < 4; ++k) kk[k] = ak[k];
      } else {
        if (!may_carry(cu, sz, pre, dg.hi)) continue;
        unit_keys(cu, sz, kk);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          klo[k] = kk[k];
          khi[k] = kk[k];
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (kk[k] != 0 && (kk[k] & dg.himask) == pre) {
          const int b = (int)((kk[k] >> dg.lo) & dmask);
          const int64_t r = step_rate(sz, k);
          if (b != rb[k]) {
            if (rb[k] >= 0) atomicAdd((unsigned long long*)&h[rb[k]], (unsigned long long)rs[k]);
            rb[k] = b;
            rs[k] = r;
          } else {
            rs[k] += r;
          }
          kmn = klo[k] < kmn ? klo[k] : kmn;
          kmx = khi[k] > kmx ? khi[k] : kmx;
        }
      }
    }
  }
  if (!TOPK) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (rb[k] >= 0) atomicAdd((unsigned long long*)&h[rb[k]], (unsigned long long)rs[k]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t mo = __shfl_xor(kmn, o, 64), xo = __shfl_xor(kmx, o, 64);
    kmn = mo < kmn ? mo : kmn;
    kmx = xo > kmx ? xo : kmx;
  }
  if ((threadIdx.x & 63) == 0) {
    wmn[threadIdx.x >> 6] = kmn;
    wmx[threadIdx.x >> 6] = kmx;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += NT) {
    if (h[b]) atomicAdd((unsigned long long*)&a.hist[(int64_t)seg * kBins + b], (unsigned long long)h[b]);
  }
  if (threadIdx.x == 0) {
    uint64_t mn = wmn[0], mx = wmx[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
      mn = wmn[w] < mn ? wmn[w] : mn;
      mx = wmx[w] > mx ? wmx[w] : mx;
    }
    if (mn <= mx) {                            // the block saw keys of the prefix set
      atomicMin((unsigned long long*)&a.pmin[seg], (unsigned long long)mn);
      atomicMax((unsigned long long*)&a.pmax[seg], (unsigned long long)mx);
    }
  }
}

// Digit choice of one pass (one block per segment), then clear the histogram for the next.
__global__ void __launch_bounds__(256)
alloc_select(AllocWs a, int pass, int nb) {
  __shared__ int64_t wave_tot[4];
  const int seg = blockIdx.x;
  SelState* st = &a.st[seg];
  if (st->done || st->none) return;            // uniform
  int64_t* hist = a.hist + (int64_t)seg * kBins;
  select_digit_set<256>(st, hist, a.pmin[seg], a.pmax[seg], pass, nb, wave_tot);
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += 256) hist[b] = 0;
  if (threadIdx.x == 0) {
    a.pmin[seg] = ~0ull;
    a.pmax[seg] = 0;
  }
}

// cu: the unit's cost (V/K) or score (top-k), from load_costs.
template <bool TOPK>
__device__ __forceinline__ int64_t unit_tie(const AllocWs& a, float cu, int64_t u, int64_t seg_len, int stage,
                                            int d, const SelState& s, int* n) {
  if (u >= seg_len) {
    *n = 0;
    return 0;
  }
  if (TOPK) {
    if (s.none) {
      *n = 0;
      return 0;
    }
    const uint64_t key = score_key(cu);
    *n = key > s.prefix ? 1 : 0;
    return key == s.prefix ? 1 : 0;
  }
  const float c = cu;
  const int64_t sz = unit_size(stage, d, u, a.rcount);
  if (!(c > 0.f) || sz <= 0) {                 // no positive key: no step, no tie
    *n = 0;
    return 0;
  }
  if (s.all_fit) {                             // every positive step is taken
    *n = 4;
    return 0;
  }
  uint64_t ak[4];
  if (key_bounds(c, sz, ak)) {                 // decided by the bounds unless a key may equal lambda*
    int cnt = 0;
    bool near = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t lo = ak[k] > kKeyMargin ? ak[k] - kKeyMargin : 0ull;
      cnt += lo > s.prefix ? 1 : 0;
      near = near || (lo <= s.prefix && ak[k] + kKeyMargin >= s.prefix);
    }
    if (!near) {
      *n = cnt;
      return 0;
    }
  }
  uint64_t kk[4];
  unit_keys(c, sz, kk);
  return steps_and_tie(kk, sz, s.prefix, false, n);
}

// Block sums of the tie rates (units in index order, UPT per thread).
template <bool TOPK, int UPT>
__global__ void __launch_bounds__(256)
alloc_ties(AllocWs a, const float* __restrict__ weight, const float* __restrict__ sigma,
           int64_t seg_len, int stage, int d) {
  __shared__ int64_t wave_tot[4];
  const int seg = blockIdx.y;
  const SelState s = a.st[seg];
  const int64_t base = (int64_t)blockIdx.x * (256 * UPT) + threadIdx.x * UPT;
  float cw[UPT];
  load_costs<UPT>(weight, TOPK ? nullptr : sigma, TOPK ? (int64_t)seg * seg_len : 0, base, 1, seg_len, cw);
  int64_t t = 0;
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    int n;
    t += unit_tie<TOPK>(a, cw[j], base + j, seg_len, stage, d, s, &n);
  }
  const int64_t tot = block_scan_incl(t, wave_tot);
  if (threadIdx.x == 255) a.bsum[(int64_t)seg * gridDim.x + blockIdx.x] = tot;
}

// Final widths: steps with key > lambda*, plus the tied step while the inclusive prefix of tie
// rates fits the remaining budget; per-block used rate and distortion.
template <bool TOPK, int UPT>
__global__ void __launch_bounds__(256)
alloc_assign(AllocWs a, const float* __restrict__ weight, const float* __restrict__ sigma,
             int64_t seg_len, int stage, int d, int keep_bits, uint8_t* __restrict__ bits_out) {
  __shared__ int64_t wave_tot[4];
  __shared__ double dbuf[4];
  __shared__ int64_t prefix_sh;
  const int seg = blockIdx.y;
  const SelState s = a.st[seg];
  const int64_t base = (int64_t)blockIdx.x * (256 * UPT) + threadIdx.x * UPT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float cw[UPT];
  load_costs<UPT>(weight, TOPK ? nullptr : sigma, TOPK ? (int64_t)seg * seg_len : 0, base, 1, seg_len, cw);
  int64_t tie[UPT];
  int n[UPT];
  int64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    tie[j] = unit_tie<TOPK>(a, cw[j], base + j, seg_len, stage, d, s, &n[j]);
    tsum += tie[j];
  }
  const int64_t incl = block_scan_incl(tsum, wave_tot);
  // tie rates of the segment's earlier blocks (at most kMaxBlocks sums, read by the whole block;
  // integers, so the order of the additions does not matter)
  int64_t before = 0;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += 256) before += a.bsum[(int64_t)seg * gridDim.x + b];
  before = block_scan_incl(before, wave_tot);
  if (threadIdx.x == 255) prefix_sh = before;
  __syncthreads();
  int64_t run = prefix_sh + incl - tsum;
  const int64_t cap = TOPK ? s.brem + 1 : s.brem;
  int64_t used = 0;
  double dist = 0.0;
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int64_t u = base + j;
    if (u >= seg_len) continue;
    int nn = n[j];
    if (tie[j] > 0) {
      run += tie[j];
      if (run <= cap) nn += 1;
    }
    const uint32_t b = TOPK ? (nn ? (uint32_t)keep_bits : 0u) : kLevels[nn];
    bits_out[(int64_t)seg * seg_len + u] = (uint8_t)b;
    if (TOPK) {
      used += (int64_t)b * d;
    } else {
      used += unit_size(stage, d, u, a.rcount) * (int64_t)b;
      dist += ldexp((double)cw[j], -(int)b);
    }
  }
  const int64_t used_blk = block_scan_incl(used, wave_tot);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double t = __shfl_down(dist, o, 64);
    if (lane < o) dist += t;
  }
  if (lane == 0) dbuf[wave] = dist;
  __syncthreads();
  if (threadIdx.x == 255) {
    a.used_part[(int64_t)seg * gridDim.x + blockIdx.x] = used_blk;
    a.dist_part[(int64_t)seg * gridDim.x + blockIdx.x] = (dbuf[0] + dbuf[1]) + (dbuf[2] + dbuf[3]);
  }
}

// Sum the per-block used rate and distortion and write the result.  256 threads each sum a
// contiguous range of parts in order; the 256 sums are combined by a fixed tree.
__global__ void __launch_bounds__(256)
alloc_finalize(const AllocWs a, int nparts, int topk, kvc_alloc_result* result) {
  __shared__ int64_t us[256];
  __shared__ double ds[256];
  if (result == nullptr) return;
  const int tid = threadIdx.x;
  const int per = (nparts + 255) / 256;
  int64_t ut = 0;
  double dt = 0.0;
  for (int i = tid * per; i < (tid + 1) * per && i < nparts; ++i) {
    ut += a.used_part[i];
    dt += a.dist_part[i];
  }
  us[tid] = ut;
  ds[tid] = dt;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) {
      us[tid] += us[tid + w];
      ds[tid] += ds[tid + w];
    }
    __syncthreads();
  }
  if (tid != 0) return;
  kvc_alloc_result r;
  if (topk) {
    r.lambda = 0.0;
    r.budget_bits = us[0];
    r.used_bits = us[0];
    r.distortion = 0.0;
  } else {
    const SelState s0 = a.st[0];
    r.lambda = s0.all_fit ? 0.0 : __longlong_as_double((long long)s0.prefix);
    r.budget_bits = s0.budget;
    r.used_bits = us[0];
    r.distortion = ds[0];
  }
  *result = r;
}

struct Plan {
  int nseg, nblk, nb, upt;
  int64_t U, seg_len;
  bool small;
};

Plan plan_of(const Layer& L, int stage) {
  Plan p;
  if (stage == KVC_ALLOC_TOPK) {
    p.nseg = L.hkv;
    p.seg_len = L.n;
    p.U = L.n * L.hkv;
    p.nb = 32;
  } else {
    p.nseg = 1;
    p.U = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)L.hkv * L.n : (int64_t)L.hkv * L.d;
    p.seg_len = p.U;
    p.nb = 64;
  }
  p.small = (stage != KVC_ALLOC_TOPK) && p.U <= kSmallUnits;
  p.upt = 1;
  while (p.upt < 16 && (int64_t)p.nseg * ((p.seg_len + 256 * p.upt - 1) / (256 * p.upt)) > kMaxBlocks)
    p.upt *= 2;
  p.nblk = (int)((p.seg_len + 256 * p.upt - 1) / (256 * p.upt));
  return p;
}

AllocWs carve(const Layer& L, int stage, char* ws, size_t* total) {
  const Plan p = plan_of(L, stage);
  WsPlan w;
  AllocWs a{};
  const size_t hn = (size_t)p.nseg * kBins;
  const size_t o_st = w.take(sizeof(SelState) * p.nseg);
  const size_t o_h = w.take(sizeof(int64_t) * hn);
  const size_t o_mn = w.take(sizeof(uint64_t) * (size_t)p.nseg);
  const size_t o_mx = w.take(sizeof(uint64_t) * (size_t)p.nseg);
  const int ncb = (int)((L.n + kCountBlock - 1) / kCountBlock);
  const bool kst = (stage == KVC_ALLOC_K_CHANNELS);
  const size_t o_rp = w.take(kst ? sizeof(int32_t) * L.hkv * ncb : 0);
  const size_t o_rb = w.take(kst ? sizeof(int32_t) * L.hkv * ncb : 0);
  const size_t o_r = w.take(sizeof(int64_t) * L.hkv);
  const size_t o_b = w.take(sizeof(int64_t) * p.nseg * p.nblk);
  const size_t o_u = w.take(sizeof(int64_t) * p.nseg * p.nblk);
  const size_t o_d = w.take(sizeof(double) * p.nseg * p.nblk);
  if (total) *total = w.off;
  if (ws) {
    a.status = reinterpret_cast<int32_t*>(ws);
    a.st = reinterpret_cast<SelState*>(ws + o_st);
    a.hist = reinterpret_cast<int64_t*>(ws + o_h);
    a.pmin = reinterpret_cast<uint64_t*>(ws + o_mn);
    a.pmax = reinterpret_cast<uint64_t*>(ws + o_mx);
    a.rpart = reinterpret_cast<int32_t*>(ws + o_rp);
    a.rbad = reinterpret_cast<int32_t*>(ws + o_rb);
    a.rcount = reinterpret_cast<int64_t*>(ws + o_r);
    a.bsum = reinterpret_cast<int64_t*>(ws + o_b);
    a.used_part = reinterpret_cast<int64_t*>(ws + o_u);
    a.dist_part = reinterpret_cast<double*>(ws + o_d);
  }
  return a;
}

// The selection passes, tie sums and assignment at UPT units per thread.
template <int UPT>
void launch_passes(const AllocWs& a, const Plan& p, const Layer& L, int stage, const float* weight,
                   const float* sigma, int keep_bits, uint8_t* bits_out, hipStream_t s) {
  const bool topk = (stage == KVC_ALLOC_TOPK);
  const dim3 g2((unsigned)p.nblk, (unsigned)p.nseg);
  const int64_t gh = (p.seg_len + 1024 * kHistUpt - 1) / (1024 * kHistUpt);
  const int npass = passes_of(p.nb);
  for (int pass = 0; pass < npass; ++pass) {
    if (topk)
      alloc_hist<true, UPT, 256><<<g2, 256, 0, s>>>(a, weight, nullptr, p.seg_len, stage, L.d, pass, p.nb);
    else if (gh >= 256)   // a large stage: 1024-thread blocks, one per compute unit, each flushing its
                          // LDS bins to the global histogram once for four times the units
      alloc_hist<false, kHistUpt, 1024><<<dim3((unsigned)gh), 1024, 0, s>>>(a, weight, sigma, p.seg_len, stage, L.d,
                                                                       pass, p.nb);
    else
      alloc_hist<false, UPT, 256><<<g2, 256, 0, s>>>(a, weight, sigma, p.seg_len, stage, L.d, pass, p.nb);
    alloc_select<<<p.nseg, 256, 0, s>>>(a, pass, p.nb);
  }
  if (topk) {
    alloc_ties<true, UPT><<<g2, 256, 0, s>>>(a, weight, nullptr, p.seg_len, stage, L.d);
    alloc_assign<true, UPT><<<g2, 256, 0, s>>>(a, weight, nullptr, p.seg_len, stage, L.d, keep_bits, bits_out);
  } else {
    alloc_ties<false, UPT><<<g2, 256, 0, s>>>(a, weight, sigma, p.seg_len, stage, L.d);
    alloc_assign<false, UPT><<<g2, 256, 0, s>>>(a, weight, sigma, p.seg_len, stage, L.d, keep_bits, bits_out);
  }
}

}  // namespace

size_t alloc_ws_bytes(const Layer& L, int stage) {
  size_t total = 0;
  carve(L, stage, nullptr, &total);
  return total;
}

hipError_t launch_allocate(const Layer& L, int stage, const float* weight, const float* sigma,
                           const uint8_t* bits_v, double avg_bits, double keep_fraction,
                           int keep_bits, uint8_t* bits_out, kvc_alloc_result* result,
                           char* ws, hipStream_t s) {
  const Plan p = plan_of(L, stage);
  if (p.nseg > kMaxSeg) return hipErrorInvalidValue;
  AllocWs a = carve(L, stage, ws, nullptr);
  const int ncb = (int)((L.n + kCountBlock - 1) / kCountBlock);
  if (stage == KVC_ALLOC_K_CHANNELS)
    alloc_count<<<dim3((unsigned)ncb, (unsigned)L.hkv), 256, 0, s>>>(bits_v, L.n, ncb, a.rpart, a.rbad);
  if (p.small) {
    alloc_small<<<1, 1024, 0, s>>>(weight, sigma, a.rpart, a.rbad, ncb, stage, L.hkv, L.n, L.d,
                                   avg_bits, bits_out, result, a.status);
    return hipGetLastError();
  }
  const bool topk = (stage == KVC_ALLOC_TOPK);
  alloc_begin<<<1, 1024, 0, s>>>(a, stage, p.nseg, L.hkv, L.n, L.d, ncb, avg_bits, keep_fraction);
  switch (p.upt) {
    case 1: launch_passes<1>(a, p, L, stage, weight, sigma, keep_bits, bits_out, s); break;
    case 2: launch_passes<2>(a, p, L, stage, weight, sigma, keep_bits, bits_out, s); break;
    case 4: launch_passes<4>(a, p, L, stage, weight, sigma, keep_bits, bits_out, s); break;
    case 8: launch_passes<8>(a, p, L, stage, weight, sigma, keep_bits, bits_out, s); break;
    default: launch_passes<16>(a, p, L, stage, weight, sigma, keep_bits, bits_out, s); break;
  }
  alloc_finalize<<<1, 256, 0, s>>>(a, p.nblk * p.nseg, topk ? 1 : 0, result);
  return hipGetLastError();
}

}  // namespace kvc
