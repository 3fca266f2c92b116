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
// weighted MSB-first radix select over the 64-bit patterns (8 passes of 8 bits: block-private
// LDS histograms of integer rates, one global integer histogram per pass, a one-block digit
// choice).  Integer histograms make the selection exact and order-independent.  The tie rule
// is an ordered exclusive scan over units (block sums, a one-block scan, then per-unit
// ranks).  Top-k uses the same machinery per KV head on order-preserving 32-bit score keys.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kUnitsPerBlock = 1024;   // 256 threads x 4 units
constexpr int kMaxSeg = 1024;          // segments (KV heads) for top-k

__constant__ uint32_t kThetaNum[4] = {3u, 3u, 15u, 255u};
__constant__ uint32_t kThetaDen[4] = {8u, 32u, 1024u, 524288u};
__constant__ uint32_t kLevels[5] = {0u, 2u, 4u, 8u, 16u};

struct SelState {
  uint64_t prefix;      // selected key bits so far
  int64_t brem;         // budget left for keys above the prefix
  int64_t budget;       // B
  int64_t elements;     // E (V/K) or kept tokens per head (top-k)
  int32_t all_fit;      // every positive key fits: lambda* = 0, no ties
  int32_t none;         // top-k with k == 0
  int64_t pad[2];
};

struct AllocWs {
  int32_t* status;
  SelState* st;         // [nseg]
  int64_t* hist;        // [passes][nseg][256]
  uint64_t* keys;       // [U][kpu]
  int64_t* rcount;      // [Hkv] retained tokens per head (K stage)
  int64_t* bsum;        // [nseg][nblk] tie rate per block
  int64_t* bexcl;       // [nseg][nblk]
  int64_t* used_part;   // [nseg][nblk]
  double* dist_part;    // [nseg][nblk]
};

// ---- stage setup -----------------------------------------------------------------------

// R_g = #tokens with bits_v > 0 (one block per head); a width outside {0,2,4,8,16} is a
// device data error.
__global__ void __launch_bounds__(256)
count_retained(const uint8_t* __restrict__ bits_v, int64_t N, int64_t* __restrict__ rcount,
               int32_t* status) {
  const int g = blockIdx.x;
  int64_t cnt = 0;
  bool bad = false;
  for (int64_t t = threadIdx.x; t < N; t += 256) {
    uint32_t b = bits_v[(int64_t)g * N + t];
    cnt += (b > 0);
    bad |= !valid_width(b);
  }
  __shared__ int64_t red[256];
  red[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (bad) set_status(status, KVC_DEV_BAD_WIDTH);
  if (threadIdx.x == 0) rcount[g] = red[0];
}

// Zero the histograms and set B.  stage: 0 V, 1 K, 2 top-k.
__global__ void __launch_bounds__(256)
alloc_init(SelState* st, int64_t* hist, int64_t hist_len, int stage, int nseg, int Hkv, int d,
           int64_t N, const int64_t* rcount, double avg, double keep_fraction) {
  for (int64_t i = threadIdx.x; i < hist_len; i += 256) hist[i] = 0;
  if (threadIdx.x == 0) {
    for (int sgi = 0; sgi < nseg; ++sgi) {
      SelState s;
      s.prefix = 0;
      s.all_fit = 0;
      s.none = 0;
      s.pad[0] = s.pad[1] = 0;
      if (stage == 0) {
        s.elements = (int64_t)Hkv * N * d;
        s.budget = (int64_t)floor(avg * (double)s.elements);
        s.brem = s.budget;
      } else if (stage == 1) {
        int64_t r = 0;
        for (int g = 0; g < Hkv; ++g) r += rcount[g];
        s.elements = (int64_t)d * r;
        s.budget = (int64_t)floor(avg * (double)s.elements);
        s.brem = s.budget;
      } else {
        int64_t kk = (int64_t)floor(keep_fraction * (double)N);
        s.elements = kk;
        s.budget = kk - 1;       // select the kk-th largest: count above <= kk-1 < count at-or-above
        s.brem = kk - 1;
        s.none = (kk == 0);
      }
      st[sgi] = s;
    }
  }
}

__device__ __forceinline__ int64_t unit_size(int stage, int d, int64_t u, const int64_t* rcount) {
  return stage == 0 ? (int64_t)d : rcount[u / d];
}

// Keys of the four steps of every unit (0 when the unit can never be granted bits).
__global__ void __launch_bounds__(256)
alloc_keys(const float* __restrict__ weight, const float* __restrict__ sigma, int64_t U, int stage,
           int d, const int64_t* __restrict__ rcount, uint64_t* __restrict__ keys) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= U) return;
  float c = weight[u];
  if (sigma) c = c * sigma[u];          // one float32 rounding of w * sigma
  const int64_t s = unit_size(stage, d, u, rcount);
  uint64_t kk[4] = {0, 0, 0, 0};
  if (c > 0.f && s > 0) {
    const double cd = (double)c;
    const double sd = (double)s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      double key = (cd * (double)kThetaNum[k]) / (sd * (double)kThetaDen[k]);
      kk[k] = __double_as_longlong(key);
    }
  }
  uint4* o = reinterpret_cast<uint4*>(keys + u * 4);
  o[0] = make_uint4((uint32_t)kk[0], (uint32_t)(kk[0] >> 32), (uint32_t)kk[1], (uint32_t)(kk[1] >> 32));
  o[1] = make_uint4((uint32_t)kk[2], (uint32_t)(kk[2] >> 32), (uint32_t)kk[3], (uint32_t)(kk[3] >> 32));
}

// Order-preserving 32-bit key of a float score (larger score -> larger key).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---- weighted radix select ---------------------------------------------------------------

// One pass of the MSB-first select.  V/K: 64-bit keys, 4 per unit, weight = step rate; top-k:
// 32-bit score keys, 1 per token, weight 1, one segment per KV head (grid.y).
template <bool TOPK>
__global__ void __launch_bounds__(256)
alloc_hist(const uint64_t* __restrict__ keys, const float* __restrict__ scores, int64_t U,
           int64_t seg_len, int stage, int d, const int64_t* __restrict__ rcount,
           const SelState* __restrict__ st, int64_t* __restrict__ hist, int pass, int nbytes) {
  const int seg = blockIdx.y;
  const SelState s = st[seg];
  if (s.all_fit || s.none) return;
  __shared__ int64_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int shift = 8 * (nbytes - 1 - pass);
  const uint64_t himask = (pass == 0) ? 0ull : (~0ull << (shift + 8));
  const int64_t base = (int64_t)blockIdx.x * kUnitsPerBlock;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t ul = base + threadIdx.x + j * 256;
    if (TOPK) {
      if (ul < seg_len) {
        uint64_t key = score_key(scores[(int64_t)seg * seg_len + ul]);
        if ((key & himask) == (s.prefix & himask)) atomicAdd((unsigned long long*)&h[(key >> shift) & 255], 1ull);
      }
    } else {
      if (ul < U) {
        const int64_t sz = unit_size(stage, d, ul, rcount);
        const uint4* kp = reinterpret_cast<const uint4*>(keys + ul * 4);
        uint4 a = kp[0], b = kp[1];
        uint64_t kk[4] = {(uint64_t)a.x | ((uint64_t)a.y << 32), (uint64_t)a.z | ((uint64_t)a.w << 32),
                          (uint64_t)b.x | ((uint64_t)b.y << 32), (uint64_t)b.z | ((uint64_t)b.w << 32)};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (kk[k] != 0 && (kk[k] & himask) == (s.prefix & himask)) {
            int64_t w = sz * (int64_t)(kLevels[k + 1] - kLevels[k]);
            atomicAdd((unsigned long long*)&h[(kk[k] >> shift) & 255], (unsigned long long)w);
          }
        }
      }
    }
  }
  __syncthreads();
  int64_t v = h[threadIdx.x];
  if (v) atomicAdd((unsigned long long*)&hist[((int64_t)pass * gridDim.y + seg) * 256 + threadIdx.x], (unsigned long long)v);
}

// Choose this pass's digit: scanning digits from high to low, the first whose inclusive
// cumulative weight exceeds the remaining budget.  One block per segment.
__global__ void __launch_bounds__(256)
alloc_select(SelState* st, const int64_t* __restrict__ hist, int pass, int nbytes, int nseg) {
  const int seg = blockIdx.x;
  SelState s = st[seg];
  if (s.all_fit || s.none) return;
  const int i = threadIdx.x;                  // position in descending digit order
  const int digit = 255 - i;
  const int64_t hv = hist[((int64_t)pass * nseg + seg) * 256 + digit];
  __shared__ int64_t cum[256];
  cum[i] = hv;
  __syncthreads();
  for (int w = 1; w < 256; w <<= 1) {          // inclusive scan (Hillis-Steele)
    int64_t add = (i >= w) ? cum[i - w] : 0;
    __syncthreads();
    cum[i] += add;
    __syncthreads();
  }
  const int64_t incl = cum[i];
  const int64_t excl = incl - hv;
  if (pass == 0 && i == 255 && incl <= s.brem) {
    st[seg].all_fit = 1;                      // every positive step fits
    return;
  }
  if (excl <= s.brem && incl > s.brem) {      // exactly one thread
    const int shift = 8 * (nbytes - 1 - pass);
    st[seg].prefix = s.prefix | ((uint64_t)digit << shift);
    st[seg].brem = s.brem - excl;
  }
}

// ---- ordered tie scan and assignment ----------------------------------------------------

__device__ __forceinline__ int64_t tie_rate_of_unit(const uint64_t* keys, int64_t u, int64_t sz,
                                                    uint64_t lam, int* nsteps) {
  const uint4* kp = reinterpret_cast<const uint4*>(keys + u * 4);
  uint4 a = kp[0], b = kp[1];
  uint64_t kk[4] = {(uint64_t)a.x | ((uint64_t)a.y << 32), (uint64_t)a.z | ((uint64_t)a.w << 32),
                    (uint64_t)b.x | ((uint64_t)b.y << 32), (uint64_t)b.z | ((uint64_t)b.w << 32)};
  int n = 0;
  int64_t tie = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (kk[k] != 0) {
      if (kk[k] > lam) ++n;
      else if (kk[k] == lam) tie = sz * (int64_t)(kLevels[k + 1] - kLevels[k]);
    }
  }
  *nsteps = n;
  return tie;
}

template <bool TOPK>
__device__ __forceinline__ int64_t unit_tie(const uint64_t* keys, const float* scores, int64_t u,
                                            int64_t seg, int64_t seg_len, int stage, int d,
                                            const int64_t* rcount, const SelState& s, int* n) {
  if (TOPK) {
    if (u >= seg_len || s.none) { *n = 0; return 0; }
    uint64_t key = score_key(scores[seg * seg_len + u]);
    *n = key > s.prefix ? 1 : 0;
    return key == s.prefix ? 1 : 0;
  } else {
    if (u >= seg_len) { *n = 0; return 0; }
    if (s.all_fit) {
      int nn = 0;
      tie_rate_of_unit(keys, u, unit_size(stage, d, u, rcount), 0ull, &nn);
      *n = nn;
      return 0;
    }
    return tie_rate_of_unit(keys, u, unit_size(stage, d, u, rcount), s.prefix, n);
  }
}

// Block sums of the tie rates (4 units per thread, units in index order).
template <bool TOPK>
__global__ void __launch_bounds__(256)
alloc_tie_sum(const uint64_t* __restrict__ keys, const float* __restrict__ scores, int64_t seg_len,
              int stage, int d, const int64_t* __restrict__ rcount, const SelState* __restrict__ st,
              int64_t* __restrict__ bsum) {
  const int seg = blockIdx.y;
  const SelState s = st[seg];
  const int64_t base = (int64_t)blockIdx.x * kUnitsPerBlock + threadIdx.x * 4;
  int64_t t = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int n;
    t += unit_tie<TOPK>(keys, scores, base + j, seg, seg_len, stage, d, rcount, s, &n);
  }
  __shared__ int64_t red[256];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[(int64_t)seg * gridDim.x + blockIdx.x] = red[0];
}

// Exclusive scan of the block sums of each segment (one block per segment).
__global__ void __launch_bounds__(1024)
alloc_tie_scan(const int64_t* __restrict__ bsum, int64_t* __restrict__ bexcl, int nblk) {
  const int seg = blockIdx.x;
  __shared__ int64_t buf[1024];
  int64_t carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 1024) {
    const int i = threadIdx.x;
    int64_t v = (b0 + i < nblk) ? bsum[(int64_t)seg * nblk + b0 + i] : 0;
    buf[i] = v;
    __syncthreads();
    for (int w = 1; w < 1024; w <<= 1) {
      int64_t add = (i >= w) ? buf[i - w] : 0;
      __syncthreads();
      buf[i] += add;
      __syncthreads();
    }
    if (b0 + i < nblk) bexcl[(int64_t)seg * nblk + b0 + i] = carry + buf[i] - v;
    int64_t tot = buf[1023];
    __syncthreads();
    carry += tot;
  }
}

// Final widths: steps with key > lambda*, plus the tied step when the inclusive prefix of tie
// rates (ascending unit index) still fits the remaining budget.  Also per-block partial sums
// of the used rate and the distortion, reduced later in a fixed order.
template <bool TOPK>
__global__ void __launch_bounds__(256)
alloc_assign(const uint64_t* __restrict__ keys, const float* __restrict__ weight,
             const float* __restrict__ sigma, int64_t seg_len, int stage, int d,
             const int64_t* __restrict__ rcount, const SelState* __restrict__ st,
             const int64_t* __restrict__ bexcl, uint8_t* __restrict__ bits_out, int keep_bits,
             int64_t* __restrict__ used_part, double* __restrict__ dist_part) {
  const int seg = blockIdx.y;
  const SelState s = st[seg];
  const int64_t base = (int64_t)blockIdx.x * kUnitsPerBlock + threadIdx.x * 4;
  int64_t tie[4];
  int n[4];
  int64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tie[j] = unit_tie<TOPK>(keys, weight, base + j, seg, seg_len, stage, d, rcount, s, &n[j]);
    tsum += tie[j];
  }
  __shared__ int64_t buf[256];
  const int i = threadIdx.x;
  buf[i] = tsum;
  __syncthreads();
  for (int w = 1; w < 256; w <<= 1) {
    int64_t add = (i >= w) ? buf[i - w] : 0;
    __syncthreads();
    buf[i] += add;
    __syncthreads();
  }
  int64_t run = bexcl[(int64_t)seg * gridDim.x + blockIdx.x] + buf[i] - tsum;
  const int64_t cap = TOPK ? s.brem + 1 : s.brem;
  int64_t used = 0;
  double dist = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t u = base + j;
    if (u >= seg_len) continue;
    int nn = n[j];
    if (tie[j] > 0) {
      run += tie[j];
      if (run <= cap) nn += 1;
    }
    uint32_t b = TOPK ? (nn ? (uint32_t)keep_bits : 0u) : kLevels[nn];
    bits_out[(int64_t)seg * seg_len + u] = (uint8_t)b;
    if (!TOPK) {
      const int64_t sz = unit_size(stage, d, u, rcount);
      used += sz * (int64_t)b;
      float c = weight[u];
      if (sigma) c = c * sigma[u];
      dist += ldexp((double)c, -(int)b);
    } else {
      used += (int64_t)b * d;
    }
  }
  __shared__ int64_t ru[256];
  __shared__ double rd[256];
  ru[i] = used;
  rd[i] = dist;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (i < w) {
      ru[i] += ru[i + w];
      rd[i] += rd[i + w];
    }
    __syncthreads();
  }
  if (i == 0) {
    used_part[(int64_t)seg * gridDim.x + blockIdx.x] = ru[0];
    dist_part[(int64_t)seg * gridDim.x + blockIdx.x] = rd[0];
  }
}

__global__ void alloc_finalize(const SelState* __restrict__ st, const int64_t* __restrict__ used_part,
                               const double* __restrict__ dist_part, int nseg, int nblk, int topk,
                               kvc_alloc_result* result) {
  if (threadIdx.x != 0 || blockIdx.x != 0 || result == nullptr) return;
  int64_t used = 0;
  double dist = 0.0;
  for (int sgi = 0; sgi < nseg; ++sgi)
    for (int b = 0; b < nblk; ++b) {
      used += used_part[(int64_t)sgi * nblk + b];
      dist += dist_part[(int64_t)sgi * nblk + b];
    }
  kvc_alloc_result r;
  if (topk) {
    r.lambda = 0.0;
    r.budget_bits = used;
    r.used_bits = used;
    r.distortion = 0.0;
  } else {
    const SelState s = st[0];
    r.lambda = s.all_fit ? 0.0 : __longlong_as_double((long long)s.prefix);
    r.budget_bits = s.budget;
    r.used_bits = used;
    r.distortion = dist;
  }
  *result = r;
}

struct Plan {
  int nseg, nblk, passes, nbytes;
  int64_t U, seg_len;
};

Plan plan_of(const Layer& L, int stage) {
  Plan p;
  if (stage == KVC_ALLOC_TOPK) {
    p.nseg = L.hkv;
    p.seg_len = L.n;
    p.U = L.n * L.hkv;
    p.nbytes = 4;
  } else {
    p.nseg = 1;
    p.U = (stage == KVC_ALLOC_V_TOKENS) ? (int64_t)L.hkv * L.n : (int64_t)L.hkv * L.d;
    p.seg_len = p.U;
    p.nbytes = 8;
  }
  p.passes = p.nbytes;
  p.nblk = (int)((p.seg_len + kUnitsPerBlock - 1) / kUnitsPerBlock);
  return p;
}

AllocWs carve(const Layer& L, int stage, char* ws, size_t* total) {
  Plan p = plan_of(L, stage);
  WsPlan w;
  AllocWs a{};
  size_t o_st = w.take(sizeof(SelState) * p.nseg);
  size_t o_h = w.take(sizeof(int64_t) * p.passes * p.nseg * 256);
  size_t o_k = w.take(stage == KVC_ALLOC_TOPK ? 0 : sizeof(uint64_t) * 4 * p.U);
  size_t o_r = w.take(sizeof(int64_t) * L.hkv);
  size_t o_b = w.take(sizeof(int64_t) * p.nseg * p.nblk);
  size_t o_e = w.take(sizeof(int64_t) * p.nseg * p.nblk);
  size_t o_u = w.take(sizeof(int64_t) * p.nseg * p.nblk);
  size_t o_d = w.take(sizeof(double) * p.nseg * p.nblk);
  if (total) *total = w.off;
  if (ws) {
    a.status = reinterpret_cast<int32_t*>(ws);
    a.st = reinterpret_cast<SelState*>(ws + o_st);
    a.hist = reinterpret_cast<int64_t*>(ws + o_h);
    a.keys = reinterpret_cast<uint64_t*>(ws + o_k);
    a.rcount = reinterpret_cast<int64_t*>(ws + o_r);
    a.bsum = reinterpret_cast<int64_t*>(ws + o_b);
    a.bexcl = reinterpret_cast<int64_t*>(ws + o_e);
    a.used_part = reinterpret_cast<int64_t*>(ws + o_u);
    a.dist_part = reinterpret_cast<double*>(ws + o_d);
  }
  return a;
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
  const bool topk = (stage == KVC_ALLOC_TOPK);
  (void)launch_reset_status(ws, s);
  if (stage == KVC_ALLOC_K_CHANNELS)
    count_retained<<<L.hkv, 256, 0, s>>>(bits_v, L.n, a.rcount, a.status);
  const int64_t hist_len = (int64_t)p.passes * p.nseg * 256;
  alloc_init<<<1, 256, 0, s>>>(a.st, a.hist, hist_len, stage, p.nseg, L.hkv, L.d, L.n, a.rcount,
                               avg_bits, keep_fraction);
  if (!topk)
    alloc_keys<<<(unsigned)((p.U + 255) / 256), 256, 0, s>>>(weight, sigma, p.U, stage, L.d, a.rcount, a.keys);
  dim3 g2((unsigned)p.nblk, (unsigned)p.nseg);
  for (int pass = 0; pass < p.passes; ++pass) {
    if (topk)
      alloc_hist<true><<<g2, 256, 0, s>>>(nullptr, weight, p.U, p.seg_len, stage, L.d, a.rcount, a.st, a.hist, pass, p.nbytes);
    else
      alloc_hist<false><<<g2, 256, 0, s>>>(a.keys, nullptr, p.U, p.seg_len, stage, L.d, a.rcount, a.st, a.hist, pass, p.nbytes);
    alloc_select<<<p.nseg, 256, 0, s>>>(a.st, a.hist, pass, p.nbytes, p.nseg);
  }
  if (topk) {
    alloc_tie_sum<true><<<g2, 256, 0, s>>>(nullptr, weight, p.seg_len, stage, L.d, a.rcount, a.st, a.bsum);
    alloc_tie_scan<<<p.nseg, 1024, 0, s>>>(a.bsum, a.bexcl, p.nblk);
    alloc_assign<true><<<g2, 256, 0, s>>>(nullptr, weight, nullptr, p.seg_len, stage, L.d, a.rcount, a.st, a.bexcl, bits_out, keep_bits, a.used_part, a.dist_part);
  } else {
    alloc_tie_sum<false><<<g2, 256, 0, s>>>(a.keys, nullptr, p.seg_len, stage, L.d, a.rcount, a.st, a.bsum);
    alloc_tie_scan<<<p.nseg, 1024, 0, s>>>(a.bsum, a.bexcl, p.nblk);
    alloc_assign<false><<<g2, 256, 0, s>>>(a.keys, weight, sigma, p.seg_len, stage, L.d, a.rcount, a.st, a.bexcl, bits_out, keep_bits, a.used_part, a.dist_part);
  }
  alloc_finalize<<<1, 64, 0, s>>>(a.st, a.used_part, a.dist_part, p.nseg, p.nblk, topk ? 1 : 0, result);
  return hipGetLastError();
}

}  // namespace kvc
