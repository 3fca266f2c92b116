// Attention over a packed cache with the dequantisation fused into the tile staging (RDKV
// summary §2.3: logits and outputs computed straight from the packed width zones).  Gives the
// output Y_hat and the row LSE l_hat whose errors against the full cache are the two terms of
// KVSculpt's loss (KVSculpt summary §2).
//
// Block = (4 waves, key split, KV head g); wave = one query head of the group x 32 query
// rows.  For each group of 32 retained tokens (the K packing unit) the block decodes
//   K_hat -> LDS as a bf16 hi/lo pair (K_hat = hi + lo to ~2^-17; the bf16 query is exact, so
//            q.K_hat = q.hi + q.lo is two bf16 matrix-core products with fp32 accumulation),
//   V_hat -> LDS transposed as fp16 [channel][token],
// then S = K_hat Q^T (32x32x16 bf16), an online base-2 softmax per row, and
// O^T += V_hat^T P^T (32x32x16 f16).  In both products a lane owns one query row, so the
// softmax statistics and the output rescale stay in-lane.  P^T is taken straight from the S
// accumulator: lane l holds keys 8(i/4) + 4(l/32) + i%4, and the V_hat^T operand is read with
// the same key order, which is a valid ordering of the contraction index.
// Each block writes (m, l, O) partials per row; a merge kernel combines the splits by LSE.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32;   // query rows per wave

template <int D>
struct AttnSmem {
  uint16_t khi[32][D + 8];
  uint16_t klo[32][D + 8];
  _Float16 vt[D][32 + 8];
  int32_t woff[D];
  int32_t qslot[D];
  int32_t width[D];
  int32_t tok[32];
  int32_t vloc[32];
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int D>
__global__ void __launch_bounds__(256)
attend_split(const uint16_t* __restrict__ q, kvc_packed_cache cache, float* __restrict__ part,
             int G, int Hkv, int64_t N, int64_t Nq, int causal, float c, int nsplit,
             int32_t* status) {
  constexpr int KS = D / 16;
  constexpr int GPR = D / 32;
  constexpr int PSTRIDE = D + 2;
  __shared__ AttnSmem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const int g = blockIdx.z;
  const int split = blockIdx.y;
  const int nRT = (int)((Nq + kRows - 1) / kRows);
  const int pair = blockIdx.x * kWaves + wave;
  const bool active = pair < G * nRT;
  const int hl = active ? pair % G : 0;
  const int rt = active ? pair / G : 0;
  const int h = g * G + hl;
  const int64_t r0 = (int64_t)rt * kRows;
  const int64_t off = N - Nq;

  const int64_t* H = cache.header;
  if (H[0] != Hkv || H[1] != D || H[2] != N) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && split == 0) set_status(status, KVC_DEV_BAD_CACHE);
    return;
  }
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t R = hp[4];
  const int64_t ngroups = hp[22];
  const int64_t Wk = hp[20];
  const int64_t Qk = hp[21];
  const int64_t gps = (ngroups + nsplit - 1) / nsplit;
  const int64_t j_begin = (int64_t)split * gps;
  const int64_t j_end_raw = j_begin + gps < ngroups ? j_begin + gps : ngroups;

  // channel tables of this head's K packing
  if (threadIdx.x == 0) {
    int32_t wo = 0, qs = 0;
    for (int cc = 0; cc < D; ++cc) {
      int b = cache.k_width[(int64_t)g * D + cc];
      if (!valid_width((uint32_t)b)) b = 0;
      sm.width[cc] = b;
      sm.woff[cc] = wo;
      sm.qslot[cc] = qs;
      wo += b;
      qs += (b == 2 || b == 4 || b == 8);
    }
  }

  // Q^T operand of this wave's rows
  bf16x8 qb[KS];
  {
    const int64_t row = r0 + lo;
    const bool ok = active && row < Nq;
    const uint16_t* qp = q + ((int64_t)h * Nq + (ok ? row : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qp + ks * 16 + 8 * hi) : make_uint4(0, 0, 0, 0));
  }
  const int64_t pos = off + r0 + lo;          // this lane's row position
  // last position among the block's active rows (rows of later pairs are later or equal)
  int64_t pmax_block;
  {
    int last_pair = blockIdx.x * kWaves + kWaves - 1;
    if (last_pair >= G * nRT) last_pair = G * nRT - 1;
    int64_t lr = (int64_t)(last_pair / G) * kRows + kRows - 1;
    if (lr >= Nq) lr = Nq - 1;
    pmax_block = causal ? off + lr : N - 1;
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[GPR];
#pragma unroll
  for (int mb = 0; mb < GPR; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;

  __syncthreads();
  for (int64_t j = j_begin; j < j_end_raw; ++j) {
    const int m_valid = (int)((R - j * 32) < 32 ? (R - j * 32) : 32);
    if (threadIdx.x < 32) {
      const int e = threadIdx.x;
      sm.tok[e] = e < m_valid ? cache.k_keep[hp[17] + j * 32 + e] : 0x7FFFFFFF;
      sm.vloc[e] = e < m_valid ? cache.k_vloc[hp[17] + j * 32 + e] : 0;
    }
    __syncthreads();
    if (sm.tok[0] > pmax_block) break;      // retained tokens ascend: nothing visible later
    // ---- decode K_hat: thread -> (channel, quarter of the 32 tokens)
    {
      constexpr int TPC = 256 / D;         // threads per channel (2 or 4)
      constexpr int EPT = 32 / TPC;        // tokens per thread
      const int cc = threadIdx.x % D;
      const int e0 = (threadIdx.x / D) * EPT;
      const int b = sm.width[cc];
      const uint32_t* wp = cache.k_words + hp[18] + j * Wk + sm.woff[cc];
      float s = 0.f, z = 0.f;
      if (b == 2 || b == 4 || b == 8) {
        const float* pp = cache.k_par + 2 * (hp[19] + j * Qk + sm.qslot[cc]);
        s = pp[0];
        z = pp[1];
      }
      for (int e = e0; e < e0 + EPT; ++e) {
        uint16_t vh = 0, vl = 0;
        if (b == 16) {
          vh = (uint16_t)((wp[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
        } else if (b != 0) {
          const int per = 32 / b;
          const uint32_t code = (wp[e / per] >> ((e % per) * b)) & ((1u << b) - 1u);
          const float x = fmaf(s, (float)code, z);
          vh = f32_to_bf16_rne(x);
          vl = f32_to_bf16_rne(x - bf16_bits_to_f32(vh));
        }
        sm.khi[e][cc] = vh;
        sm.klo[e][cc] = vl;
      }
    }
    // ---- decode V_hat^T: thread -> (token, 32-channel group, half of the group)
    {
      for (int task = threadIdx.x; task < 32 * GPR * 2; task += 256) {
        const int e = task / (GPR * 2);
        const int rem = task % (GPR * 2);
        const int grp = rem / 2;
        const int half = rem % 2;
        if (e >= m_valid) {
          for (int cc = 0; cc < 16; ++cc) sm.vt[grp * 32 + half * 16 + cc][e] = (_Float16)0.f;
          continue;
        }
        const int32_t loc = sm.vloc[e];
        const int z = loc >> 29;
        const int64_t vpos = loc & ((1 << 29) - 1);
        const int b = 2 << z;
        const uint32_t* wp = cache.v_words + hp[9 + z] + (vpos * GPR + grp) * b;
        if (b == 16) {
          for (int cc = 0; cc < 16; ++cc) {
            const int el = half * 16 + cc;
            float x = bf16_bits_to_f32((wp[el >> 1] >> ((el & 1) * 16)) & 0xFFFFu);
            sm.vt[grp * 32 + el][e] = (_Float16)x;
          }
        } else {
          const float* pp = cache.v_par + 2 * (hp[13 + z] + vpos * GPR + grp);
          const float s = pp[0], zz = pp[1];
          const int per = 32 / b;
          for (int cc = 0; cc < 16; ++cc) {
            const int el = half * 16 + cc;
            const uint32_t code = (wp[el / per] >> ((el % per) * b)) & ((1u << b) - 1u);
            sm.vt[grp * 32 + el][e] = (_Float16)fmaf(s, (float)code, zz);
          }
        }
      }
    }
    __syncthreads();
    const int64_t t_first = sm.tok[0];
    if (active && (!causal || t_first <= off + r0 + kRows - 1)) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 ah = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.khi[lo][ks * 16 + 8 * hi]));
        bf16x8 al = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.klo[lo][ks * 16 + 8 * hi]));
        acc = mfma32(ah, qb[ks], acc);
        acc = mfma32(al, qb[ks], acc);
      }
      float x[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = acc_row(i, hi);
        const int64_t t = sm.tok[e];
        float v = acc[i] * c;
        if (e >= m_valid || (causal && t > pos)) v = -INFINITY;
        x[i] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = fmaxf(tmax, swap_half(tmax));
      const float mnew = fmaxf(m_run, tmax);
      float p[16];
      float alpha = 1.f;
      if (mnew > -INFINITY) {
        alpha = fast_exp2(m_run - mnew);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = fast_exp2(x[i] - mnew);
          ps += p[i];
        }
        l_run = l_run * alpha + ps;
        m_run = mnew;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = 0.f;
      }
#pragma unroll
      for (int mb = 0; mb < GPR; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
      // O^T[ch][row] += sum_key V^T[ch][key] P^T[key][row], keys in the accumulator's order
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        f16x8 pb;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pb[jj] = (_Float16)p[ks2 * 8 + jj];
        const int kbase = 16 * ks2 + 4 * hi;
#pragma unroll
        for (int mb = 0; mb < GPR; ++mb) {
          const _Float16* vr = &sm.vt[mb * 32 + lo][0];
          f16x8 va;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            va[jj] = vr[kbase + jj];
            va[4 + jj] = vr[kbase + 8 + jj];
          }
          o[mb] = mfma32h(va, pb, o[mb]);
        }
      }
    }
    __syncthreads();
  }

  if (!active) return;
  const float lt = l_run + swap_half(l_run);
  const int64_t row = r0 + lo;
  if (row >= Nq) return;
  float* pr = part + (((int64_t)h * Nq + row) * nsplit + split) * PSTRIDE;
  if (hi == 0) {
    pr[0] = m_run;
    pr[1] = lt;
  }
#pragma unroll
  for (int mb = 0; mb < GPR; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) pr[2 + mb * 32 + acc_row(i, hi)] = o[mb][i];
}

// Combine the splits of each (head, row): M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum O_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.
__global__ void __launch_bounds__(128)
attend_merge(const float* __restrict__ part, float* __restrict__ out, float* __restrict__ lse,
             int D, int nsplit) {
  const int64_t hr = blockIdx.x;             // h * Nq + row
  const int PSTRIDE = D + 2;
  const float* pr = part + hr * nsplit * PSTRIDE;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pr[s * PSTRIDE]);
  float L = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = pr[s * PSTRIDE];
    if (ms > -INFINITY) L += pr[s * PSTRIDE + 1] * exp2f(ms - M);
  }
  for (int cc = threadIdx.x; cc < D; cc += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = pr[s * PSTRIDE];
      if (ms > -INFINITY) acc += pr[s * PSTRIDE + 2 + cc] * exp2f(ms - M);
    }
    out[hr * D + cc] = (L > 0.f) ? acc / L : 0.f;
  }
  if (threadIdx.x == 0) lse[hr] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

int nsplit_of(const Layer& L) {
  const int nRT = (int)((L.nq + kRows - 1) / kRows);
  const int64_t bps = (int64_t)L.hkv * ((L.G * nRT + kWaves - 1) / kWaves);   // blocks per split
  int64_t want = (1024 + bps - 1) / bps;
  const int64_t maxs = (L.n + 32 * 8 - 1) / (32 * 8);   // at least 8 groups per split
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  if (want > 256) want = 256;
  return (int)want;
}

}  // namespace

size_t attend_ws_bytes(const Layer& L) {
  WsPlan p;
  p.take((size_t)L.hq * L.nq * nsplit_of(L) * (L.d + 2) * sizeof(float));
  return p.off;
}

hipError_t launch_attend(const Layer& L, const uint16_t* q, const kvc_packed_cache& cache,
                         float* out, float* lse, char* ws, hipStream_t s) {
  const int nsplit = nsplit_of(L);
  WsPlan p;
  float* part = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * L.nq * nsplit * (L.d + 2) * sizeof(float)));
  (void)launch_reset_status(ws, s);
  const int nRT = (int)((L.nq + kRows - 1) / kRows);
  dim3 grid((unsigned)((L.G * nRT + kWaves - 1) / kWaves), (unsigned)nsplit, (unsigned)L.hkv);
  int32_t* status = reinterpret_cast<int32_t*>(ws);
  if (L.d == 128)
    attend_split<128><<<grid, 256, 0, s>>>(q, cache, part, L.G, L.hkv, L.n, L.nq, L.causal, L.c_log2, nsplit, status);
  else
    attend_split<64><<<grid, 256, 0, s>>>(q, cache, part, L.G, L.hkv, L.n, L.nq, L.causal, L.c_log2, nsplit, status);
  attend_merge<<<(unsigned)((int64_t)L.hq * L.nq), 128, 0, s>>>(part, out, lse, L.d, nsplit);
  return hipGetLastError();
}

}  // namespace kvc
