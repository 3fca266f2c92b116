// Attention over a packed cache with the dequantisation fused into the tile staging (RDKV
// summary §2.3: logits and outputs computed straight from the packed width zones).  Gives the
// output Y_hat and the row LSE l_hat whose errors against the full cache are the two terms of
// KVSculpt's loss (KVSculpt summary §2).
//
// Block = (8 waves, key split, KV head g); wave = one query head of the group x 32 query
// rows.  The block first lays out the head's K channel table once (block scan over the
// channel widths: word offset and parameter slot per channel, channels ordered by width).
// Then for each group of 32 retained tokens (the K packing unit) it decodes
//   K_hat -> LDS as a bf16 hi/lo pair (K_hat = hi + lo to ~2^-17; the bf16 query is exact, so
//            q.K_hat = q.hi + q.lo is two bf16 matrix-core products with fp32 accumulation),
//   V_hat -> LDS transposed as fp16 [channel][token],
// each thread unpacking a run of codes of one channel (K) or one token's group (V) from a
// 64-bit window with shifts (no divisions); the channel order by width keeps the lanes of a
// wave on one width.  Then S = K_hat Q^T (32x32x16 bf16), an online base-2 softmax per row,
// and O^T += V_hat^T P^T (32x32x16 f16).  In both products a lane owns one query row, so the
// softmax statistics and the output rescale stay in-lane.  P^T is taken straight from the S
// accumulator: lane l holds keys 8(i/4) + 4(l/32) + i%4, and the V_hat^T operand is read with
// the same key order, which is a valid ordering of the contraction index.
// Each block writes (m, l, O) partials per row; a merge kernel combines the splits by LSE.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kWaves = 8;
constexpr int kThreadsA = 64 * kWaves;
constexpr int kRows = 32;   // query rows per wave

template <int D>
struct AttnSmem {
  uint16_t khi[32][D + 8];
  uint16_t klo[32][D + 8];
  _Float16 vt[D][32 + 8];
  int32_t kinfo[D][4];     // channels in width order: {channel, word offset, param slot, width}
  int32_t tok[32];
  int32_t vloc[32];
  uint64_t scan[kWaves];
};

// bf16 hi/lo split of x (hardware round-to-nearest-even conversions): low 16 bits hi, high lo.
__device__ __forceinline__ uint32_t bf16_hilo(float x) {
  const __bf16 h = (__bf16)x;
  const __bf16 l = (__bf16)(x - (float)h);
  return (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
}

// 64 bits of a word stream starting at word wi (the second word only if `two`).
__device__ __forceinline__ uint64_t load_window(const uint32_t* w, int64_t wi, bool two) {
  const uint64_t lo = w[wi];
  const uint64_t hi = two ? w[wi + 1] : 0u;
  return lo | (hi << 32);
}

template <int D>
__global__ void __launch_bounds__(kThreadsA)
attend_split(const uint16_t* __restrict__ q, kvc_packed_cache cache, float* __restrict__ part,
             int G, int Hkv, int64_t N, int64_t Nq, int causal, float c, int nsplit,
             int32_t* status) {
  constexpr int KS = D / 16;
  constexpr int GPR = D / 32;
  constexpr int PSTRIDE = D + 2;
  constexpr int KP = kThreadsA / D;        // K decode: threads per channel
  constexpr int KE = 32 / KP;              // K decode: tokens per thread (8 or 4)
  constexpr int VP = kThreadsA / (32 * GPR);   // V decode: threads per (token, group)
  constexpr int VE = 32 / VP;              // V decode: channels per thread (8)
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

  // channel table of this head's K packing: one uint64 per channel packs {words (16 bits),
  // params (16 bits), an 8-bit count per width class}; one block scan places every channel
  {
    uint32_t b = 0;
    int cls = 4;
    uint64_t f = 0;
    const int t = threadIdx.x;
    if (t < D) {
      b = cache.k_width[(int64_t)g * D + t];
      cls = b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : b == 16 ? 3 : 4;
      if (cls < 4) f = (uint64_t)b | ((uint64_t)(cls < 3) << 16) | (1ull << (32 + 8 * cls));
    }
    uint64_t tf;
    const uint64_t ef = block_excl_scan<kThreadsA>(f, &tf, sm.scan);
    if (t < D) {
      int pos = 0, before = 0, nnz = 0;
      for (int k2 = 0; k2 < 4; ++k2) {
        const int tk = (int)((tf >> (32 + 8 * k2)) & 0xFF);
        if (k2 < cls) pos += tk;
        before += (int)((ef >> (32 + 8 * k2)) & 0xFF);
        nnz += tk;
      }
      pos = cls < 4 ? pos + (int)((ef >> (32 + 8 * cls)) & 0xFF) : nnz + (t - before);
      sm.kinfo[pos][0] = t;
      sm.kinfo[pos][1] = (int32_t)(ef & 0xFFFF);
      sm.kinfo[pos][2] = (int32_t)((ef >> 16) & 0xFFFF);
      sm.kinfo[pos][3] = cls < 4 ? (int32_t)b : 0;
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
  const int4 kinf = *reinterpret_cast<const int4*>(sm.kinfo[threadIdx.x % D]);   // this thread's K channel
  for (int64_t j = j_begin; j < j_end_raw; ++j) {
    const int m_valid = (int)((R - j * 32) < 32 ? (R - j * 32) : 32);
    if (threadIdx.x < 32) {
      const int e = threadIdx.x;
      sm.tok[e] = e < m_valid ? cache.k_keep[hp[17] + j * 32 + e] : 0x7FFFFFFF;
      sm.vloc[e] = e < m_valid ? cache.k_vloc[hp[17] + j * 32 + e] : 0;
    }
    __syncthreads();
    if (sm.tok[0] > pmax_block) break;      // retained tokens ascend: nothing visible later
    // ---- decode K_hat: thread -> (channel in width order, run of KE tokens)
    {
      const int cc = kinf.x, b = kinf.w;
      const int e0 = (threadIdx.x / D) * KE;
      uint32_t hl2[KE];
      if (b == 0) {
#pragma unroll
        for (int k = 0; k < KE; ++k) hl2[k] = 0u;
      } else {
        const uint32_t* wp = cache.k_words + hp[18] + j * Wk + kinf.y;
        if (b == 16) {                       // raw bf16 (lo = 0): KE / 2 words
#pragma unroll
          for (int k = 0; k < KE; k += 2) {
            const uint32_t w = wp[(e0 + k) >> 1];
            hl2[k] = w & 0xFFFFu;
            hl2[k + 1] = w >> 16;
          }
        } else {
          const int bit0 = e0 * b;             // KE * b <= 64 bits from bit0
          const uint64_t win = load_window(wp, bit0 >> 5, (bit0 & 31) + KE * b > 32) >> (bit0 & 31);
          const float2 sz = *reinterpret_cast<const float2*>(cache.k_par + 2 * (hp[19] + j * Qk + kinf.z));
          const uint32_t mask = (1u << b) - 1u;
#pragma unroll
          for (int k = 0; k < KE; ++k) {
            const uint32_t code = (uint32_t)(win >> (k * b)) & mask;
            hl2[k] = bf16_hilo(fmaf(sz.x, (float)code, sz.y));
          }
        }
      }
#pragma unroll
      for (int k = 0; k < KE; ++k) {
        sm.khi[e0 + k][cc] = (uint16_t)(hl2[k] & 0xFFFFu);
        sm.klo[e0 + k][cc] = (uint16_t)(hl2[k] >> 16);
      }
    }
    // ---- decode V_hat^T: thread -> (token e, 32-channel group, run of VE channels)
    {
      const int task = threadIdx.x;
      const int e = task / (GPR * VP);
      const int grp = (task / VP) % GPR;
      const int c0 = (task % VP) * VE;
      _Float16 vv[VE];
      if (e >= m_valid) {
#pragma unroll
        for (int k = 0; k < VE; ++k) vv[k] = (_Float16)0.f;
      } else {
        const int32_t loc = sm.vloc[e];
        const int z = loc >> 29;
        const int64_t vpos = loc & ((1 << 29) - 1);
        const int b = 2 << z;
        const uint32_t* wp = cache.v_words + hp[9 + z] + (vpos * GPR + grp) * b;
        if (b == 16) {                       // raw bf16: VE / 2 words
#pragma unroll
          for (int k = 0; k < VE; k += 2) {
            const uint32_t w = wp[(c0 + k) >> 1];
            vv[k] = (_Float16)bf16_bits_to_f32(w & 0xFFFFu);
            vv[k + 1] = (_Float16)bf16_bits_to_f32(w >> 16);
          }
        } else {
          const int bit0 = c0 * b;             // VE * b <= 64 bits from bit0
          const uint64_t win = load_window(wp, bit0 >> 5, (bit0 & 31) + VE * b > 32) >> (bit0 & 31);
          const float2 sz = *reinterpret_cast<const float2*>(cache.v_par + 2 * (hp[13 + z] + vpos * GPR + grp));
          const uint32_t mask = (1u << b) - 1u;
#pragma unroll
          for (int k = 0; k < VE; ++k)
            vv[k] = (_Float16)fmaf(sz.x, (float)((uint32_t)(win >> (k * b)) & mask), sz.y);
        }
      }
#pragma unroll
      for (int k = 0; k < VE; ++k) sm.vt[grp * 32 + c0 + k][e] = vv[k];
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
      const bool full = m_valid == 32 && (!causal || sm.tok[31] <= off + r0);   // uniform per wave
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = acc[i] * c;
      if (!full) {
        // slots past m_valid hold the sentinel 0x7FFFFFFF, so one compare covers both masks
        const int lim = causal ? (int)pos : 0x7FFFFFFE;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (sm.tok[acc_row(i, hi)] <= lim) ? x[i] : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, x[i]);
      tmax = half_max(tmax);
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
    attend_split<128><<<grid, kThreadsA, 0, s>>>(q, cache, part, L.G, L.hkv, L.n, L.nq, L.causal, L.c_log2, nsplit, status);
  else
    attend_split<64><<<grid, kThreadsA, 0, s>>>(q, cache, part, L.G, L.hkv, L.n, L.nq, L.causal, L.c_log2, nsplit, status);
  attend_merge<<<(unsigned)((int64_t)L.hq * L.nq), 128, 0, s>>>(part, out, lse, L.d, nsplit);
  return hipGetLastError();
}

}  // namespace kvc
