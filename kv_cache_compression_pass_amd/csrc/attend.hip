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
// each thread unpacking a run of codes of one channel (K) or two tokens' channel run (V) from
// a 64-bit window with shifts (no divisions).  Two LDS buffers hold consecutive groups: while
// the block multiplies group j it decodes group j+1 into the other buffer (one barrier per
// group), and group j+2's words are in flight in registers.  Then S = K_hat Q^T (32x32x16
// bf16, the hi and lo products in two chains), an online base-2 softmax per row,
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
  uint16_t khi[2][32][D + 8];   // two buffers: group j is decoded into buffer j & 1
  uint16_t klo[2][32][D + 8];
  _Float16 vt[2][D][32 + 8];
  int32_t tok[2][32];
  int32_t kinfo[D][4];     // channels in width order: {channel, word offset, param slot, width}
  int64_t vzone[4][2];     // V zones by width class: first word, first (scale, zero) pair
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
             int64_t shift, int pstride, int32_t* status) {
  constexpr int KS = D / 16;
  constexpr int GPR = D / 32;
  constexpr int PSTRIDE = D + 2;
  constexpr int KP = kThreadsA / D;        // K decode: threads per channel
  constexpr int KE = 32 / KP;              // K decode: tokens per thread (8 or 4)
  constexpr int VC = GPR;                  // V decode: channels per thread, for 2 tokens
  constexpr int VRUNS = 32 / VC;           // V decode: channel runs per 32-channel group
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
  const int64_t off = N - Nq + shift;         // row r sits at position off + r

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
    if (t < 4) {
      sm.vzone[t][0] = hp[9 + t];
      sm.vzone[t][1] = hp[13 + t];
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
  // K decode task: channel kinf.x (width kb), tokens ke0 .. ke0 + KE - 1 of the group
  const int kb = kinf.w;
  const int ke0 = (threadIdx.x / D) * KE;
  const int kbit0 = ke0 * kb;                  // KE * kb <= 64 bits from kbit0
  const bool ktwo = (kbit0 & 31) + KE * kb > 32;
  // V decode task: tokens 2 vtp and 2 vtp + 1, 32-channel group vgrp, channels vc0 .. vc0 + VC - 1.
  // The four 16-lane quarters of a wave take consecutive runs of one group, so a wave's
  // 32-bit stores of a token pair into V_hat^T land in distinct LDS banks.
  const int vtp = threadIdx.x & 15;
  const int vr = threadIdx.x >> 4;
  const int vgrp = vr / VRUNS;
  const int vc0 = (vr % VRUNS) * VC;
  // header fields used in the loop, read once (the zone bases sit in LDS)
  const int64_t slot0 = hp[17];                // the head's first retained-token slot
  const int64_t kword0 = hp[18], kpar0 = hp[19];

  // The global words of group j+1 (and the V locations of group j+2) are requested while
  // group j is in LDS, so their latency overlaps the products of group j.
  auto m_valid_of = [&](int64_t j) { return (int)((R - j * 32) < 32 ? (R - j * 32) : 32); };
  auto load_k = [&](int64_t j, uint32_t (&w)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = 0u;
    if (kb == 0) return;
    const uint32_t* wp = cache.k_words + kword0 + j * Wk + kinf.y;
    if (kb == 16) {                            // raw bf16: KE / 2 words
#pragma unroll
      for (int k = 0; k < KE / 2; ++k) w[k] = wp[(ke0 >> 1) + k];
    } else {
      w[0] = wp[kbit0 >> 5];
      if (ktwo) w[1] = wp[(kbit0 >> 5) + 1];
      const float2 sz = *reinterpret_cast<const float2*>(cache.k_par + 2 * (kpar0 + j * Qk + kinf.z));
      w[2] = __float_as_uint(sz.x);
      w[3] = __float_as_uint(sz.y);
    }
  };
  auto load_vloc = [&](int64_t j, int32_t (&vl)[2]) {   // -1 past the retained tokens
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t e = j * 32 + 2 * vtp + u;
      vl[u] = (e < R) ? cache.k_vloc[slot0 + e] : -1;
    }
  };
  // One token's VC channels: VC * b bits, aligned to their own size, so one word (two at
  // 16 bits, VC = 4), and the row's (scale, zero) pair.
  auto load_v = [&](int32_t loc, uint32_t (&w)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = 0u;
    if (loc < 0) return;
    const int z = loc >> 29;
    const int64_t vpos = loc & ((1 << 29) - 1);
    const int b = 2 << z;
    const uint32_t* wp = cache.v_words + sm.vzone[z][0] + (vpos * GPR + vgrp) * b + ((vc0 * b) >> 5);
    w[0] = wp[0];
    if (VC * b > 32) {
      w[1] = wp[1];
    } else if (b != 16) {
      const float2 sz = *reinterpret_cast<const float2*>(cache.v_par + 2 * (sm.vzone[z][1] + vpos * GPR + vgrp));
      w[2] = __float_as_uint(sz.x);
      w[3] = __float_as_uint(sz.y);
    }
  };
  auto load_tok = [&](int64_t j) -> int32_t {    // slots past the group's end hold the sentinel
    const int e = threadIdx.x & 31;
    return (threadIdx.x < 32 && e < m_valid_of(j)) ? cache.k_keep[slot0 + j * 32 + e] : 0x7FFFFFFF;
  };

  // Decode of one group from its raw words into LDS buffer `bf`, without branches (every lane
  // runs the same instructions, so the products of the previous group can interleave).
  auto decode_k = [&](const uint32_t (&w)[4], int bf) {
    const int kq = kb < 16 ? kb : 0;           // quantised width (0 for raw and evicted channels)
    const uint64_t win = ((uint64_t)w[0] | ((uint64_t)w[1] << 32)) >> (kbit0 & 31);
    const float sc = __uint_as_float(w[2]), zp = __uint_as_float(w[3]);
    const uint32_t mask = (1u << kq) - 1u;
    const int cc = kinf.x;
    // both forms are computed and blended with bit masks (a select would become a branch)
    const uint32_t mq = kq != 0 ? 0xFFFFFFFFu : 0u, mr = kb == 16 ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int k = 0; k < KE; ++k) {
      const uint32_t code = (uint32_t)(win >> (k * kq)) & mask;
      const uint32_t q = bf16_hilo(fmaf(sc, (float)code, zp));
      const uint32_t raw = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;   // lo = 0
      const uint32_t hl = (q & mq) | (raw & mr);
      sm.khi[bf][ke0 + k][cc] = (uint16_t)(hl & 0xFFFFu);
      sm.klo[bf][ke0 + k][cc] = (uint16_t)(hl >> 16);
    }
  };
  auto decode_v = [&](const uint32_t (&w)[2][4], const int32_t (&vl)[2], int bf) {
    uint32_t vv[2][VC];                        // fp16 bits
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int b = 2 << ((vl[u] >> 29) & 3);
      const int bq = b < 16 ? b : 0;
      const uint32_t win = w[u][0] >> ((vc0 * bq) & 31);
      const float sc = __uint_as_float(w[u][2]), zp = __uint_as_float(w[u][3]);
      const uint32_t mask = (1u << bq) - 1u;
      const uint32_t mq = (vl[u] >= 0 && bq != 0) ? 0xFFFFu : 0u, mr = (vl[u] >= 0 && bq == 0) ? 0xFFFFu : 0u;
#pragma unroll
      for (int k = 0; k < VC; ++k) {
        const _Float16 hq = (_Float16)fmaf(sc, (float)((win >> (k * bq)) & mask), zp);
        const _Float16 hr = (_Float16)bf16_bits_to_f32((w[u][k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
        vv[u][k] = ((uint32_t)__builtin_bit_cast(uint16_t, hq) & mq) | ((uint32_t)__builtin_bit_cast(uint16_t, hr) & mr);
      }
    }
#pragma unroll
    for (int k = 0; k < VC; ++k)
      *reinterpret_cast<uint32_t*>(&sm.vt[bf][vgrp * 32 + vc0 + k][2 * vtp]) = vv[0][k] | (vv[1][k] << 16);
  };

  // Pipeline: at the top of iteration j, LDS buffer j & 1 holds group j decoded, the registers
  // hold group j+1's raw words (set 1) and group j+2's V locations.  Iteration j requests group
  // j+2's words (set 2), multiplies group j while decoding group j+1 into the other buffer,
  // then moves set 2 into set 1.
  uint32_t kw1[4] = {0u, 0u, 0u, 0u}, vw1[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  int32_t vl1[2] = {-1, -1}, vl2[2] = {-1, -1}, tok1 = 0x7FFFFFFF, tf0 = 0, tf1 = 0;
  if (j_begin < j_end_raw) {
    uint32_t kw0[4], vw0[2][4];
    int32_t vl0[2];
    load_vloc(j_begin, vl0);
    load_k(j_begin, kw0);
    const int32_t tok0 = load_tok(j_begin);
    tf0 = cache.k_keep[slot0 + j_begin * 32];
    load_v(vl0[0], vw0[0]);
    load_v(vl0[1], vw0[1]);
    load_vloc(j_begin + 1, vl1);
    decode_k(kw0, (int)(j_begin & 1));
    decode_v(vw0, vl0, (int)(j_begin & 1));
    if (threadIdx.x < 32) sm.tok[j_begin & 1][threadIdx.x] = tok0;
    if (j_begin + 1 < j_end_raw) {
      load_k(j_begin + 1, kw1);
      tok1 = load_tok(j_begin + 1);
      tf1 = cache.k_keep[slot0 + (j_begin + 1) * 32];
      load_v(vl1[0], vw1[0]);
      load_v(vl1[1], vw1[1]);
    }
    load_vloc(j_begin + 2, vl2);
  }
  for (int64_t j = j_begin; j < j_end_raw; ++j) {
    if ((int64_t)tf0 > pmax_block) break;      // retained tokens ascend: nothing visible later
    const int buf = (int)(j & 1);
    const int m_valid = m_valid_of(j);
    // One barrier per group: group j is in LDS, and every wave has finished group j-1, the
    // last reader of the buffer that group j+1 is decoded into below.
    __syncthreads();
    // ---- requests for group j + 2 (set 2), in flight while group j is multiplied
    uint32_t kw2[4] = {0u, 0u, 0u, 0u}, vw2[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    int32_t vl3[2] = {-1, -1}, tok2 = 0x7FFFFFFF, tf2 = 0;
    if (j + 2 < j_end_raw) {
      load_k(j + 2, kw2);
      tok2 = load_tok(j + 2);
      tf2 = cache.k_keep[slot0 + (j + 2) * 32];
      load_v(vl2[0], vw2[0]);
      load_v(vl2[1], vw2[1]);
      load_vloc(j + 3, vl3);
    }
    // Group j+1 is decoded unconditionally (past the split's end the words are zeros and the
    // buffer is not read again), so the decode has no branch to keep it apart from the products.
    const int nbuf = buf ^ 1;
    // Every wave multiplies every group, so the decode sits in the same straight-line code as
    // the products: an inactive wave has zero queries and writes nothing, and a group that
    // lies past all of a wave's rows is masked to -inf, which leaves (m, l, O) unchanged.
    {
      f32x16 acc, acc_lo;                      // q.hi and q.lo in two chains, added at the end
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc_lo[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 ah = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.khi[buf][lo][ks * 16 + 8 * hi]));
        bf16x8 al = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.klo[buf][lo][ks * 16 + 8 * hi]));
        acc = mfma32(ah, qb[ks], acc);
        acc_lo = mfma32(al, qb[ks], acc_lo);
      }
      decode_k(kw1, nbuf);                     // VALU work beside the matrix products
      // issue order: each product of the two chains followed by a share of the decode
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read (K operand)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix product
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU (decode)
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += acc_lo[i];
      float x[16];
      float tmax = -INFINITY;
      const bool full = m_valid == 32 && (!causal || sm.tok[buf][31] <= off + r0);   // uniform per wave
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = acc[i];   // raw products; the scale c > 0 is applied below
      if (!full) {
        // slots past m_valid hold the sentinel 0x7FFFFFFF, so one compare covers both masks
        const int lim = causal ? (int)pos : 0x7FFFFFFE;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (sm.tok[buf][acc_row(i, hi)] <= lim) ? x[i] : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, x[i]);
      tmax = half_max(tmax);
      const float mnew = fmaxf(m_run, tmax * c);   // max(c x) = c max(x) for c > 0
      // an all-masked row so far (mnew = -inf) keeps l = 0 and adds p = 0
      const float msafe = mnew > -INFINITY ? mnew : 0.f;
      const float alpha = mnew > -INFINITY ? fast_exp2(m_run - mnew) : 1.f;
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(fmaf(x[i], c, -msafe));
        ps += p[i];
      }
      l_run = l_run * alpha + ps;
      m_run = mnew;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {   // no row of the wave moved its max: skip
#pragma unroll
        for (int mb = 0; mb < GPR; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
      }
      // O^T[ch][row] += sum_key V^T[ch][key] P^T[key][row], keys in the accumulator's order
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        f16x8 pb;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pb[jj] = (_Float16)p[ks2 * 8 + jj];
        const int kbase = 16 * ks2 + 4 * hi;
#pragma unroll
        for (int mb = 0; mb < GPR; ++mb) {
          const _Float16* vr = &sm.vt[buf][mb * 32 + lo][0];
          f16x8 va;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            va[jj] = vr[kbase + jj];
            va[4 + jj] = vr[kbase + 8 + jj];
          }
          o[mb] = mfma32h(va, pb, o[mb]);
        }
      }
      decode_v(vw1, vl1, nbuf);
#pragma unroll
      for (int i = 0; i < 2 * GPR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read (V operand)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix product
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU (decode)
      }
    }
    if (threadIdx.x < 32) sm.tok[nbuf][threadIdx.x] = tok1;
    // set 2 becomes set 1
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      kw1[k] = kw2[k];
      vw1[0][k] = vw2[0][k];
      vw1[1][k] = vw2[1][k];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      vl1[u] = vl2[u];
      vl2[u] = vl3[u];
    }
    tok1 = tok2;
    tf0 = tf1;
    tf1 = tf2;
  }

  if (!active) return;
  const float lt = l_run + swap_half(l_run);
  const int64_t row = r0 + lo;
  if (row >= Nq) return;
  float* pr = part + (((int64_t)h * Nq + row) * pstride + split) * PSTRIDE;
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
// out = sum O_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.  One block per (head, row): the
// splits' (m, l) are read in parallel into LDS, M and L come from fixed-order trees, and
// each output channel is summed by 256 / D threads over interleaved splits (independent
// loads), whose partials are then added in thread order.  Deterministic for a given nsplit.
constexpr int kMergeThreads = 256;
constexpr int kMaxSplit = 256;

__global__ void __launch_bounds__(kMergeThreads)
attend_merge(const float* __restrict__ part, float* __restrict__ out, float* __restrict__ lse,
             int D, int nsplit) {
  __shared__ float sc[kMaxSplit], red[kMergeThreads];
  const int64_t hr = blockIdx.x;             // h * Nq + row
  const int PSTRIDE = D + 2;
  const float* pr = part + hr * nsplit * PSTRIDE;
  const int t = threadIdx.x;
  float mv = -INFINITY, lv = 0.f;
  if (t < nsplit) {
    mv = pr[(int64_t)t * PSTRIDE];
    lv = pr[(int64_t)t * PSTRIDE + 1];
  }
  red[t] = mv;
  __syncthreads();
  for (int w = kMergeThreads / 2; w >= 1; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float scale = 0.f;
  if (t < nsplit && mv > -INFINITY) scale = exp2f(mv - M);
  sc[t] = scale;                             // kMergeThreads == kMaxSplit
  red[t] = lv * scale;
  __syncthreads();
  for (int w = kMergeThreads / 2; w >= 1; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  const float L = red[0];
  __syncthreads();
  const int per = kMergeThreads / D;         // threads per channel (2 or 4)
  const int cc = t % D, q = t / D;
  float acc = 0.f;
#pragma unroll 4
  for (int s2 = q; s2 < nsplit; s2 += per) acc += pr[(int64_t)s2 * PSTRIDE + 2 + cc] * sc[s2];
  red[t] = acc;
  __syncthreads();
  if (q == 0) {
    float o = 0.f;
    for (int k = 0; k < per; ++k) o += red[k * D + cc];
    out[hr * D + cc] = (L > 0.f) ? o / L : 0.f;
  }
  if (t == 0) lse[hr] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// Decode-shaped calls (G * Nq <= 16 query rows per KV head, e.g. one new token per query
// head).  A 32-row matrix-core tile would be almost all padding, so the rows' dot products
// run on the VALU in float32, and the packed cache is streamed by many small independent
// waves, each with one round of loads:
//   attend_dec_logits: one wave per K group of 32 retained tokens.  The group's code words
//     and (scale, zero) pairs are staged in LDS by coalesced loads; lane = (token, half of
//     the channel list); the halves are added with a lane swap.  Writes x = s * q.K_hat (base
//     2, -inf where the causal mask hides the token) to a scratch row indexed by token.
//   attend_dec_values: one wave per 64 consecutive V rows of one width zone (contiguous, one
//     width).  Lane = row: gathers the rows' logits, online softmax per query row (wave max,
//     per-lane sums); then lane = channels: O[r][c] += p * V_hat, 16 rows' words in flight at
//     a time.  The block's four waves merge in LDS into one split partial (attend_merge).
// ---------------------------------------------------------------------------------------
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecMaxRows = 16;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Copy n consecutive elements (n < 2^31) from global memory to LDS with the 64 lanes of a wave:
// batches of 16 independent loads per lane, then their stores, so a batch costs one latency.
template <typename T>
__device__ __forceinline__ void wave_stage(T* __restrict__ dst, const T* __restrict__ src, int n, int lane) {
  constexpr int B = 16;
  for (int w0 = 0; w0 < n; w0 += 64 * B) {
    T t[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int w = w0 + k * 64 + lane;
      if (w < n) t[k] = src[w];
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int w = w0 + k * 64 + lane;
      if (w < n) dst[w] = t[k];
    }
  }
}

// Nonzero-width K channels of head g grouped by width (2, 4, 8, then 16 bits), each group in
// channel order: {channel, word offset, param slot, width}, by one block scan.  cnt[k] is the
// first position of width class k (cnt[4] = all nonzero channels).  Widths outside
// {2,4,8,16} count as 0.
template <int D, int NT>
__device__ void dec_channel_table(const kvc_packed_cache& cache, int g, int32_t (*kch)[4], uint64_t* scan,
                                  int* cnt) {
  const int t = threadIdx.x;
  uint32_t b = 0;
  int cls = 4;
  uint64_t f = 0;
  if (t < D) {
    b = cache.k_width[(int64_t)g * D + t];
    cls = b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : b == 16 ? 3 : 4;
    // word offset [0,16), param slot [16,24), one 8-bit count per width class from bit 24
    if (cls < 4) f = (uint64_t)b | ((uint64_t)(cls < 3) << 16) | (1ull << (24 + 8 * cls));
  }
  uint64_t tf;
  const uint64_t ef = block_excl_scan<NT>(f, &tf, scan);
  if (t < D && cls < 4) {
    int pos = (int)((ef >> (24 + 8 * cls)) & 0xFF);
    for (int k = 0; k < cls; ++k) pos += (int)((tf >> (24 + 8 * k)) & 0xFF);
    kch[pos][0] = t;
    kch[pos][1] = (int32_t)(ef & 0xFFFF);
    kch[pos][2] = (int32_t)((ef >> 16) & 0xFF);
    kch[pos][3] = (int32_t)b;
  }
  if (t == 0) {
    int acc = 0;
    for (int k = 0; k < 4; ++k) {
      cnt[k] = acc;
      acc += (int)((tf >> (24 + 8 * k)) & 0xFF);
    }
    cnt[4] = acc;
  }
  __syncthreads();
}

// s[r] += code * a[pos][r] over the positions [p0, p1) of one width class B in {2,4,8}, for
// this lane's token lo and channel half hi (positions p0 + hi, p0 + hi + 2, ...).  The
// group's words are staged in width-class order, so position pos's words start at
// wbase + B * (pos - p0): no table lookup between the loads.
template <int B, int R>
__device__ __forceinline__ void dec_dot_class(float (&s)[R], const uint32_t* kw, const float (*a)[R], int p0,
                                              int p1, int wbase, int lo, int hi) {
  const int wo = (lo * B) >> 5, sh = (lo * B) & 31;
#pragma unroll 4
  for (int pos = p0 + hi; pos < p1; pos += 2) {
    const float cf = (float)((kw[wbase + B * (pos - p0) + wo] >> sh) & ((1u << B) - 1u));
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = fmaf(cf, a[pos][r], s[r]);
  }
}

// Per row r < G * Nq of KV head g: query head g*G + r/Nq, query row r%Nq.  Row-indexed tables
// once per block (no divisions in the loops): the row's index in [H_q][Nq] and its last
// visible token.
__device__ __forceinline__ void dec_row_tables(int g, int G, int64_t N, int64_t Nq, int64_t shift, int causal,
                                               int nr, int64_t* rowi, int64_t* lim) {
  const int r = threadIdx.x;
  if (r < kDecMaxRows) {
    const int nqi = (int)Nq;
    rowi[r] = r < nr ? (int64_t)(g * G + r / nqi) * Nq + r % nqi : 0;
    lim[r] = r < nr ? (causal ? N - Nq + shift + r % nqi : N - 1) : -1;
  }
}

template <int D, int R>
struct DecLogitSmem {
  float qt[D][R];                        // query rows, channel-major
  float a[kDecWaves][D][R];              // a group's scale * q (quantised positions), q (16-bit ones)
  uint16_t wmap[16 * D];                 // a group's word w goes to LDS word wmap[w] (width-class order)
  int32_t kch[D][4];
  uint32_t kw[kDecWaves][16 * D];        // a group's code words (at most 16 per channel)
  float2 kp[kDecWaves][D];               // a group's (scale, zero) pairs
  int64_t rowi[kDecMaxRows], lim[kDecMaxRows];
  uint64_t scan[kDecWaves];
  int cnt[5];
  int wb[5];                             // first staged word of each width class
};

template <int D, int R>
__global__ void __launch_bounds__(kDecThreads)
attend_dec_logits(const uint16_t* __restrict__ q, kvc_packed_cache cache, float* __restrict__ xl,
                  int G, int Hkv, int64_t N, int64_t Nq, int64_t shift, int causal, float c, int32_t* status) {
  __shared__ DecLogitSmem<D, R> sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const int g = blockIdx.y;
  const int nr = G * (int)Nq;
  const int64_t* H = cache.header;
  if (H[0] != Hkv || H[1] != D || H[2] != N) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && g == 0) set_status(status, KVC_DEV_BAD_CACHE);
    return;
  }
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t Rg = hp[4], ngroups = hp[22], Wk = hp[20], Qk = hp[21];
  if ((int64_t)blockIdx.x * kDecWaves >= ngroups) return;   // uniform for the block
  dec_row_tables(g, G, N, Nq, shift, causal, nr, sm.rowi, sm.lim);
  dec_channel_table<D, kDecThreads>(cache, g, sm.kch, sm.scan, sm.cnt);
  const int nq = sm.cnt[3], nnz = sm.cnt[4];
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int k = 0; k < 4; ++k) {
      sm.wb[k] = acc;
      acc += (sm.cnt[k + 1] - sm.cnt[k]) * (2 << k);
    }
    sm.wb[4] = acc;
  }
  __syncthreads();
  for (int pos = threadIdx.x; pos < nnz; pos += kDecThreads) {   // the word map (the same for every group)
    const int b = sm.kch[pos][3], cls = b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : 3;
    const int dst = sm.wb[cls] + b * (pos - sm.cnt[cls]);
    for (int i = 0; i < b; ++i) sm.wmap[sm.kch[pos][1] + i] = (uint16_t)(dst + i);
  }
  for (int idx = threadIdx.x; idx < R * D; idx += kDecThreads) {
    const int r = idx / D, cc = idx % D;
    sm.qt[cc][r] = r < nr ? bf16_bits_to_f32(q[sm.rowi[r] * D + cc]) : 0.f;
  }
  __syncthreads();
  // groups blockIdx.x * 4 + wave, then every gridDim.x * 4 further (no block barrier follows)
  for (int64_t j = (int64_t)blockIdx.x * kDecWaves + wave; j < ngroups; j += (int64_t)gridDim.x * kDecWaves) {
    const uint32_t* gw = cache.k_words + hp[18] + j * Wk;
    {
      constexpr int SB = 16;
      for (int w0 = 0; w0 < (int)Wk; w0 += 64 * SB) {
        uint32_t t[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int w = w0 + k * 64 + lane;
          if (w < (int)Wk) t[k] = gw[w];
        }
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int w = w0 + k * 64 + lane;
          if (w < (int)Wk) sm.kw[wave][sm.wmap[w]] = t[k];
        }
      }
    }
    wave_stage(sm.kp[wave], reinterpret_cast<const float2*>(cache.k_par) + hp[19] + j * Qk, (int)Qk, lane);
    const int64_t tix = j * 32 + lo;
    const bool tok_ok = tix < Rg;
    const int64_t tok = tok_ok ? (int64_t)cache.k_keep[hp[17] + tix] : 0;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // quantised channels: K_hat = scale * code + zero, so q . K_hat = sum code * (scale q) + sum zero q
    float bias[R];
#pragma unroll
    for (int r = 0; r < R; ++r) bias[r] = 0.f;
    for (int pos = lane; pos < nnz; pos += 64) {
      const int4 ch = *reinterpret_cast<const int4*>(sm.kch[pos]);
      const float2 sz = pos < nq ? sm.kp[wave][ch.z] : make_float2(1.f, 0.f);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float qv = sm.qt[ch.x][r];
        sm.a[wave][pos][r] = sz.x * qv;
        bias[r] = fmaf(sz.y, qv, bias[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) bias[r] = wave_sum(bias[r]);
    __builtin_amdgcn_wave_barrier();

    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = 0.f;
    dec_dot_class<2, R>(s, sm.kw[wave], sm.a[wave], sm.cnt[0], sm.cnt[1], sm.wb[0], lo, hi);
    dec_dot_class<4, R>(s, sm.kw[wave], sm.a[wave], sm.cnt[1], sm.cnt[2], sm.wb[1], lo, hi);
    dec_dot_class<8, R>(s, sm.kw[wave], sm.a[wave], sm.cnt[2], sm.cnt[3], sm.wb[2], lo, hi);
    {                                                        // 16-bit channels: raw bf16
      const int wo = sm.wb[3] + (lo >> 1);
      const uint32_t s16 = (lo & 1) ? 0u : 16u;
#pragma unroll 4
      for (int pos = nq + hi; pos < nnz; pos += 2) {
        const float kv = __uint_as_float((sm.kw[wave][wo + 16 * (pos - nq)] << s16) & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = fmaf(kv, sm.a[wave][pos][r], s[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] += swap_half(s[r]) + bias[r];
    if (hi == 0 && tok_ok) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r < nr) xl[sm.rowi[r] * N + tok] = tok <= sm.lim[r] ? s[r] * c : -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

constexpr int kVRows = 64;              // V rows per chunk of the value pass (one per lane)

template <int D, int R>
struct DecValueSmem {
  int64_t rowi[kDecMaxRows], lim[kDecMaxRows];
  float pv[kDecWaves][kVRows][R];        // per V row of the chunk: the query rows' weights
  float wml[kDecWaves][2][R];
  float wo[kDecWaves][R][D];
};

template <int D, int R>
__global__ void __launch_bounds__(kDecThreads)
attend_dec_values(kvc_packed_cache cache, const float* __restrict__ xl, float* __restrict__ part,
                  int G, int Hkv, int64_t N, int64_t Nq, int nsplit, int pstride) {
  constexpr int CPL = D / 64;            // channels per lane
  constexpr int GPR = D / 32;
  constexpr int PSTRIDE = D + 2;
  constexpr int NB = 16;                 // V rows whose words are in flight together
  __shared__ DecValueSmem<D, R> sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, g = blockIdx.y;
  const int nr = G * (int)Nq;
  const int64_t* H = cache.header;
  if (H[0] != Hkv || H[1] != D || H[2] != N) return;         // reported by attend_dec_logits
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  dec_row_tables(g, G, N, Nq, 0, 0, nr, sm.rowi, sm.lim);
  __syncthreads();
  int64_t nch[4], ctot = 0;
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    nch[z] = (hp[z] + kVRows - 1) / kVRows;
    ctot += nch[z];
  }
  const int64_t cps = (ctot + nsplit - 1) / nsplit;
  const int64_t cb = (int64_t)split * cps;
  const int64_t ce = cb + cps < ctot ? cb + cps : ctot;

  float m[R], l[R], o[R][CPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[r][k] = 0.f;
  }
  const int c0 = lane * CPL, grp = c0 / 32, e2 = c0 % 32;
  for (int64_t ck = cb + wave; ck < ce; ck += kDecWaves) {
    int z = 0;
    int64_t cz = ck;
    while (z < 3 && cz >= nch[z]) {
      cz -= nch[z];
      ++z;
    }
    const int b = 2 << z;
    const int64_t r0 = cz * kVRows;
    const int nrows = (int)(hp[z] - r0 < kVRows ? hp[z] - r0 : kVRows);
    // lane = row: the query rows' logits of this V row's token, then the online softmax
    const bool rok = lane < nrows;
    const int64_t tok = rok ? (int64_t)cache.v_idx[hp[5 + z] + r0 + lane] : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float x = -INFINITY;
      if (rok && r < nr) x = xl[sm.rowi[r] * N + tok];
      const float mn = fmaxf(m[r], wave_max(x));
      float p = 0.f;
      if (mn > -INFINITY) {                                  // uniform
        const float alpha = fast_exp2(m[r] - mn);
        p = fast_exp2(x - mn);
        l[r] = fmaf(l[r], alpha, p);
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[r][k] *= alpha;
        m[r] = mn;
      }
      if (lane < kVRows) sm.pv[wave][lane][r] = p;
    }
    __builtin_amdgcn_wave_barrier();
    // lane = channels: O += p * V_hat over the chunk's rows (width b for all of them), the
    // words (and pairs) of 16 rows in flight at a time; rows past nrows repeat the last and
    // contribute 0
    const int vstride = GPR * b;                             // words per V row
    const uint32_t* vw = cache.v_words + hp[9 + z] + r0 * vstride + grp * b + ((e2 * b) >> 5);
    const float2* vp = reinterpret_cast<const float2*>(cache.v_par) + hp[13 + z] + r0 * GPR + grp;
    const uint32_t mask = b == 16 ? 0xFFFFu : (1u << b) - 1u;
    const int shift = (e2 * b) & 31;
#pragma unroll 1
    for (int t0 = 0; t0 < nrows; t0 += NB) {
      uint32_t w[NB];
      float2 sz[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int tp = t0 + k < nrows ? t0 + k : nrows - 1;
        w[k] = vw[tp * vstride];
        sz[k] = make_float2(0.f, 0.f);
      }
      if (b < 16) {                                          // uniform: zones 2/4/8 have pairs
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          const int tp = t0 + k < nrows ? t0 + k : nrows - 1;
          sz[k] = vp[tp * GPR];
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int tp = t0 + k;
        const float* pr = sm.pv[wave][tp < kVRows ? tp : kVRows - 1];
        float v[CPL];
#pragma unroll
        for (int kk = 0; kk < CPL; ++kk) {
          const uint32_t code = (w[k] >> (shift + kk * b)) & mask;
          const float vv = b == 16 ? bf16_bits_to_f32(code) : fmaf(sz[k].x, (float)code, sz[k].y);
          v[kk] = tp < nrows ? vv : 0.f;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int kk = 0; kk < CPL; ++kk) o[r][kk] = fmaf(pr[r], v[kk], o[r][kk]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // merge the four waves' (m, l, O) and write this split's partial for every row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float lt = wave_sum(l[r]);
    if (lane == 0) {
      sm.wml[wave][0][r] = m[r];
      sm.wml[wave][1][r] = lt;
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) sm.wo[wave][r][lane * CPL + k] = o[r][k];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nr * D; idx += kDecThreads) {
    const int r = idx / D, cc = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm.wml[w][0][r]);
    float Lr = 0.f, Or = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = sm.wml[w][0][r];
        const float sc = mw > -INFINITY ? fast_exp2(mw - M) : 0.f;
        Lr = fmaf(sm.wml[w][1][r], sc, Lr);
        Or = fmaf(sm.wo[w][r][cc], sc, Or);
      }
    }
    float* pr = part + (sm.rowi[r] * pstride + split) * PSTRIDE;
    if (cc == 0) {
      pr[0] = M;
      pr[1] = Lr;
    }
    pr[2 + cc] = Or;
  }
}

// ---------------------------------------------------------------------------------------
// The append buffer: tokens generated after compression, raw bf16 [H_kv][n_new][d] at positions
// N .. N+n_new-1 (RDKV summary §2.3 keeps new tokens beside the packed zones).  One wave per
// query row: lanes = 64 new tokens at a time for the logits (the row in LDS, each lane reading
// its token's key row as 16-byte loads), an exact online softmax, then lanes = channels for
// O += p * v.  The row's (m, l, O) is one more split for attend_merge.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
attend_append(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
              float* __restrict__ part, int G, int Hq, int64_t Nq, int64_t n_new, int causal, float c,
              int split, int pstride) {
  constexpr int CPL = D / 64;
  constexpr int PSTRIDE = D + 2;
  __shared__ float qs[4][D];
  __shared__ float pv[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t hr = (int64_t)blockIdx.x * 4 + wave;          // h * Nq + i
  if (hr >= (int64_t)Hq * Nq) return;                         // uniform per wave; no block barrier follows
  const int h = (int)(hr / Nq);
  const int64_t i = hr % Nq;
  const int g = h / G;
  for (int cc = lane; cc < D; cc += 64) qs[wave][cc] = bf16_bits_to_f32(q[hr * D + cc]);
  // the row sits at position N + n_new - Nq + i: it sees new tokens t <= n_new - Nq + i
  int64_t nt = n_new;
  if (causal) {
    const int64_t lim = n_new - Nq + i + 1;
    nt = lim < nt ? lim : nt;
    if (nt < 0) nt = 0;
  }
  const uint16_t* kg = kn + (int64_t)g * n_new * D;
  const uint16_t* vg = vn + (int64_t)g * n_new * D;
  float m = -INFINITY, l = 0.f, o[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) o[k] = 0.f;
  __builtin_amdgcn_wave_barrier();
  for (int64_t t0 = 0; t0 < nt; t0 += 64) {
    const int64_t t = t0 + lane;
    float x = -INFINITY;
    if (t < nt) {
      const uint4* kr = reinterpret_cast<const uint4*>(kg + t * D);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const uint4 w = kr[j];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fmaf(qs[wave][8 * j + 2 * e], __uint_as_float(ww[e] << 16), acc);
          acc = fmaf(qs[wave][8 * j + 2 * e + 1], __uint_as_float(ww[e] & 0xFFFF0000u), acc);
        }
      }
      x = acc * c;
    }
    const float mn = fmaxf(m, wave_max(x));
    float p = 0.f;
    if (mn > -INFINITY) {                                    // uniform
      const float alpha = fast_exp2(m - mn);
      p = fast_exp2(x - mn);
      l = fmaf(l, alpha, p);
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[k] *= alpha;
      m = mn;
    }
    pv[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    const int cnt = (int)(nt - t0 < 64 ? nt - t0 : 64);
#pragma unroll 8
    for (int tp = 0; tp < cnt; ++tp) {
      const float pp = pv[wave][tp];
      const uint16_t* vr = vg + (t0 + tp) * D + lane * CPL;
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[k] = fmaf(pp, bf16_bits_to_f32(vr[k]), o[k]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float lt = wave_sum(l);
  float* pr = part + (hr * pstride + split) * PSTRIDE;
  if (lane == 0) {
    pr[0] = m;
    pr[1] = lt;
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k) pr[2 + lane * CPL + k] = o[k];
}

// The decode path addresses a head's V words with 32-bit offsets: N * d / 2 (the words of a
// head whose every token is kept at 16 bits) must stay below 2^32.
bool use_decode(const Layer& L) {
  return (int64_t)L.G * L.nq <= kDecMaxRows && L.n * (int64_t)L.d / 2 < (int64_t(1) << 32);
}

int nsplit_decode(const Layer& L) {
  const int64_t cmax = (L.n + kVRows - 1) / kVRows + 4;  // V chunks per head, at most
  int64_t want = (1024 + L.hkv - 1) / L.hkv;
  const int64_t cap = (cmax + 3) / 4;                    // at least 4 chunks (one per wave) per split
  if (want > cap) want = cap;
  if (want > kMaxSplit - 1) want = kMaxSplit - 1;   // one more for the append buffer
  if (want < 1) want = 1;
  return (int)want;
}

int nsplit_of(const Layer& L) {
  const int nRT = (int)((L.nq + kRows - 1) / kRows);
  const int64_t bps = (int64_t)L.hkv * ((L.G * nRT + kWaves - 1) / kWaves);   // blocks per split
  int64_t want = (1024 + bps - 1) / bps;
  const int64_t maxs = (L.n + 32 * 8 - 1) / (32 * 8);   // at least 8 groups per split
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  if (want > kMaxSplit - 1) want = kMaxSplit - 1;   // one more for the append buffer
  return (int)want;
}

}  // namespace

size_t attend_ws_bytes(const Layer& L) {
  WsPlan p;
  const bool dec = use_decode(L);
  const int nsplit = dec ? nsplit_decode(L) : nsplit_of(L);
  p.take((size_t)L.hq * L.nq * (nsplit + 1) * (L.d + 2) * sizeof(float));   // + the append buffer's split
  if (dec) p.take((size_t)L.hq * L.nq * L.n * sizeof(float));     // logits by token
  return p.off;
}

hipError_t launch_attend(const Layer& L, const uint16_t* q, const kvc_packed_cache& cache,
                         float* out, float* lse, char* ws, hipStream_t s, const uint16_t* k_new,
                         const uint16_t* v_new, int64_t n_new) {
  const bool dec = use_decode(L);
  const int nsplit = dec ? nsplit_decode(L) : nsplit_of(L);
  const int pstride = n_new > 0 ? nsplit + 1 : nsplit;      // partials per row
  WsPlan p;
  float* part = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * L.nq * (nsplit + 1) * (L.d + 2) * sizeof(float)));
  (void)launch_reset_status(ws, s);
  int32_t* status = reinterpret_cast<int32_t*>(ws);
  if (dec) {
    float* xl = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * L.nq * L.n * sizeof(float)));
    int64_t nb1 = ((L.n + 31) / 32 + kDecWaves - 1) / kDecWaves;   // blocks of 4 groups per head, at most
    const int64_t cap1 = (1024 + L.hkv - 1) / L.hkv;                 // the blocks loop over the rest
    if (nb1 > cap1) nb1 = cap1;
    const dim3 g1((unsigned)nb1, (unsigned)L.hkv);
    const dim3 g3((unsigned)nsplit, (unsigned)L.hkv);
    const int rows = L.G * (int)L.nq;
#define KVC_DEC(DD, RR)                                                                                   \
  do {                                                                                                    \
    attend_dec_logits<DD, RR><<<g1, kDecThreads, 0, s>>>(q, cache, xl, L.G, L.hkv, L.n, L.nq, n_new,      \
                                                         L.causal, L.c_log2, status);                    \
    attend_dec_values<DD, RR><<<g3, kDecThreads, 0, s>>>(cache, xl, part, L.G, L.hkv, L.n, L.nq, nsplit,  \
                                                         pstride);                                       \
  } while (0)
    if (L.d == 128) {
      if (rows <= 1) KVC_DEC(128, 1);
      else if (rows <= 2) KVC_DEC(128, 2);
      else if (rows <= 4) KVC_DEC(128, 4);
      else if (rows <= 8) KVC_DEC(128, 8);
      else KVC_DEC(128, 16);
    } else {
      if (rows <= 1) KVC_DEC(64, 1);
      else if (rows <= 2) KVC_DEC(64, 2);
      else if (rows <= 4) KVC_DEC(64, 4);
      else if (rows <= 8) KVC_DEC(64, 8);
      else KVC_DEC(64, 16);
    }
#undef KVC_DEC
  } else {
    const int nRT = (int)((L.nq + kRows - 1) / kRows);
    dim3 grid((unsigned)((L.G * nRT + kWaves - 1) / kWaves), (unsigned)nsplit, (unsigned)L.hkv);
    if (L.d == 128)
      attend_split<128><<<grid, kThreadsA, 0, s>>>(q, cache, part, L.G, L.hkv, L.n, L.nq, L.causal, L.c_log2, nsplit,
                                                   n_new, pstride, status);
    else
      attend_split<64><<<grid, kThreadsA, 0, s>>>(q, cache, part, L.G, L.hkv, L.n, L.nq, L.causal, L.c_log2, nsplit,
                                                  n_new, pstride, status);
  }
  if (n_new > 0) {
    const unsigned nb = (unsigned)(((int64_t)L.hq * L.nq + 3) / 4);
    if (L.d == 128)
      attend_append<128><<<nb, 256, 0, s>>>(q, k_new, v_new, part, L.G, L.hq, L.nq, n_new, L.causal, L.c_log2,
                                            nsplit, pstride);
    else
      attend_append<64><<<nb, 256, 0, s>>>(q, k_new, v_new, part, L.G, L.hq, L.nq, n_new, L.causal, L.c_log2,
                                           nsplit, pstride);
  }
  attend_merge<<<(unsigned)((int64_t)L.hq * L.nq), kMergeThreads, 0, s>>>(part, out, lse, L.d, pstride);
  return hipGetLastError();
}

}  // namespace kvc
