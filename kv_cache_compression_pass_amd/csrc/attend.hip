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
//   V_hat -> LDS transposed as fp16 [channel][token], scaled by 2^-E_g: E_g is chosen per KV head
//            from a bound on |V_hat| over the whole packed head (attend_vbound), so that the
//            largest value lands in [2^14, 2^15) and every value keeps fp16's 11 bits down to
//            2^-24 of that bound, whatever the magnitude of V (the partial O is scaled back by
//            2^E_g when it is written),
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
// With many query rows, each group would be decoded once per block of 64 rows.  Then a first
// launch of the same kernel only decodes, one block per key split and head, and writes every
// group's K_hat hi / lo and V_hat^T to the workspace (192 d bytes a group); the second launch
// copies those records into its LDS buffers in place of the decode (same values, so the same
// results), and its loop is left with the products and the softmax.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kWaves = 8;
constexpr int kThreadsA = 64 * kWaves;
constexpr int kRows = 32;   // query rows per wave
// attend_split modes: decode each group into LDS and multiply it (one pass); decode only, writing
// each group's decoded record to the workspace; multiply records decoded by the previous mode
constexpr int kModeFused = 0, kModeDecodeOut = 1, kModePredecoded = 2;

template <int D>
struct AttnSmem {
  // two buffers: group j is decoded into buffer j & 1.  Rows of D/2 + 2 words: the operand reads
  // (two 8-byte halves a lane, 32 lanes a pass) start 2 words apart, so every lane has its own banks
  uint16_t khi[2][32][D + 4];
  uint16_t klo[2][32][D + 4];
  _Float16 vt[2][D][32 + 4];   // rows of 18 words: the operand reads (8 bytes a lane) hit distinct banks
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

// ---------------------------------------------------------------------------------------
// Bound on |V_hat| per KV head, for the fp16 staging of V_hat in attend_split: the largest of
// |zero| and |zero + scale * (2^b - 1)| over every (scale, zero) pair of the 2/4/8-bit zones (the
// dequantiser fmaf(scale, code, zero) is monotone in the code, so these are its extremes) and of
// |v| over the raw bf16 words of the 16-bit zone.  Non-negative floats order as their bit
// patterns, so the bound is kept as uint32 bits and combined with atomicMax (order-free, so the
// result does not depend on scheduling).
// ---------------------------------------------------------------------------------------
__global__ void attend_vbound_init(uint32_t* vb, int Hkv) {
  if ((int)threadIdx.x < Hkv) vb[threadIdx.x] = 0u;
}

template <int D>
__global__ void __launch_bounds__(256)
attend_vbound(kvc_packed_cache cache, uint32_t* __restrict__ vb, int Hkv, int64_t N) {
  constexpr int GPR = D / 32;
  __shared__ uint32_t red[4];
  const int64_t* H = cache.header;
  if (H[0] != Hkv || H[1] != D || H[2] != N) return;   // reported by attend_split
  const int g = blockIdx.y;
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t np0 = hp[0] * GPR, np1 = hp[1] * GPR, np2 = hp[2] * GPR;
  const int64_t nw3 = hp[3] * GPR * 16;
  const int64_t total = np0 + np1 + np2 + nw3;
  const float2* par = reinterpret_cast<const float2*>(cache.v_par);
  uint32_t m = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    if (i < np0 + np1 + np2) {
      const int z = i < np0 ? 0 : (i < np0 + np1 ? 1 : 2);
      const int64_t k = i - (z == 0 ? 0 : (z == 1 ? np0 : np0 + np1));
      const float2 sz = par[hp[13 + z] + k];
      const float top = (float)((1 << (2 << z)) - 1);
      const uint32_t a = __float_as_uint(fabsf(sz.y));
      const uint32_t b = __float_as_uint(fabsf(fmaf(sz.x, top, sz.y)));
      m = max(m, max(a, b));
    } else {
      const uint32_t w = cache.v_words[hp[12] + (i - np0 - np1 - np2)];
      m = max(m, max((w & 0x7FFFu) << 16, w & 0x7FFF0000u));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t r = max(max(red[0], red[1]), max(red[2], red[3]));
    if (r != 0u) atomicMax(vb + g, r);
  }
}

// Power-of-two exponent E for the fp16 staging of a head whose |V_hat| bound has bits vb: the
// bound times 2^-E lies in [2^14, 2^15) (E is clamped so that 2^E and 2^-E are normal floats).
__device__ __forceinline__ int vscale_exp(uint32_t vb) {
  if (vb == 0u) return 0;
  const int e = (int)((vb >> 23) & 0xFF) - 127 - 14;
  return e < -100 ? -100 : (e > 110 ? 110 : e);
}

template <int D, int MODE>
__global__ void __launch_bounds__(kThreadsA)
attend_split(const uint16_t* __restrict__ q, kvc_packed_cache cache, float* __restrict__ part,
             const uint32_t* __restrict__ vbound, int G, int Hkv, int64_t N, int64_t Nq, int causal, float c,
             int nsplit, int64_t shift, int pstride, int32_t* status, uint16_t* __restrict__ pre) {
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
  const int nRT = (int)((Nq + kRows - 1) / kRows);
  int rb = blockIdx.x, split = blockIdx.y, g = blockIdx.z;
  if constexpr (MODE == kModePredecoded) {
    // One-dimensional grid.  Blocks are dealt to the eight XCDs in turn, so the row blocks of one
    // (split, head), which read the same records, are given ids eight apart: one XCD, one L2.
    const int nrb = (G * nRT + kWaves - 1) / kWaves;
    const int id = blockIdx.x, chunk = id / (8 * nrb), rem = id % (8 * nrb);
    const int u = chunk * 8 + rem % 8;
    if (u >= nsplit * Hkv) return;             // padding of the last eight (split, head) units
    rb = rem / 8;
    split = u % nsplit;
    g = u / nsplit;
  }
  const int pair = rb * kWaves + wave;
  const bool active = MODE != kModeDecodeOut && pair < G * nRT;
  const int hl = active ? pair % G : 0;
  const int rt = active ? pair / G : 0;
  const int h = g * G + hl;
  const int64_t r0 = (int64_t)rt * kRows;
  const int64_t off = N - Nq + shift;         // row r sits at position off + r

  const int64_t* H = cache.header;
  if (H[0] != Hkv || H[1] != D || H[2] != N) {
    if (threadIdx.x == 0 && rb == 0 && split == 0) set_status(status, KVC_DEV_BAD_CACHE);
    return;
  }
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t R = hp[4];
  const int64_t ngroups = hp[22];
  const int64_t Wk = hp[20];
  const int64_t Qk = hp[21];
  const int vexp = vscale_exp(vbound[g]);
  const float vscale = __builtin_amdgcn_ldexpf(1.f, -vexp);   // V_hat is staged as fp16(V_hat * 2^-E)
  const int64_t gps = (ngroups + nsplit - 1) / nsplit;
  const int64_t j_begin = (int64_t)split * gps;
  const int64_t j_end_raw = j_begin + gps < ngroups ? j_begin + gps : ngroups;

  // channel table of this head's K packing: one uint64 per channel packs {words (16 bits),
  // params (16 bits), an 8-bit count per width class}; one block scan places every channel
  if constexpr (MODE != kModePredecoded) {
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
  if constexpr (MODE != kModeDecodeOut) {
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
    int last_pair = rb * kWaves + kWaves - 1;
    if (last_pair >= G * nRT) last_pair = G * nRT - 1;
    int64_t lr = (int64_t)(last_pair / G) * kRows + kRows - 1;
    if (lr >= Nq) lr = Nq - 1;
    pmax_block = causal ? off + lr : N - 1;
    if (MODE == kModeDecodeOut) pmax_block = causal ? off + Nq - 1 : N - 1;
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

  // A group's decoded record in `pre` (written by the decode-only mode, read by the predecoded
  // mode): K_hat hi [32][D] and lo [32][D] (bf16 bits), then V_hat^T [D][32] (fp16 bits of the
  // scaled values), 192 D bytes.  Thread t moves the t-th chunk of D / 8 bytes of each array.
  using Chunk = typename std::conditional<D == 128, uint4, uint2>::type;
  const int64_t ngmax = (N + 31) / 32;
  auto rec_ptr = [&](int64_t j, int u) -> Chunk* {
    return reinterpret_cast<Chunk*>(pre + ((int64_t)g * ngmax + j) * (3 * 32 * D) + (int64_t)u * 32 * D) +
           threadIdx.x;
  };
  auto lds_chunk = [&](int u, int bf) -> uint2* {   // rows are 8-byte aligned: 8-byte accesses
    const int t = threadIdx.x;
    if (u < 2) {
      const int row = t >> 4, col = (t & 15) * (D / 16);
      return reinterpret_cast<uint2*>(u == 0 ? &sm.khi[bf][row][col] : &sm.klo[bf][row][col]);
    }
    constexpr int CPR = kThreadsA / D;          // chunks per V_hat^T row of 32 tokens
    return reinterpret_cast<uint2*>(&sm.vt[bf][t / CPR][(t % CPR) * (D / 16)]);
  };
  auto put_chunk = [&](const Chunk& v, int u, int bf) {
    uint2* d = lds_chunk(u, bf);
    if constexpr (D == 128) {
      d[0] = make_uint2(v.x, v.y);
      d[1] = make_uint2(v.z, v.w);
    } else {
      d[0] = v;
    }
  };
  auto get_chunk = [&](int u, int bf) -> Chunk {
    const uint2* d = lds_chunk(u, bf);
    if constexpr (D == 128) {
      const uint2 a = d[0], b = d[1];
      return make_uint4(a.x, a.y, b.x, b.y);
    } else {
      return d[0];
    }
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
        const _Float16 hq = (_Float16)(fmaf(sc, (float)((win >> (k * bq)) & mask), zp) * vscale);
        const _Float16 hr = (_Float16)(bf16_bits_to_f32((w[u][k >> 1] >> (16 * (k & 1))) & 0xFFFFu) * vscale);
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
  Chunk ch1[3] = {};                           // the predecoded mode's set 1
  if (MODE == kModePredecoded && j_begin < j_end_raw) {
    const int32_t tok0 = load_tok(j_begin);
    tf0 = cache.k_keep[slot0 + j_begin * 32];
#pragma unroll
    for (int u = 0; u < 3; ++u) put_chunk(*rec_ptr(j_begin, u), u, (int)(j_begin & 1));
    if (threadIdx.x < 32) sm.tok[j_begin & 1][threadIdx.x] = tok0;
    if (j_begin + 1 < j_end_raw) {
      tok1 = load_tok(j_begin + 1);
      tf1 = cache.k_keep[slot0 + (j_begin + 1) * 32];
#pragma unroll
      for (int u = 0; u < 3; ++u) ch1[u] = *rec_ptr(j_begin + 1, u);
    }
  } else if (j_begin < j_end_raw) {
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
    Chunk ch2[3] = {};
    if (j + 2 < j_end_raw) {
      tok2 = load_tok(j + 2);
      tf2 = cache.k_keep[slot0 + (j + 2) * 32];
      if constexpr (MODE == kModePredecoded) {
#pragma unroll
        for (int u = 0; u < 3; ++u) ch2[u] = *rec_ptr(j + 2, u);
      } else {
        load_k(j + 2, kw2);
        load_v(vl2[0], vw2[0]);
        load_v(vl2[1], vw2[1]);
        load_vloc(j + 3, vl3);
      }
    }
    // Group j+1 is decoded unconditionally (past the split's end the words are zeros and the
    // buffer is not read again), so the decode has no branch to keep it apart from the products.
    const int nbuf = buf ^ 1;
    // Every wave multiplies every group, so the decode sits in the same straight-line code as
    // the products: an inactive wave has zero queries and writes nothing, and a group that
    // lies past all of a wave's rows is masked to -inf, which leaves (m, l, O) unchanged.
    if constexpr (MODE == kModeDecodeOut) {
#pragma unroll
      for (int u = 0; u < 3; ++u) *rec_ptr(j, u) = get_chunk(u, buf);
      decode_k(kw1, nbuf);
      decode_v(vw1, vl1, nbuf);
    } else {
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
      if constexpr (MODE == kModeFused) {
        decode_k(kw1, nbuf);                   // VALU work beside the matrix products
        // issue order: each product of the two chains followed by a share of the decode
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read (K operand)
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix product
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU (decode)
        }
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
      if constexpr (MODE == kModeFused) {
        decode_v(vw1, vl1, nbuf);
#pragma unroll
        for (int i = 0; i < 2 * GPR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read (V operand)
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix product
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU (decode)
        }
      } else {
#pragma unroll
        for (int u = 0; u < 3; ++u) put_chunk(ch1[u], u, nbuf);   // group j+1, decoded once before
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
#pragma unroll
    for (int u = 0; u < 3; ++u) ch1[u] = ch2[u];
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
  const float oscale = __builtin_amdgcn_ldexpf(1.f, vexp);   // undo the staging scale (exact)
#pragma unroll
  for (int mb = 0; mb < GPR; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) pr[2 + mb * 32 + acc_row(i, hi)] = o[mb][i] * oscale;
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

// Decode-shaped calls (G * Nq <= 16 query rows per KV head) run the decode kernels (decode.hip).
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

// The decode kernels address a head's V words with 32-bit offsets (N * d / 2, the words of a head
// whose every token is kept at 16 bits, stays below 2^32) and the logits of every retained token
// (at most H_kv N, 16 rows each) likewise.
bool use_decode(const Layer& L) {
  return (int64_t)L.G * L.nq <= kDecMaxRows && L.n * (int64_t)L.d / 2 < (int64_t(1) << 32) &&
         (int64_t)L.hkv * L.n * kDecMaxRows < (int64_t(1) << 31);
}

int nsplit_of(const Layer& L) {
  const int nRT = (int)((L.nq + kRows - 1) / kRows);
  const int64_t bps = (int64_t)L.hkv * ((L.G * nRT + kWaves - 1) / kWaves);   // blocks per split
  int64_t want = (768 + bps - 1) / bps;                  // about 768 blocks (1024 was 2-10 % slower)
  const int64_t maxs = (L.n + 32 * 8 - 1) / (32 * 8);   // at least 8 groups per split
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  if (want > kMaxSplit - 1) want = kMaxSplit - 1;   // one more for the append buffer
  return (int)want;
}

// The decoded records pay off once several row blocks would each decode every group of a head.
constexpr int kPredecodeRowBlocks = 4;
bool use_predecode(const Layer& L) {
  const int nRT = (int)((L.nq + kRows - 1) / kRows);
  return (L.G * nRT + kWaves - 1) / kWaves >= kPredecodeRowBlocks;
}
size_t predecode_bytes(const Layer& L) {
  return (size_t)L.hkv * (size_t)((L.n + 31) / 32) * 3 * 32 * (size_t)L.d * sizeof(uint16_t);
}
// Blocks per head of the decode-only pass: about 1024 in all, at least 8 groups each.
int predecode_nsplit(const Layer& L) {
  int64_t want = (1024 + L.hkv - 1) / L.hkv;
  const int64_t maxs = (L.n + 32 * 8 - 1) / (32 * 8);
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  if (want > 65535) want = 65535;
  return (int)want;
}

}  // namespace

size_t attend_ws_bytes(const Layer& L) {
  WsPlan p;
  const bool dec = use_decode(L);
  const int nsplit = dec ? decode_nsplit(L) : nsplit_of(L);
  p.take((size_t)L.hq * L.nq * (nsplit + 1) * (L.d + 2) * sizeof(float));   // + the append buffer's split
  if (!dec) {
    p.take((size_t)L.hkv * sizeof(uint32_t));                     // |V_hat| bound per head
    if (use_predecode(L)) p.take(predecode_bytes(L));            // decoded records
  } else {
    p.take(decode_ws_bytes(L));
  }
  return p.off;
}

hipError_t launch_attend(const Layer& L, const uint16_t* q, const kvc_packed_cache& cache,
                         float* out, float* lse, char* ws, hipStream_t s, const uint16_t* k_new,
                         const uint16_t* v_new, int64_t n_new) {
  const bool dec = use_decode(L);
  const int nsplit = dec ? decode_nsplit(L) : nsplit_of(L);
  const int pstride = n_new > 0 ? nsplit + 1 : nsplit;      // partials per row
  WsPlan p;
  float* part = reinterpret_cast<float*>(ws + p.take((size_t)L.hq * L.nq * (nsplit + 1) * (L.d + 2) * sizeof(float)));
  if (!dec) (void)launch_reset_status(ws, s);   // the decode path's logits kernel writes the status itself
  int32_t* status = reinterpret_cast<int32_t*>(ws);
  if (dec) {
    char* dws = ws + p.take(decode_ws_bytes(L));
    const hipError_t e = launch_attend_decode(L, q, cache, part, nsplit, pstride, n_new, status, dws, s);
    if (e != hipSuccess) return e;
  } else {
    uint32_t* vb = reinterpret_cast<uint32_t*>(ws + p.take((size_t)L.hkv * sizeof(uint32_t)));
    attend_vbound_init<<<1, 256, 0, s>>>(vb, L.hkv);
    const dim3 gb(64, (unsigned)L.hkv);
    if (L.d == 128)
      attend_vbound<128><<<gb, 256, 0, s>>>(cache, vb, L.hkv, L.n);
    else
      attend_vbound<64><<<gb, 256, 0, s>>>(cache, vb, L.hkv, L.n);
    const int nRT = (int)((L.nq + kRows - 1) / kRows);
    dim3 grid((unsigned)((L.G * nRT + kWaves - 1) / kWaves), (unsigned)nsplit, (unsigned)L.hkv);
    if (use_predecode(L)) {
      uint16_t* pre = reinterpret_cast<uint16_t*>(ws + p.take(predecode_bytes(L)));
      const int ns1 = predecode_nsplit(L);
      const dim3 g1(1, (unsigned)ns1, (unsigned)L.hkv);
      const int64_t units = (int64_t)nsplit * L.hkv;
      const dim3 g2((unsigned)((units + 7) / 8 * 8 * grid.x));
      if (L.d == 128) {
        attend_split<128, kModeDecodeOut><<<g1, kThreadsA, 0, s>>>(q, cache, part, vb, L.G, L.hkv, L.n, L.nq,
                                                                   L.causal, L.c_log2, ns1, n_new, pstride, status, pre);
        attend_split<128, kModePredecoded><<<g2, kThreadsA, 0, s>>>(q, cache, part, vb, L.G, L.hkv, L.n, L.nq,
                                                                      L.causal, L.c_log2, nsplit, n_new, pstride,
                                                                      status, pre);
      } else {
        attend_split<64, kModeDecodeOut><<<g1, kThreadsA, 0, s>>>(q, cache, part, vb, L.G, L.hkv, L.n, L.nq,
                                                                  L.causal, L.c_log2, ns1, n_new, pstride, status, pre);
        attend_split<64, kModePredecoded><<<g2, kThreadsA, 0, s>>>(q, cache, part, vb, L.G, L.hkv, L.n, L.nq,
                                                                     L.causal, L.c_log2, nsplit, n_new, pstride,
                                                                     status, pre);
      }
    } else if (L.d == 128) {
      attend_split<128, kModeFused><<<grid, kThreadsA, 0, s>>>(q, cache, part, vb, L.G, L.hkv, L.n, L.nq, L.causal,
                                                               L.c_log2, nsplit, n_new, pstride, status, nullptr);
    } else {
      attend_split<64, kModeFused><<<grid, kThreadsA, 0, s>>>(q, cache, part, vb, L.G, L.hkv, L.n, L.nq, L.causal,
                                                              L.c_log2, nsplit, n_new, pstride, status, nullptr);
    }
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
