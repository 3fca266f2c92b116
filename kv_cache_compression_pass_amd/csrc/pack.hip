// Mixed-width quantise/pack of one layer's cache (RDKV summary §2.2: every retained unit at its
// allocated width from {0,2,4,8,16}, width 0 evicts; §2.3: rows grouped by width so each
// width has one dequantisation path).  The byte layout is documented in kvc.h.
//
// Kernels, all on one stream (kernel boundaries order every step):
//   pack_count   per (1024-token chunk, head): tokens per width zone; width validation
//   pack_place   per (chunk, head): head totals and offsets (the header, the status word, the
//                K-channel table), the chunk's zone bases, ordered ranks -> v_idx, k_keep,
//                k_vloc
//   pack_k       one wave per (group of 32 retained tokens, head) quantises every K channel
//   pack_v       one block per 32 tokens of one width zone quantises their V groups
// Codes follow the definition z = min, s = float32(float64(max - min) / (2^b - 1)),
// code = clamp(rint(float64(x - z) / s)).  The kernels evaluate v = (x - z) / s in fp32, whose
// error is at most about 3 * 2^-24 * v; only where v lies within 2^(b-21) (over 2.6 times that
// error for every v < 2^b) of a rounding boundary (k + 1/2) can fp32 and fp64 round
// differently, and there the code is recomputed with the fp64 division.  Codes, scales and
// zeros are therefore bit-exact.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kChunk = 1024;      // tokens per index chunk (256 threads x 4)

struct PackWs {
  int32_t* status;     // word 0 of the workspace
  int32_t* cnt;        // [Hkv][nchunk][4]  tokens per zone in each chunk
  int32_t* cbad;       // [Hkv][nchunk]     invalid token widths seen in the chunk
  int32_t* kchc;       // [Hkv][D][4]       per K channel: {word offset, param slot, width, 0}
};

__device__ __forceinline__ int zone_of(uint32_t b) {
  return b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : b == 16 ? 3 : -1;
}

__global__ void __launch_bounds__(256)
pack_count(const uint8_t* __restrict__ bits_v, int64_t N, int nchunk, int32_t* __restrict__ cnt,
           int32_t* __restrict__ cbad) {
  const int ch = blockIdx.x, g = blockIdx.y;
  __shared__ uint64_t part[4];
  __shared__ int32_t badw[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)ch * kChunk + threadIdx.x * 4;
  uint32_t b4 = 0;
  if (t0 + 3 < N && (reinterpret_cast<uintptr_t>(bits_v + (int64_t)g * N + t0) & 3) == 0) {
    b4 = *reinterpret_cast<const uint32_t*>(bits_v + (int64_t)g * N + t0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (t0 + j < N) b4 |= (uint32_t)bits_v[(int64_t)g * N + t0 + j] << (8 * j);
  }
  // the thread's four zone counts as 16-bit fields (a block counts at most 1024 tokens)
  uint64_t mine = 0;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j < N) {
      const uint32_t b = (b4 >> (8 * j)) & 0xFFu;
      bad |= !valid_width(b);
      const int z = zone_of(b);
      if (z >= 0) mine += 1ull << (16 * z);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)mine, o, 64), hi = __shfl_xor((uint32_t)(mine >> 32), o, 64);
    mine += ((uint64_t)hi << 32) | lo;
  }
  const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (lane == 0) {
    part[wid] = mine;
    badw[wid] = wbad ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const uint64_t s = part[0] + part[1] + part[2] + part[3];
    cnt[((int64_t)g * nchunk + ch) * 4 + threadIdx.x] = (int32_t)((s >> (16 * threadIdx.x)) & 0xFFFF);
  }
  if (threadIdx.x == 0) cbad[(int64_t)g * nchunk + ch] = badw[0] | badw[1] | badw[2] | badw[3];
}

// Placement, one block per (1024-token chunk ch, head g).  The chunk's own width bytes are
// loaded first.  One wave per head then rebuilds, in LDS, the zone totals of every head (from
// the chunk counts) and the K words / parameters per group (from bits_k).  Next, three waves
// work side by side: wave 0 sums the sizes of the heads before g (the header offsets of head g;
// for block (0, 0) also the totals), wave 1 the zone counts of the head's earlier chunks (the
// chunk's zone bases), and in blocks (0, g) wave 2 scans head g's channels (its channel table
// and k_width).  Finally the chunk's tokens get their ordered ranks: the four zone counters of a
// thread's 4 tokens are packed into one 64-bit word (16 bits per zone) and scanned.  Block
// (0, g) writes head g's header entries; block (0, 0) the global header and the status word.
// All sums are of integers, so their order does not matter.
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, o, 64), hi = __shfl_xor((uint32_t)(x >> 32), o, 64);
    x += ((uint64_t)hi << 32) | lo;
  }
  return x;
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)x, o, 64), hi = __shfl_up((uint32_t)(x >> 32), o, 64);
    if (lane >= o) x += ((uint64_t)hi << 32) | lo;
  }
  return x;
}

template <int D>
__global__ void __launch_bounds__(256)
pack_place(const uint8_t* __restrict__ bits_v, const uint8_t* __restrict__ bits_k, int64_t N, int Hkv,
           int nchunk, const int32_t* __restrict__ cnt, const int32_t* __restrict__ cbad,
           int64_t* __restrict__ header, int32_t* __restrict__ status, int32_t* __restrict__ kchc,
           uint8_t* __restrict__ k_width, int32_t* __restrict__ v_idx, int32_t* __restrict__ k_keep,
           int32_t* __restrict__ k_vloc) {
  __shared__ int32_t tot[256][4];
  __shared__ int32_t kw_s[256], kq_s[256];
  __shared__ int64_t hv[24];
  __shared__ int64_t bzs[4];
  __shared__ uint64_t sh[4];
  __shared__ int32_t bad_s;
  const int ch = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int gpr = D / 32;

  // the chunk's own tokens: loads that depend on nothing below
  const int64_t t0 = (int64_t)ch * kChunk + tid * 4;
  uint32_t b4 = 0;
  if (t0 + 3 < N && (reinterpret_cast<uintptr_t>(bits_v + (int64_t)g * N + t0) & 3) == 0) {
    b4 = *reinterpret_cast<const uint32_t*>(bits_v + (int64_t)g * N + t0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (t0 + j < N) b4 |= (uint32_t)bits_v[(int64_t)g * N + t0 + j] << (8 * j);
  }
  if (tid == 0) bad_s = 0;
  __syncthreads();

  // per-head totals, one wave per head
  bool bad = false;
  for (int h = wid; h < Hkv; h += 4) {
    uint64_t a = 0, b = 0;
    uint32_t kwv = 0, kqv = 0;
    for (int c2 = lane; c2 < nchunk; c2 += 64) {
      const int4 c = *reinterpret_cast<const int4*>(cnt + ((int64_t)h * nchunk + c2) * 4);
      a += (uint32_t)c.x | ((uint64_t)(uint32_t)c.y << 32);
      b += (uint32_t)c.z | ((uint64_t)(uint32_t)c.w << 32);
      bad |= cbad[(int64_t)h * nchunk + c2] != 0;
    }
    for (int c = lane; c < D; c += 64) {
      const uint32_t bk = bits_k[(int64_t)h * D + c];
      bad |= !valid_width(bk);
      if (zone_of(bk) >= 0) {
        kwv += bk;
        kqv += bk != 16 ? 1u : 0u;
      }
    }
    a = wave_sum_u64(a);
    b = wave_sum_u64(b);
    const uint64_t kk = wave_sum_u64((uint64_t)kwv | ((uint64_t)kqv << 32));
    if (lane == 0) {
      tot[h][0] = (int32_t)(a & 0xFFFFFFFFu);
      tot[h][1] = (int32_t)(a >> 32);
      tot[h][2] = (int32_t)(b & 0xFFFFFFFFu);
      tot[h][3] = (int32_t)(b >> 32);
      kw_s[h] = (int32_t)(kk & 0xFFFFFFFFu);
      kq_s[h] = (int32_t)(kk >> 32);
    }
  }
  if (bad) bad_s = 1;                               // benign race: every writer stores 1
  __syncthreads();

  if (wid == 0) {
    // sizes of heads h < g (head g's offsets), and of all heads (the global header)
    const bool all = ch == 0 && g == 0;
    uint64_t s[5] = {0, 0, 0, 0, 0}, t[5] = {0, 0, 0, 0, 0};
    for (int h = lane; h < Hkv; h += 64) {
      const int64_t n0 = tot[h][0], n1 = tot[h][1], n2 = tot[h][2], n3 = tot[h][3];
      const int64_t R = n0 + n1 + n2 + n3, ng = (R + 31) / 32;
      const uint64_t v[5] = {(uint64_t)R, (uint64_t)((n0 * 2 + n1 * 4 + n2 * 8 + n3 * 16) * gpr),
                             (uint64_t)((n0 + n1 + n2) * gpr), (uint64_t)(ng * kw_s[h]), (uint64_t)(ng * kq_s[h])};
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        if (h < g) s[u] += v[u];
        t[u] += v[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 5; ++u) s[u] = wave_sum_u64(s[u]);
    if (all) {
#pragma unroll
      for (int u = 0; u < 5; ++u) t[u] = wave_sum_u64(t[u]);
    }
    if (lane == 0) {
      const int64_t nv[4] = {tot[g][0], tot[g][1], tot[g][2], tot[g][3]};
      const int64_t R = nv[0] + nv[1] + nv[2] + nv[3];
      int64_t a = (int64_t)s[0], b = (int64_t)s[1], c = (int64_t)s[2];
      for (int z = 0; z < 4; ++z) {
        hv[z] = nv[z];
        hv[5 + z] = a;
        hv[9 + z] = b;
        hv[13 + z] = c;
        a += nv[z];
        b += nv[z] * gpr * (2 << z);
        c += (z < 3) ? nv[z] * gpr : 0;
      }
      hv[4] = R;
      hv[17] = (int64_t)s[0];   // k_keep lists the same R tokens per head, in the same head order
      hv[18] = (int64_t)s[3];
      hv[19] = (int64_t)s[4];
      hv[20] = kw_s[g];
      hv[21] = kq_s[g];
      hv[22] = (R + 31) / 32;
      hv[23] = 0;
      if (all) {
        header[0] = Hkv;
        header[1] = D;
        header[2] = N;
        header[3] = 32;
        header[4] = (int64_t)t[0];
        header[5] = (int64_t)t[1];
        header[6] = (int64_t)t[2];
        header[7] = (int64_t)t[0];
        header[8] = (int64_t)t[3];
        header[9] = (int64_t)t[4];
        for (int i = 10; i < KVC_HDR_GLOBAL; ++i) header[i] = 0;
        *status = bad_s ? KVC_DEV_BAD_WIDTH : 0;
      }
    }
  } else if (wid == 1) {
    // zone bases of this chunk: sums over the head's earlier chunks (32-bit fields)
    uint64_t pa = 0, pb = 0;
    for (int c2 = lane; c2 < ch; c2 += 64) {
      const int4 c = *reinterpret_cast<const int4*>(cnt + ((int64_t)g * nchunk + c2) * 4);
      pa += (uint32_t)c.x | ((uint64_t)(uint32_t)c.y << 32);
      pb += (uint32_t)c.z | ((uint64_t)(uint32_t)c.w << 32);
    }
    pa = wave_sum_u64(pa);
    pb = wave_sum_u64(pb);
    if (lane == 0) {
      bzs[0] = (int64_t)(pa & 0xFFFFFFFFu);
      bzs[1] = (int64_t)(pa >> 32);
      bzs[2] = (int64_t)(pb & 0xFFFFFFFFu);
      bzs[3] = (int64_t)(pb >> 32);
    }
  } else if (wid == 2 && ch == 0) {
    // head g's K channels: word offset and parameter slot inside a group (scan in channel order)
    uint64_t carry = 0;
    for (int c0 = 0; c0 < D; c0 += 64) {
      const int c = c0 + lane;
      const uint32_t bk = bits_k[(int64_t)g * D + c];
      k_width[(int64_t)g * D + c] = (uint8_t)bk;
      const int cls = zone_of(bk);
      const uint64_t f = cls >= 0 ? ((uint64_t)bk | ((uint64_t)(cls < 3) << 16)) : 0;
      const uint64_t inc = wave_incl_scan_u64(f, lane);
      const uint64_t ef = carry + inc - f;
      *reinterpret_cast<int4*>(kchc + ((int64_t)g * D + c) * 4) =
          make_int4((int32_t)(ef & 0xFFFF), (int32_t)((ef >> 16) & 0xFFFF), f ? (int32_t)bk : 0, 0);
      carry += __shfl(inc, 63, 64);
    }
  }
  __syncthreads();
  if (ch == 0 && tid < KVC_HDR_PER_HEAD) header[KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD + tid] = hv[tid];

  // ordered ranks of the chunk's tokens
  int z4[4];
  uint64_t mine = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z4[j] = (t0 + j < N) ? zone_of((b4 >> (8 * j)) & 0xFFu) : -1;
    if (z4[j] >= 0) mine += 1ull << (16 * z4[j]);
  }
  uint64_t total;
  uint64_t run = block_excl_scan<256>(mine, &total, sh);
  const int64_t bz[4] = {bzs[0], bzs[1], bzs[2], bzs[3]};
  const int64_t kbase = hv[17] + bz[0] + bz[1] + bz[2] + bz[3];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int z = z4[j];
    if (z < 0) continue;
    const int64_t rz = (int64_t)((run >> (16 * z)) & 0xFFFF);
    const int64_t rall = (int64_t)((run & 0xFFFF) + ((run >> 16) & 0xFFFF) + ((run >> 32) & 0xFFFF) + ((run >> 48) & 0xFFFF));
    const int64_t pos = bz[z] + rz;
    const int32_t t = (int32_t)(t0 + j);
    v_idx[hv[5 + z] + pos] = t;
    k_keep[kbase + rall] = t;
    k_vloc[kbase + rall] = (int32_t)(((int64_t)z << 29) | pos);
    run += 1ull << (16 * z);
  }
}

// Group quantiser.  min / max use v_min3 / v_max3 (values are finite; fminf would first quiet
// NaNs).  quantize_rt quantises the 32 values of one group a lane holds at width b in {2, 4, 8}
// and stores the group's b code words and its (scale, zero) pair.  Only the first m_own (1..32)
// values are valid; the rest code 0.  b is a runtime value (the K channels of one wave have mixed
// widths) and every lane runs the same instructions: codes are first placed one per byte, then
// the bytes are compacted to b bits.
//  * v = (x - z) * (1 / s) in fp32: 0 <= v < maxc + 2^-16, so rint(v) needs no clamp;
//  * a value whose fp32 v lies within 2^(b-21) of a half-integer (over 2.6 times the error
//    bound 3 * 2^-24 * v for v < 2^b) is decided again with the defining fp64 division,
//    reading the value back through src.fetch().  The codes equal those of that definition.
// quantize_ct is the same quantiser at a compile-time width (the V blocks, whose width is uniform).
// Src provides elem(e) (value e as float), refresh() (makes the held registers opaque, so
// that a later pass unpacks them afresh instead of keeping every unpacked value alive) and
// fetch(e) (value e again for the fp64 decision, from memory or from the lane's registers).
__device__ __forceinline__ float min3_raw(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ uint32_t nibbles_of(uint32_t lo, uint32_t hi) {
  // 8 byte codes < 16 (4 in lo, 4 in hi) -> 8 nibbles, code k in bits 4k .. 4k+3
  const uint32_t a = lo | (lo >> 4), c = hi | (hi >> 4);   // bytes 0 and 2 hold code pairs
  return (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((c & 0xFFu) << 16) | ((c << 8) & 0xFF000000u);
}
__device__ __forceinline__ uint32_t crumbs_of(uint32_t w) {
  // 4 byte codes < 4 -> one byte, code k in bits 2k .. 2k+1
  const uint32_t t = w | (w >> 6);                          // bytes 0 and 2 hold code pairs
  return (t | (t >> 12)) & 0xFFu;
}

// Near-boundary flags of a group, one bit per value in value order: flags = 2 * flags + (|t| > lim),
// one compare and one add-with-carry per value (value e of 32 ends at bit 31 - e).
__device__ __forceinline__ uint32_t shift_in_flag(uint32_t flags, float t, float lim) {
  asm("v_cmp_gt_f32_e64 vcc, |%1|, %2\n\tv_addc_co_u32_e32 %0, vcc, %0, %0, vcc"
      : "+v"(flags) : "v"(t), "v"(lim) : "vcc");
  return flags;
}

// min and max of the first m_own of a lane's 32 values (all 32 when FULL)
template <bool FULL, class Src>
__device__ __forceinline__ void group_min_max(const Src& src, int m_own, float& mn, float& mx) {
  constexpr int NE = 32;
  mn = src.elem(0);
  mx = mn;
#pragma unroll
  for (int e = 1; e < NE - 1; e += 2) {
    const float a = (FULL || e < m_own) ? src.elem(e) : mn;
    const float c = (FULL || e + 1 < m_own) ? src.elem(e + 1) : mn;
    const float a2 = (FULL || e < m_own) ? a : mx;
    const float c2 = (FULL || e + 1 < m_own) ? c : mx;
    mn = min3_raw(mn, a, c);
    mx = max3_raw(mx, a2, c2);
  }
  const float a = (FULL || NE - 1 < m_own) ? src.elem(NE - 1) : mn;
  const float a2 = (FULL || NE - 1 < m_own) ? a : mx;
  mn = min3_raw(mn, a, a);
  mx = max3_raw(mx, a2, a2);
}

template <bool FULL, class Src>
__device__ __forceinline__ void quantize_rt(Src& src, int m_own, int b, uint32_t* __restrict__ dst,
                                            float* __restrict__ par) {
  constexpr int NE = 32;
  float mn, mx;
  group_min_max<FULL>(src, m_own, mn, mx);
  const int maxi = (1 << b) - 1;
  const float s = (float)(((double)mx - (double)mn) / (double)maxi);
  const float lim = 0.5f - __uint_as_float((uint32_t)(b - 21 + 127) << 23);   // 1/2 - 2^(b-21)
  constexpr int NW = NE / 4;                       // byte-code words
  uint32_t w8[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) w8[i] = 0u;
  if (s != 0.f) {
    src.refresh();
    const float rs = 1.0f / s;
    const bool fin = __builtin_isfinite(rs);
    const float rsf = fin ? rs : 0.f;
    uint32_t near = 0u;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float v = (src.elem(e) - mn) * rsf;
      const float r = rintf(v);
      near = shift_in_flag(near, v - r, lim);
      const float code = (FULL || e < m_own) ? r : 0.f;
      w8[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(code, e & 3, w8[e >> 2]);
    }
    if (!fin) near = 0xFFFFFFFFu;                  // an infinite 1/s sends every value to fp64
    if (!FULL) near &= (m_own >= 32) ? 0xFFFFFFFFu : ~(0xFFFFFFFFu >> m_own);   // values e < m_own
    // values near a rounding boundary (rare): decide them with the defining fp64 division
    const double sd = (double)s;
    while (near != 0u) {
      const int e = __builtin_clz(near);
      near &= ~(0x80000000u >> e);
      const double vd = rint(((double)src.fetch(e) - (double)mn) / sd);
      const float code = (float)(vd < 0.0 ? 0.0 : (vd > (double)maxi ? (double)maxi : vd));
#pragma unroll
      for (int i = 0; i < NW; ++i)
        if (i == (e >> 2)) w8[i] = __builtin_amdgcn_cvt_pk_u8_f32(code, e & 3, w8[i]);
    }
  }
  uint32_t o[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) o[i] = w8[i];
  if (b == 4) {
#pragma unroll
    for (int i = 0; i < NW / 2; ++i) o[i] = nibbles_of(w8[2 * i], w8[2 * i + 1]);
  } else if (b == 2) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      o[i] = crumbs_of(w8[4 * i]) | (crumbs_of(w8[4 * i + 1]) << 8) | (crumbs_of(w8[4 * i + 2]) << 16) |
             (crumbs_of(w8[4 * i + 3]) << 24);
  }
  const int nw = (NE * b) >> 5;
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < nw) dst[i] = o[i];
  *reinterpret_cast<float2*>(par) = make_float2(s, mn);
}

// The same quantiser at a width B in {2, 4, 8} fixed at compile time, for a lane's 32 values
// (all valid).  At 2 and 4 bits the codes of a 16-bit half word are gathered as an exact fp32
// sum  sum_j code_j * 2^(B j)  (integers below 2^16, so every fma is exact) and converted once;
// at 8 bits each code goes to its byte directly.
template <int B, class Src>
__device__ __forceinline__ void quantize_ct(Src& src, uint32_t* __restrict__ dst, float* __restrict__ par) {
  constexpr int NE = 32, NW = B;                   // B code words per group
  constexpr int maxi = (1 << B) - 1;
  constexpr int PER = 16 / B;                      // codes per 16-bit half word (B < 8)
  float mn, mx;
  group_min_max<true>(src, NE, mn, mx);
  const float s = (float)(((double)mx - (double)mn) / (double)maxi);
  const float lim = 0.5f - __uint_as_float((uint32_t)(B - 21 + 127) << 23);   // 1/2 - 2^(B-21)
  uint32_t wd[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) wd[i] = 0u;
  if (s != 0.f) {
    src.refresh();
    const float rs = 1.0f / s;
    const bool fin = __builtin_isfinite(rs);
    const float rsf = fin ? rs : 0.f;
    uint32_t near = 0u;
    if constexpr (B == 8) {
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float v = (src.elem(e) - mn) * rsf;
        const float r = rintf(v);
        near = shift_in_flag(near, v - r, lim);
        wd[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(r, e & 3, wd[e >> 2]);
      }
    } else {
      float acc[NE / PER];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float v = (src.elem(e) - mn) * rsf;
        const float r = rintf(v);
        near = shift_in_flag(near, v - r, lim);
        const int a = e / PER, j = e % PER;
        acc[a] = j == 0 ? r : __builtin_fmaf(r, (float)(1u << (B * j)), acc[a]);
      }
#pragma unroll
      for (int i = 0; i < NW; ++i) wd[i] = (uint32_t)acc[2 * i] | ((uint32_t)acc[2 * i + 1] << 16);
    }
    if (!fin) near = 0xFFFFFFFFu;                  // an infinite 1/s sends every value to fp64
    // values near a rounding boundary (rare): decide them with the defining fp64 division
    const double sd = (double)s;
    while (near != 0u) {
      const int e = __builtin_clz(near);
      near &= ~(0x80000000u >> e);
      const double vd = rint(((double)src.fetch(e) - (double)mn) / sd);
      const uint32_t code = (uint32_t)(vd < 0.0 ? 0.0 : (vd > (double)maxi ? (double)maxi : vd));
      const int sh = (e * B) & 31;
#pragma unroll
      for (int i = 0; i < NW; ++i)
        if (i == ((e * B) >> 5)) wd[i] = (wd[i] & ~((uint32_t)maxi << sh)) | (code << sh);
    }
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) dst[i] = wd[i];
  *reinterpret_cast<float2*>(par) = make_float2(s, mn);
}

// A lane's 32 values of one group as 16 packed bf16 pairs (element 2i in the low half of
// w[i]); Fetch reads value e back from memory.
template <class Fetch>
struct PairSrc {
  uint32_t w[16];
  Fetch fetch_fn;
  __device__ __forceinline__ float elem(int e) const {
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
  }
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(w[i]));
  }
  __device__ __forceinline__ float fetch(int e) const { return fetch_fn(e); }
};

// The same 32 values, read back for the fp64 decision from the lane's own registers (a select
// over the 16 words) instead of from memory: a K wave meets several such values per group, and
// a dependent global load for each cost more than the select.
struct RegPairSrc {
  uint32_t w[16];
  __device__ __forceinline__ float elem(int e) const {
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
  }
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(w[i]));
  }
  __device__ __forceinline__ float fetch(int e) const {
    uint32_t x = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) x = (i == (e >> 1)) ? w[i] : x;
    return (e & 1) ? __uint_as_float(x & 0xFFFF0000u) : __uint_as_float(x << 16);
  }
};

// K: one wave per (group j of 32 retained tokens, head g).  Lane l < D/2 holds channels 2l and
// 2l+1, so each load instruction reads one retained token's whole K row (D*2 bytes, coalesced)
// with no staging or transposition; the group's token indices are wave-uniform.
template <int D, bool FULL>
__device__ __forceinline__ void pack_k_group(const uint16_t* __restrict__ k, int64_t N, int g, int64_t j, int m,
                                             const int64_t* __restrict__ hp, const int32_t* __restrict__ kchc,
                                             const int32_t* __restrict__ k_keep, uint32_t* __restrict__ k_words,
                                             float* __restrict__ k_par) {
  const int lane = threadIdx.x & 63;
  const int32_t* tk = k_keep + hp[17] + j * 32;              // wave-uniform
  const uint16_t* kh = k + (int64_t)g * N * D;
  const uint32_t* rows = reinterpret_cast<const uint32_t*>(kh) + lane;
  uint32_t ld[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) ld[i] = (FULL || i < m) ? rows[(int64_t)tk[i] * (D / 2)] : 0u;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = 2 * lane + q;
    const int4 info = *reinterpret_cast<const int4*>(kchc + ((int64_t)g * D + c) * 4);
    const int b = info.z;
    uint32_t* dst = k_words + hp[18] + j * hp[20] + info.x;
    RegPairSrc src{{}};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t lo = ld[2 * i], hi = ld[2 * i + 1];
      src.w[i] = q ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    if (b == 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[i] = src.w[i];
    } else if (b != 0) {
      float* par = k_par + 2 * (hp[19] + j * hp[21] + info.y);
      quantize_rt<FULL>(src, m, b, dst, par);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256)
pack_k(const uint16_t* __restrict__ k, int64_t N, const int64_t* __restrict__ header,
       const int32_t* __restrict__ kchc, const int32_t* __restrict__ k_keep,
       uint32_t* __restrict__ k_words, float* __restrict__ k_par) {
  const int g = blockIdx.y;
  const int64_t* hp = header + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t j = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t R = hp[4];
  if (j * 32 >= R || (threadIdx.x & 63) >= D / 2) return;
  const int m = (int)((R - j * 32) < 32 ? (R - j * 32) : 32);
  if (m == 32) pack_k_group<D, true>(k, N, g, j, 32, hp, kchc, k_keep, k_words, k_par);
  else pack_k_group<D, false>(k, N, g, j, m, hp, kchc, k_keep, k_words, k_par);
}

// V: block (slab x of 32 tokens of one width zone, head g) with D threads = 32 tokens x
// (D / 32) groups; the width is uniform over the block.
template <int D>
__device__ __forceinline__ void pack_v_slab(const uint16_t* __restrict__ v, int64_t N, int g, int64_t x,
                                            const int64_t* __restrict__ hp, const int32_t* __restrict__ v_idx,
                                            uint32_t* __restrict__ v_words, float* __restrict__ v_par) {
  constexpr int GPR = D / 32;
  int z = 0;
  int64_t slab = x;
  for (; z < 4; ++z) {
    const int64_t ns = (hp[z] + 31) / 32;
    if (slab < ns) break;
    slab -= ns;
  }
  if (z == 4) return;
  const int tid = threadIdx.x;
  const int row = tid / GPR, grp = tid % GPR;
  const int64_t pos = slab * 32 + row;
  if (pos >= hp[z]) return;
  const int32_t t = v_idx[hp[5 + z] + pos];
  const uint16_t* vrow = v + ((int64_t)g * N + t) * D + grp * 32;
  auto fetch = [=](int e) { return __uint_as_float((uint32_t)vrow[e] << 16); };
  PairSrc<decltype(fetch)> src{{}, fetch};
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const uint4 wv = *reinterpret_cast<const uint4*>(vrow + q4 * 8);
    src.w[4 * q4 + 0] = wv.x;
    src.w[4 * q4 + 1] = wv.y;
    src.w[4 * q4 + 2] = wv.z;
    src.w[4 * q4 + 3] = wv.w;
  }
  const int b = 2 << z;
  uint32_t* dst = v_words + hp[9 + z] + (pos * GPR + grp) * b;
  if (z == 3) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = src.w[i];
    return;
  }
  float* par = v_par + 2 * (hp[13 + z] + pos * GPR + grp);
  if (z == 0) quantize_ct<2>(src, dst, par);       // the width is uniform over the block
  else if (z == 1) quantize_ct<4>(src, dst, par);
  else quantize_ct<8>(src, dst, par);
}

template <int D>
__global__ void __launch_bounds__(D)
pack_v(const uint16_t* __restrict__ v, int64_t N, const int64_t* __restrict__ header,
       const int32_t* __restrict__ v_idx, uint32_t* __restrict__ v_words, float* __restrict__ v_par) {
  const int g = blockIdx.y;
  const int64_t* hp = header + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  pack_v_slab<D>(v, N, g, blockIdx.x, hp, v_idx, v_words, v_par);
}

PackWs carve(const Layer& L, char* ws, size_t* total) {
  const int nchunk = (int)((L.n + kChunk - 1) / kChunk);
  WsPlan p;
  size_t oc = p.take(sizeof(int32_t) * L.hkv * nchunk * 4);
  size_t obad = p.take(sizeof(int32_t) * L.hkv * nchunk);
  size_t okc = p.take(sizeof(int32_t) * L.hkv * L.d * 4);
  if (total) *total = p.off;
  PackWs w{};
  if (ws) {
    w.status = reinterpret_cast<int32_t*>(ws);
    w.cnt = reinterpret_cast<int32_t*>(ws + oc);
    w.cbad = reinterpret_cast<int32_t*>(ws + obad);
    w.kchc = reinterpret_cast<int32_t*>(ws + okc);
  }
  return w;
}

}  // namespace

void packed_capacity(const Layer& L, size_t bytes[KVC_PK_NBUF]) {
  const int64_t T = (int64_t)L.hkv * L.n;               // tokens
  const int64_t gpr = L.d / 32;
  const int64_t ng = (int64_t)L.hkv * ((L.n + 31) / 32);  // K groups (upper bound)
  bytes[KVC_PK_HEADER] = sizeof(int64_t) * (KVC_HDR_GLOBAL + L.hkv * KVC_HDR_PER_HEAD);
  bytes[KVC_PK_V_IDX] = sizeof(int32_t) * T;
  bytes[KVC_PK_V_WORDS] = sizeof(uint32_t) * T * gpr * 16;
  bytes[KVC_PK_V_PAR] = sizeof(float) * 2 * T * gpr;
  bytes[KVC_PK_K_KEEP] = sizeof(int32_t) * T;
  bytes[KVC_PK_K_VLOC] = sizeof(int32_t) * T;
  bytes[KVC_PK_K_WORDS] = sizeof(uint32_t) * ng * 16 * L.d;
  bytes[KVC_PK_K_PAR] = sizeof(float) * 2 * ng * L.d;
  bytes[KVC_PK_K_WIDTH] = (size_t)L.hkv * L.d;
}

size_t pack_ws_bytes(const Layer& L) {
  size_t total = 0;
  carve(L, nullptr, &total);
  return total;
}

hipError_t launch_pack(const Layer& L, const uint16_t* k, const uint16_t* v,
                       const uint8_t* bits_v, const uint8_t* bits_k,
                       const kvc_packed_cache& out, char* ws, hipStream_t s) {
  const int nchunk = (int)((L.n + kChunk - 1) / kChunk);
  PackWs w = carve(L, ws, nullptr);
  dim3 gc((unsigned)nchunk, (unsigned)L.hkv);
  pack_count<<<gc, 256, 0, s>>>(bits_v, L.n, nchunk, w.cnt, w.cbad);
  if (L.d == 128)
    pack_place<128><<<gc, 256, 0, s>>>(bits_v, bits_k, L.n, L.hkv, nchunk, w.cnt, w.cbad, out.header,
                                       w.status, w.kchc, out.k_width, out.v_idx, out.k_keep, out.k_vloc);
  else
    pack_place<64><<<gc, 256, 0, s>>>(bits_v, bits_k, L.n, L.hkv, nchunk, w.cnt, w.cbad, out.header,
                                      w.status, w.kchc, out.k_width, out.v_idx, out.k_keep, out.k_vloc);
  dim3 gv((unsigned)((L.n + 31) / 32 + 4), (unsigned)L.hkv);
  dim3 gk2((unsigned)(((L.n + 31) / 32 + 3) / 4), (unsigned)L.hkv);
  if (L.d == 128) {
    pack_k<128><<<gk2, 256, 0, s>>>(k, L.n, out.header, w.kchc, out.k_keep, out.k_words, out.k_par);
    pack_v<128><<<gv, 128, 0, s>>>(v, L.n, out.header, out.v_idx, out.v_words, out.v_par);
  } else {
    pack_k<64><<<gk2, 256, 0, s>>>(k, L.n, out.header, w.kchc, out.k_keep, out.k_words, out.k_par);
    pack_v<64><<<gv, 64, 0, s>>>(v, L.n, out.header, out.v_idx, out.v_words, out.v_par);
  }
  return hipGetLastError();
}

}  // namespace kvc
