// Mixed-width quantise/pack of one layer's cache (RDKV summary §2.2: every retained unit at its
// allocated width from {0,2,4,8,16}, width 0 evicts; §2.3: rows grouped by width so each
// width has one dequantisation path).  The byte layout is documented in kvc.h.
//
// Kernels, all on one stream:
//   pack_count   per (1024-token chunk, head): tokens per width zone; width validation
//   pack_layout  one block: per-chunk zone bases, the header, the k_width copy
//   pack_index   per chunk: ordered ranks -> v_idx, k_keep, k_vloc
//   pack_kv      one block per (32 retained tokens, head): quantise every K channel and
//                every V group of those tokens
// The quantiser does its division in float64 exactly as the definition reads
// (z = min, s = float32(float64(max - min) / (2^b - 1)), code = rint(float64(x - z) / s)), so
// codes, scales and zeros are bit-exact against a float64 reference.
#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kChunk = 1024;      // tokens per index chunk (256 threads x 4)

struct PackWs {
  int32_t* status;
  int32_t* cnt;        // [Hkv][nchunk][4]  tokens per zone in each chunk
  int64_t* base;       // [Hkv][nchunk][4]  zone position of each chunk's first token
  int64_t* rbase;      // [Hkv][nchunk]     retained index of each chunk's first token
};

__device__ __forceinline__ int zone_of(uint32_t b) {
  return b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : b == 16 ? 3 : -1;
}

__global__ void __launch_bounds__(256)
pack_count(const uint8_t* __restrict__ bits_v, const uint8_t* __restrict__ bits_k, int64_t N,
           int d, int nchunk, int32_t* __restrict__ cnt, int32_t* status) {
  const int ch = blockIdx.x, g = blockIdx.y;
  __shared__ int32_t c4[4];
  if (threadIdx.x < 4) c4[threadIdx.x] = 0;
  __syncthreads();
  int my[4] = {0, 0, 0, 0};
  bool bad = false;
  const int64_t t0 = (int64_t)ch * kChunk;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t t = t0 + threadIdx.x * 4 + j;
    if (t < N) {
      uint32_t b = bits_v[(int64_t)g * N + t];
      bad |= !valid_width(b);
      int z = zone_of(b);
      if (z >= 0) my[z]++;
    }
  }
  if (ch == 0 && (int)threadIdx.x < d) bad |= !valid_width(bits_k[(int64_t)g * d + threadIdx.x]);
  if (bad) set_status(status, KVC_DEV_BAD_WIDTH);
#pragma unroll
  for (int z = 0; z < 4; ++z)
    if (my[z]) atomicAdd(&c4[z], my[z]);     // integer: order-independent
  __syncthreads();
  if (threadIdx.x < 4) cnt[((int64_t)g * nchunk + ch) * 4 + threadIdx.x] = c4[threadIdx.x];
}

// Header and per-chunk bases.  One block: threads (g, z) scan their chunks, the K-channel
// widths are summed per head in parallel, then thread 0 lays the heads out in order.
__global__ void __launch_bounds__(1024)
pack_layout(const int32_t* __restrict__ cnt, const uint8_t* __restrict__ bits_k, int Hkv, int d,
            int64_t N, int nchunk, int64_t* __restrict__ base, int64_t* __restrict__ rbase,
            int64_t* __restrict__ header, uint8_t* __restrict__ k_width) {
  __shared__ int64_t tot[1024];      // tokens per (g, z)
  __shared__ int32_t wk_s[256], qk_s[256];
  const int tid = threadIdx.x;
  for (int g = tid; g < Hkv; g += blockDim.x) {
    wk_s[g] = 0;
    qk_s[g] = 0;
  }
  for (int gz = tid; gz < Hkv * 4; gz += blockDim.x) {
    const int g = gz / 4, z = gz % 4;
    int64_t run = 0;
    for (int ch = 0; ch < nchunk; ++ch) {
      base[((int64_t)g * nchunk + ch) * 4 + z] = run;
      run += cnt[((int64_t)g * nchunk + ch) * 4 + z];
    }
    tot[gz] = run;
  }
  for (int g = tid; g < Hkv; g += blockDim.x) {
    int64_t run = 0;
    for (int ch = 0; ch < nchunk; ++ch) {
      rbase[(int64_t)g * nchunk + ch] = run;
      const int32_t* cc = cnt + ((int64_t)g * nchunk + ch) * 4;
      run += (int64_t)cc[0] + cc[1] + cc[2] + cc[3];
    }
  }
  __syncthreads();
  for (int e = tid; e < Hkv * d; e += blockDim.x) {
    const uint32_t b = bits_k[e];
    k_width[e] = (uint8_t)b;
    if (valid_width(b) && b) atomicAdd(&wk_s[e / d], (int32_t)b);   // integer sums: order-free
    if (b == 2 || b == 4 || b == 8) atomicAdd(&qk_s[e / d], 1);
  }
  for (int i = tid; i < KVC_HDR_GLOBAL + Hkv * KVC_HDR_PER_HEAD; i += blockDim.x) header[i] = 0;
  __syncthreads();
  if (tid == 0) {
    const int gpr = d / 32;
    const int widths[4] = {2, 4, 8, 16};
    int64_t o_vi = 0, o_vw = 0, o_vp = 0, o_kk = 0, o_kw = 0, o_kp = 0;
    header[0] = Hkv;
    header[1] = d;
    header[2] = N;
    header[3] = 32;
    for (int g = 0; g < Hkv; ++g) {
      int64_t* hp = header + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
      int64_t R = 0;
      for (int z = 0; z < 4; ++z) {
        const int64_t nv = tot[g * 4 + z];
        hp[z] = nv;
        hp[5 + z] = o_vi;
        hp[9 + z] = o_vw;
        hp[13 + z] = o_vp;
        o_vi += nv;
        o_vw += nv * gpr * widths[z];
        o_vp += (z < 3) ? nv * gpr : 0;
        R += nv;
      }
      const int64_t wk = wk_s[g], qk = qk_s[g];
      const int64_t ng = (R + 31) / 32;
      hp[4] = R;
      hp[17] = o_kk;
      hp[18] = o_kw;
      hp[19] = o_kp;
      hp[20] = wk;
      hp[21] = qk;
      hp[22] = ng;
      o_kk += R;
      o_kw += ng * wk;
      o_kp += ng * qk;
    }
    header[4] = o_vi;
    header[5] = o_vw;
    header[6] = o_vp;
    header[7] = o_kk;
    header[8] = o_kw;
    header[9] = o_kp;
  }
}

// Ordered ranks inside each chunk: the four zone counters of a thread's 4 tokens are packed
// into one 64-bit word (16 bits per zone; a chunk holds at most 1024 tokens) and scanned.
__global__ void __launch_bounds__(256)
pack_index(const uint8_t* __restrict__ bits_v, int64_t N, int nchunk,
           const int64_t* __restrict__ base, const int64_t* __restrict__ rbase,
           const int64_t* __restrict__ header, int32_t* __restrict__ v_idx,
           int32_t* __restrict__ k_keep, int32_t* __restrict__ k_vloc) {
  const int ch = blockIdx.x, g = blockIdx.y;
  const int64_t t0 = (int64_t)ch * kChunk + threadIdx.x * 4;
  int z4[4];
  uint64_t mine = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t t = t0 + j;
    z4[j] = (t < N) ? zone_of(bits_v[(int64_t)g * N + t]) : -1;
    if (z4[j] >= 0) mine += 1ull << (16 * z4[j]);
  }
  __shared__ uint64_t sc[256];
  const int i = threadIdx.x;
  sc[i] = mine;
  __syncthreads();
  for (int w = 1; w < 256; w <<= 1) {
    uint64_t add = (i >= w) ? sc[i - w] : 0;
    __syncthreads();
    sc[i] += add;
    __syncthreads();
  }
  uint64_t run = sc[i] - mine;        // exclusive
  const int64_t* hp = header + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t* bz = base + ((int64_t)g * nchunk + ch) * 4;
  const int64_t kbase = hp[17] + rbase[(int64_t)g * nchunk + ch];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int z = z4[j];
    if (z < 0) continue;
    const int64_t rz = (int64_t)((run >> (16 * z)) & 0xFFFF);
    const int64_t rall = (int64_t)((run & 0xFFFF) + ((run >> 16) & 0xFFFF) + ((run >> 32) & 0xFFFF) + ((run >> 48) & 0xFFFF));
    const int64_t pos = bz[z] + rz;
    const int32_t t = (int32_t)(t0 + j);
    v_idx[hp[5 + z] + pos] = t;
    k_keep[kbase + rall] = t;
    k_vloc[kbase + rall] = (int32_t)(((int64_t)z << 29) | pos);
    run += 1ull << (16 * z);
  }
}

// Quantise one group held as 32 float32 bf16 values (m of them valid) at width b in {2,4,8}.
__device__ __forceinline__ void quantize32(const float (&x)[32], int m, int b, uint32_t (&w)[8],
                                           float* s_out, float* z_out) {
  float mn = x[0], mx = x[0];
  for (int e = 1; e < m; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
  const double range = (double)mx - (double)mn;
  const float s = (float)(range / (double)((1 << b) - 1));
  const double sd = (double)s;
  const double maxc = (double)((1 << b) - 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 0u;
  const int per = 32 / b;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    uint32_t code = 0;
    if (e < m && s != 0.f) {
      double v = ((double)x[e] - (double)mn) / sd;
      double r = rint(v);
      r = r < 0.0 ? 0.0 : (r > maxc ? maxc : r);
      code = (uint32_t)r;
    }
    w[e / per] |= code << ((e % per) * b);
  }
  *s_out = s;
  *z_out = mn;
}

// One block per (group of 32 retained tokens j, head g), 2*D threads: thread c < D quantises
// K channel c over the 32 tokens (group-major words), thread D + i quantises V group
// i % (D/32) of token i / (D/32).  Every thread handles one 32-element group.
template <int D>
__global__ void __launch_bounds__(2 * D)
pack_kv(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t N,
        const int64_t* __restrict__ header, const uint8_t* __restrict__ bits_k,
        const int32_t* __restrict__ k_keep, const int32_t* __restrict__ k_vloc,
        uint32_t* __restrict__ k_words, float* __restrict__ k_par, uint32_t* __restrict__ v_words,
        float* __restrict__ v_par) {
  constexpr int GPR = D / 32;
  const int g = blockIdx.y;
  const int64_t jg = blockIdx.x;
  const int64_t* hp = header + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t R = hp[4];
  if (jg * 32 >= R) return;
  const int m = (int)((R - jg * 32) < 32 ? (R - jg * 32) : 32);
  __shared__ uint16_t tile[32][D + 2];
  __shared__ int32_t woff[D], qslot[D], tok[32], vloc[32];
  const int tid = threadIdx.x;
  if (tid < 32) {
    tok[tid] = tid < m ? k_keep[hp[17] + jg * 32 + tid] : 0;
    vloc[tid] = tid < m ? k_vloc[hp[17] + jg * 32 + tid] : 0;
  }
  if (tid == 32) {
    int32_t wo = 0, qs = 0;
    for (int c = 0; c < D; ++c) {
      const int b = bits_k[(int64_t)g * D + c];
      woff[c] = wo;
      qslot[c] = qs;
      wo += valid_width(b) ? b : 0;
      qs += (b == 2 || b == 4 || b == 8);
    }
  }
  __syncthreads();
  // stage the retained K rows (16-byte loads)
  for (int e = tid; e < 32 * (D / 8); e += 2 * D) {
    const int r = e / (D / 8), c8 = e % (D / 8);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < m) val = *reinterpret_cast<const uint4*>(k + ((int64_t)g * N + tok[r]) * D + c8 * 8);
    const uint32_t vv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[r][c8 * 8 + 2 * i] = (uint16_t)(vv[i] & 0xFFFFu);
      tile[r][c8 * 8 + 2 * i + 1] = (uint16_t)(vv[i] >> 16);
    }
  }
  __syncthreads();
  float x[32];
  uint32_t w[8];
  float sc, zz;
  if (tid < D) {
    const int c = tid;
    const int b = bits_k[(int64_t)g * D + c];
    if (b == 0 || !valid_width(b)) return;
    uint32_t* dst = k_words + hp[18] + jg * hp[20] + woff[c];
    if (b == 16) {
      for (int i = 0; i < 16; ++i) {
        const uint32_t lo16 = (2 * i < m) ? tile[2 * i][c] : 0u;
        const uint32_t hi16 = (2 * i + 1 < m) ? tile[2 * i + 1][c] : 0u;
        dst[i] = lo16 | (hi16 << 16);
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = bf16_bits_to_f32(tile[e][c]);
    quantize32(x, m, b, w, &sc, &zz);
    for (int i = 0; i < b; ++i) dst[i] = w[i];
    float* par = k_par + 2 * (hp[19] + jg * hp[21] + qslot[c]);
    par[0] = sc;
    par[1] = zz;
    return;
  }
  const int task = tid - D;
  const int e = task / GPR, grp = task % GPR;
  if (task >= 32 * GPR || e >= m) return;
  const int32_t loc = vloc[e];
  const int z = loc >> 29;
  const int64_t pos = loc & ((1 << 29) - 1);
  const int b = 2 << z;    // 2,4,8,16
  const uint16_t* src = v + ((int64_t)g * N + tok[e]) * D + grp * 32;
  uint32_t raw[16];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const uint4 wv = *reinterpret_cast<const uint4*>(src + q4 * 8);
    raw[4 * q4 + 0] = wv.x;
    raw[4 * q4 + 1] = wv.y;
    raw[4 * q4 + 2] = wv.z;
    raw[4 * q4 + 3] = wv.w;
  }
  uint32_t* dst = v_words + hp[9 + z] + (pos * GPR + grp) * b;
  if (b == 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = raw[i];
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[2 * i] = bf16_bits_to_f32(raw[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
  }
  quantize32(x, 32, b, w, &sc, &zz);
  for (int i = 0; i < b; ++i) dst[i] = w[i];
  float* par = v_par + 2 * (hp[13 + z] + pos * GPR + grp);
  par[0] = sc;
  par[1] = zz;
}

PackWs carve(const Layer& L, char* ws, size_t* total) {
  const int nchunk = (int)((L.n + kChunk - 1) / kChunk);
  WsPlan p;
  size_t oc = p.take(sizeof(int32_t) * L.hkv * nchunk * 4);
  size_t ob = p.take(sizeof(int64_t) * L.hkv * nchunk * 4);
  size_t orb = p.take(sizeof(int64_t) * L.hkv * nchunk);
  if (total) *total = p.off;
  PackWs w{};
  if (ws) {
    w.status = reinterpret_cast<int32_t*>(ws);
    w.cnt = reinterpret_cast<int32_t*>(ws + oc);
    w.base = reinterpret_cast<int64_t*>(ws + ob);
    w.rbase = reinterpret_cast<int64_t*>(ws + orb);
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
  (void)launch_reset_status(ws, s);
  dim3 gc((unsigned)nchunk, (unsigned)L.hkv);
  pack_count<<<gc, 256, 0, s>>>(bits_v, bits_k, L.n, L.d, nchunk, w.cnt, w.status);
  pack_layout<<<1, 1024, 0, s>>>(w.cnt, bits_k, L.hkv, L.d, L.n, nchunk, w.base, w.rbase,
                                 out.header, out.k_width);
  pack_index<<<gc, 256, 0, s>>>(bits_v, L.n, nchunk, w.base, w.rbase, out.header, out.v_idx,
                                out.k_keep, out.k_vloc);
  dim3 gk((unsigned)((L.n + 31) / 32), (unsigned)L.hkv);
  if (L.d == 128)
    pack_kv<128><<<gk, 256, 0, s>>>(k, v, L.n, out.header, bits_k, out.k_keep, out.k_vloc,
                                    out.k_words, out.k_par, out.v_words, out.v_par);
  else
    pack_kv<64><<<gk, 128, 0, s>>>(k, v, L.n, out.header, bits_k, out.k_keep, out.k_vloc,
                                   out.k_words, out.k_par, out.v_words, out.v_par);
  return hipGetLastError();
}

}  // namespace kvc
