// Attention of a few query rows (G * Nq <= 16 per KV head, e.g. one new token per query head)
// straight from the packed zones, on the matrix cores (RDKV summary §2.3: decode reads the
// packed cache, dequantisation fused into attention; KVSculpt summary §2: the output and LSE
// whose errors form the loss).  Two streaming kernels:
//
//  attend_dec_logits: the K groups (32 retained tokens each) of a KV head, dealt to the waves of
//  the head's blocks.  With R the padded row count (1, 2, 4, 8 or 16), the 16 "columns" n of a
//  16x16x32 bf16 product hold row n % R (the rows are repeated), and per 16-token half
//      S^T = codes x (q * scale)_hi + codes x (q * scale)_lo + zero x q
//  over the head's nonzero K channels, since q . k_hat = sum_c q_c zero_c + sum_c (q_c scale_c) code_c
//  for a quantised channel and q . k for a raw one (code = the raw bf16, scale 1, zero 0).  A
//  32-position block's B operands serve both halves, and its zero term (the same for every token)
//  is one product.  Codes
//  and raw bf16 are exact bf16 operands, q * scale enters as a bf16 hi + lo pair (to 2^-17), q and
//  the zeros (minima of bf16 values) are exact: the logits carry only the float32 accumulation
//  error.  The channels are ordered by width ("positions"), each width class padded to a multiple
//  of 8, so the 8 positions a lane feeds share one width.  A group's code words are copied into LDS
//  word-major within each class ([class][word][position]): a lane reads its 8 positions' words with
//  two 16-byte loads, gathers the byte holding its token's code from each with byte permutes,
//  shifts and masks; 2-bit and 4-bit codes become bf16 through the fp8 (e4m3) conversion, whose
//  bytes 0..15 encode n * 2^-9 exactly (scale 2^9), 8-bit codes convert per byte.  The masked
//  logits are stored in V-zone row order (the token's place in its V zone), with each block's
//  maximum per row.
//
//  attend_dec_values: a zone lists the tokens of one width in token order, so its rows, their
//  logits and (scale, zero) pairs are contiguous; the head's zone rows are cut into chunks of up to
//  32 rows of one width and dealt to the waves.  With M the head's maximum per row (over the logits
//  blocks), p = 2^(S c - M) and
//      O^T[channel][n] += V codes^T x (p * scale_v)_hi,lo,  O_zero[n] += sum_t p_t zero_v,
//  the value scale folded into the probability operand and column n taking channel group n / R
//  (16 / R groups per pass, more passes when that is below the number of groups).  Each block
//  writes (M, l, O) per row as one split; attend_merge combines the splits.
//
// Both kernels copy their data straight into per-wave LDS rings (global -> LDS loads) one or more
// groups or chunks ahead and wait for exactly the copies they need; no block barrier runs in the
// streaming loops.  Both run four waves per SIMD (at most 128 registers; rings sized so that four
// blocks share a compute unit's LDS): more waves in flight hide the copies and the LDS reads better
// than deeper rings at three waves.
#include <utility>

#include "common.hpp"
#include "internal.hpp"

namespace kvc {

namespace {

constexpr int kDcWaves = 4;
constexpr int kDcThreads = 64 * kDcWaves;
constexpr int kPPMax = 160;            // padded K positions: D <= 128 channels + up to 7 per class
constexpr int kKBMax = kPPMax / 32;    // 32-position blocks
constexpr int kKSt = 2304;             // >= staged K words of a group (sum_c b_c * padded count)
constexpr int kKRing = 1344;           // K ring words per wave (group slots: words, pairs, tokens)
constexpr int kKMaxSlots = 8;
constexpr int kVSlotWords = 792;       // V chunk words and pairs: 12 blocks of 64 words, 2 apart
constexpr int kVSlots = 2;             // V ring slots per wave

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Every earlier LDS access of the wave has completed; no memory access moves across.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}
// Every earlier global load of the wave, the copies into LDS included, has landed.
__device__ __forceinline__ void wave_vm_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Until at most n (wave-uniform, 0..63) of the wave's global loads are outstanding: loads complete
// in issue order, so everything issued before the last n has landed.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
    case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 33: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
    case 34: asm volatile("s_waitcnt vmcnt(34)" ::: "memory"); break;
    case 35: asm volatile("s_waitcnt vmcnt(35)" ::: "memory"); break;
    case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
    case 37: asm volatile("s_waitcnt vmcnt(37)" ::: "memory"); break;
    case 38: asm volatile("s_waitcnt vmcnt(38)" ::: "memory"); break;
    case 39: asm volatile("s_waitcnt vmcnt(39)" ::: "memory"); break;
    case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 41: asm volatile("s_waitcnt vmcnt(41)" ::: "memory"); break;
    case 42: asm volatile("s_waitcnt vmcnt(42)" ::: "memory"); break;
    case 43: asm volatile("s_waitcnt vmcnt(43)" ::: "memory"); break;
    case 44: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
    case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
    case 46: asm volatile("s_waitcnt vmcnt(46)" ::: "memory"); break;
    case 47: asm volatile("s_waitcnt vmcnt(47)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    case 49: asm volatile("s_waitcnt vmcnt(49)" ::: "memory"); break;
    case 50: asm volatile("s_waitcnt vmcnt(50)" ::: "memory"); break;
    case 51: asm volatile("s_waitcnt vmcnt(51)" ::: "memory"); break;
    case 52: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
    case 53: asm volatile("s_waitcnt vmcnt(53)" ::: "memory"); break;
    case 54: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
    case 55: asm volatile("s_waitcnt vmcnt(55)" ::: "memory"); break;
    case 56: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
    case 57: asm volatile("s_waitcnt vmcnt(57)" ::: "memory"); break;
    case 58: asm volatile("s_waitcnt vmcnt(58)" ::: "memory"); break;
    case 59: asm volatile("s_waitcnt vmcnt(59)" ::: "memory"); break;
    case 60: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
    case 61: asm volatile("s_waitcnt vmcnt(61)" ::: "memory"); break;
    case 62: asm volatile("s_waitcnt vmcnt(62)" ::: "memory"); break;
    case 63: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
  __builtin_amdgcn_wave_barrier();
}

// One dword per lane from `src` into LDS at dst + 4 * lane (dst wave-uniform).
__device__ __forceinline__ void stage_dword(const void* src, lds_u32* dst) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Bytes 2k, 2k + 1 of x (values 0..15) as the bf16 pair of the integers they hold: the e4m3
// byte n < 16 encodes n * 2^-9 (subnormal for n < 8, exponent 1 above), scaled back by 2^9.
template <bool HI>
__device__ __forceinline__ uint32_t nib_bf16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 512.0f, HI));
}
// Bytes 2k, 2k + 1 of x (values 0..255) as a bf16 pair (exact: at most 8 significant bits).
__device__ __forceinline__ uint32_t byte_bf16x2(uint32_t x, int k) {
  const float a = (float)((x >> (16 * k)) & 0xFFu), b = (float)((x >> (16 * k + 8)) & 0xFFu);
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight elements from 8 words (element i in w[i], at byte (sel_a & 3), bit `bit`), in element
// order as bf16: path 1: 2-bit / 4-bit codes (`mask` wide); path 2: 8-bit codes; path 3: raw
// bf16 (sel_a picks the half of each word).
template <int PATH>
__device__ __forceinline__ uint4 codes8(uint4 w0, uint4 w1, uint32_t sel_a, int bit, uint32_t mask) {
  if (PATH == 3)
    return make_uint4(perm(w0.y, w0.x, sel_a), perm(w0.w, w0.z, sel_a), perm(w1.y, w1.x, sel_a),
                      perm(w1.w, w1.z, sel_a));
  const uint32_t sel_b = __builtin_amdgcn_alignbit(sel_a, sel_a, 16);
  const uint32_t x0 = perm(w0.y, w0.x, sel_a) | perm(w0.w, w0.z, sel_b);
  const uint32_t x1 = perm(w1.y, w1.x, sel_a) | perm(w1.w, w1.z, sel_b);
  if (PATH == 2) return make_uint4(byte_bf16x2(x0, 0), byte_bf16x2(x0, 1), byte_bf16x2(x1, 0), byte_bf16x2(x1, 1));
  const uint32_t y0 = (x0 >> bit) & mask, y1 = (x1 >> bit) & mask;
  return make_uint4(nib_bf16x2<false>(y0), nib_bf16x2<true>(y0), nib_bf16x2<false>(y1), nib_bf16x2<true>(y1));
}

// A lane's 8 bf16 A-operand codes of one 32-position block (descriptor dA: path, bit, byte, 2-bit
// flag, real positions of a raw run); zero for a block past the positions.
__device__ __forceinline__ uint4 kcodes(uint32_t dA, uint4 w0, uint4 w1) {
  const int path = (int)((dA >> 12) & 3);
  uint4 a = make_uint4(0u, 0u, 0u, 0u);
  if (path != 0) {
    const int bit = (int)((dA >> 16) & 7);
    const uint32_t byte = (dA >> 20) & 3;
    const uint32_t sel = path == 3 ? (byte ? 0x07060302u : 0x05040100u) : 0x0C0C0400u + byte * 0x101u;
    const uint32_t mask = (dA >> 22) & 1 ? 0x03030303u : 0x0F0F0F0Fu;
    if (path == 1) a = codes8<1>(w0, w1, sel, bit, mask);
    else if (path == 2) a = codes8<2>(w0, w1, sel, bit, mask);
    else {
      a = codes8<3>(w0, w1, sel, bit, mask);
      const int nval = (int)((dA >> 24) & 15);   // raw class padding holds copies: zero it
      uint32_t aa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        aa[i] &= (2 * i < nval ? 0x0000FFFFu : 0u) | (2 * i + 1 < nval ? 0xFFFF0000u : 0u);
      a = make_uint4(aa[0], aa[1], aa[2], aa[3]);
    }
  }
  return a;
}

// bf16 hi / lo words of 8 values (element order), lo = bf16(x - hi).
__device__ __forceinline__ void hilo8(const float (&x)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 hv = {(__bf16)x[2 * i], (__bf16)x[2 * i + 1]};
    const uint32_t hb = __builtin_bit_cast(uint32_t, hv);
    const float r0 = x[2 * i] - __uint_as_float(hb << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(hb & 0xFFFF0000u);
    const bf16x2 lv = {(__bf16)r0, (__bf16)r1};
    h[i] = hb;
    l[i] = __builtin_bit_cast(uint32_t, lv);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Reads of the copy buffers.  The compiler would wait for every copy in flight before any read of
// the array they fill, so these reads are written out (each asm statement waits for its own data
// before it ends) and the copies are waited for explicitly (wait_vm).  addr: LDS byte address.
// The operands of one 32-position block for both token halves: two 16-byte reads each at aw0 and
// aw1 (the halves' code words) and one each at ah, al, az, aq (q * scale hi, lo, zeros, q).
__device__ __forceinline__ void lds_rd_kblock(uint32_t aw0, uint32_t aw1, uint32_t ah, uint32_t al, uint32_t az,
                                               uint32_t aq, uint4& w00, uint4& w01, uint4& w10, uint4& w11,
                                               uint4& bh, uint4& bl, uint4& bz, uint4& bq) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 x0, x1, x2, x3, x4, x5, x6, x7;
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\tds_read_b128 %2, %9\n\t"
      "ds_read_b128 %3, %9 offset:16\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\t"
      "ds_read_b128 %6, %12\n\tds_read_b128 %7, %13\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4), "=&v"(x5), "=&v"(x6), "=&v"(x7)
      : "v"(aw0), "v"(aw1), "v"(ah), "v"(al), "v"(az), "v"(aq));
  w00 = make_uint4(x0[0], x0[1], x0[2], x0[3]);
  w01 = make_uint4(x1[0], x1[1], x1[2], x1[3]);
  w10 = make_uint4(x2[0], x2[1], x2[2], x2[3]);
  w11 = make_uint4(x3[0], x3[1], x3[2], x3[3]);
  bh = make_uint4(x4[0], x4[1], x4[2], x4[3]);
  bl = make_uint4(x5[0], x5[1], x5[2], x5[3]);
  bz = make_uint4(x6[0], x6[1], x6[2], x6[3]);
  bq = make_uint4(x7[0], x7[1], x7[2], x7[3]);
}
__device__ __forceinline__ uint64_t lds_rd_64(uint32_t addr) {
  uint64_t x;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(addr));
  return x;
}
// Eight dwords at addr + O0 .. addr + O7 (bytes, compile-time).
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_rd_8x32(uint32_t addr, uint32_t (&w)[8]) {
  asm volatile(
      "ds_read_b32 %0, %8 offset:%9\n\tds_read_b32 %1, %8 offset:%10\n\t"
      "ds_read_b32 %2, %8 offset:%11\n\tds_read_b32 %3, %8 offset:%12\n\t"
      "ds_read_b32 %4, %8 offset:%13\n\tds_read_b32 %5, %8 offset:%14\n\t"
      "ds_read_b32 %6, %8 offset:%15\n\tds_read_b32 %7, %8 offset:%16\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7])
      : "v"(addr), "i"(O0), "i"(O1), "i"(O2), "i"(O3), "i"(O4), "i"(O5), "i"(O6), "i"(O7));
}
// Eight 64-bit values at addr + k * S (bytes, S compile-time).
template <int S>
__device__ __forceinline__ void lds_rd_8x64(uint32_t addr, uint64_t (&w)[8]) {
  asm volatile(
      "ds_read_b64 %0, %8\n\tds_read_b64 %1, %8 offset:%9\n\t"
      "ds_read_b64 %2, %8 offset:%10\n\tds_read_b64 %3, %8 offset:%11\n\t"
      "ds_read_b64 %4, %8 offset:%12\n\tds_read_b64 %5, %8 offset:%13\n\t"
      "ds_read_b64 %6, %8 offset:%14\n\tds_read_b64 %7, %8 offset:%15\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7])
      : "v"(addr), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S), "i"(7 * S));
}

template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {   // the LDS byte address of a shared variable
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

template <int... I, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// Staged V words sit in blocks of 64, 66 words apart (copy i of a chunk fills block i).
__host__ __device__ constexpr int vpad(int u) { return (u >> 6) * 66 + (u & 63); }

// The words of rows 0..7 of two consecutive value tiles (tile CT and CT + 1, HB words per tile per
// row, RW words per row, padded every 64 words), one wait.
template <int RW, int CT, int HB>
__device__ __forceinline__ void lds_rd_tile2(uint32_t addr, uint32_t (&w)[16]) {
  asm volatile(
      "ds_read_b32 %0, %16 offset:%17\n\tds_read_b32 %1, %16 offset:%18\n\t"
      "ds_read_b32 %2, %16 offset:%19\n\tds_read_b32 %3, %16 offset:%20\n\t"
      "ds_read_b32 %4, %16 offset:%21\n\tds_read_b32 %5, %16 offset:%22\n\t"
      "ds_read_b32 %6, %16 offset:%23\n\tds_read_b32 %7, %16 offset:%24\n\t"
      "ds_read_b32 %8, %16 offset:%25\n\tds_read_b32 %9, %16 offset:%26\n\t"
      "ds_read_b32 %10, %16 offset:%27\n\tds_read_b32 %11, %16 offset:%28\n\t"
      "ds_read_b32 %12, %16 offset:%29\n\tds_read_b32 %13, %16 offset:%30\n\t"
      "ds_read_b32 %14, %16 offset:%31\n\tds_read_b32 %15, %16 offset:%32\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7]),
        "=&v"(w[8]), "=&v"(w[9]), "=&v"(w[10]), "=&v"(w[11]), "=&v"(w[12]), "=&v"(w[13]), "=&v"(w[14]),
        "=&v"(w[15])
      : "v"(addr), "i"(4 * vpad(0 * RW + CT * HB)), "i"(4 * vpad(1 * RW + CT * HB)),
        "i"(4 * vpad(2 * RW + CT * HB)), "i"(4 * vpad(3 * RW + CT * HB)), "i"(4 * vpad(4 * RW + CT * HB)),
        "i"(4 * vpad(5 * RW + CT * HB)), "i"(4 * vpad(6 * RW + CT * HB)), "i"(4 * vpad(7 * RW + CT * HB)),
        "i"(4 * vpad(0 * RW + (CT + 1) * HB)), "i"(4 * vpad(1 * RW + (CT + 1) * HB)),
        "i"(4 * vpad(2 * RW + (CT + 1) * HB)), "i"(4 * vpad(3 * RW + (CT + 1) * HB)),
        "i"(4 * vpad(4 * RW + (CT + 1) * HB)), "i"(4 * vpad(5 * RW + (CT + 1) * HB)),
        "i"(4 * vpad(6 * RW + (CT + 1) * HB)), "i"(4 * vpad(7 * RW + (CT + 1) * HB)));
}

// Row r < G * Nq of KV head g: query head g * G + r / Nq, query row r % Nq; its index in [H_q][Nq].
__device__ __forceinline__ int64_t dec_row_index(int g, int G, int64_t Nq, int r) {
  return (int64_t)(g * G + r / (int)Nq) * Nq + r % (int)Nq;
}

// V chunk rows per zone: a chunk's code words and (scale, zero) pairs fit 12 blocks of 64 words.
__host__ __device__ constexpr int vchunk_rows(int D, int z) {
  return z == 3 ? (D == 128 ? 8 : 16) : (z == 2 && D == 128) ? 16 : 32;
}


// Reads of two 16-byte values at a0 and a1 (LDS byte addresses) of a copy buffer.
__device__ __forceinline__ void lds_rd_128_pair(uint32_t a0, uint32_t a1, uint4& x, uint4& y) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 p, r;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)" : "=&v"(p), "=&v"(r) : "v"(a0), "v"(a1));
  x = make_uint4(p[0], p[1], p[2], p[3]);
  y = make_uint4(r[0], r[1], r[2], r[3]);
}

// ---------------------------------------------------------------------------------------
// attend_dec_logits

template <int RP>
struct LgSmem {
  uint16_t qb[RP][kPPMax];           // q of row r at position pp as bf16 bits (0: padding)
  int16_t ppslot[kPPMax];            // K parameter slot of position pp (-1: raw or padding)
  int16_t ppch[kPPMax];              // channel of position pp (-1: padding)
  int16_t srcw[kKSt];                // staged K word -> word of the group (class padding: word 0)
  alignas(16) uint16_t qah[kDcWaves][RP][kPPMax];   // per wave: bf16 hi of q * scale
  alignas(16) uint16_t qal[kDcWaves][RP][kPPMax];   // bf16 lo
  alignas(16) uint16_t zbv[kDcWaves][kPPMax];       // K zeros as bf16 bits (0: raw and padding)
  int64_t zrow[4];                   // first logits row of each V zone of the head
  int64_t lim[RP];                   // last visible token of row r (-1: padding row)
  float red[kDcWaves][RP];
  uint64_t scan[kDcWaves];
  int pp0[5], sbase[5], ccnt[4];     // per width class: first position, first staged word, channels
};

template <int D, int RP>
__global__ void __launch_bounds__(kDcThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
attend_dec_logits(const uint16_t* __restrict__ q, kvc_packed_cache cache, float* __restrict__ logit,
                  float* __restrict__ bmax, int G, int Hkv, int64_t N, int64_t Nq, int64_t shift, int causal,
                  float c, int nsplit, int32_t* __restrict__ status) {
  __shared__ LgSmem<RP> sm;
  __shared__ uint32_t ring[kDcWaves * kKRing];   // copy buffers: written by global -> LDS loads only
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: scalar registers and branches
  const int ln = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y;
  const int R = G * (int)Nq;
  const int64_t* H = cache.header;
  const bool bad = H[0] != Hkv || H[1] != D || H[2] != N;
  // the call's only status writer (every block sees the same header): no separate reset launch
  if (t == 0 && split == 0 && g == 0 && status) *status = bad ? KVC_DEV_BAD_CACHE : 0;
  if (bad) return;
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  const int64_t Rg = hp[4], ngroups = hp[22];
  const int Wk = (int)hp[20], Qk = (int)hp[21];
  const int64_t slot0 = hp[17], kword0 = hp[18], kpar0 = hp[19];
  const int64_t gps = (ngroups + nsplit - 1) / nsplit;
  const int64_t j_begin = (int64_t)split * gps;
  const int64_t j_end = j_begin + gps < ngroups ? j_begin + gps : ngroups;

  // ---- set-up: positions (K channels by width class, each class padded to a multiple of 8), the
  // staging order of a group's words, the query and row tables
  {
    uint32_t b = 0;
    int cls = 4;
    uint64_t f = 0;
    if (t < D) {
      b = cache.k_width[(int64_t)g * D + t];
      cls = b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : b == 16 ? 3 : 4;
      // word offset [0,16), parameter slot [16,24), one 8-bit count per width class from bit 24
      if (cls < 4) f = (uint64_t)b | ((uint64_t)(cls < 3) << 16) | (1ull << (24 + 8 * cls));
    }
    uint64_t tf;
    const uint64_t ef = block_excl_scan<kDcThreads>(f, &tf, sm.scan);
    if (t == 0) {
      int pp = 0, sb = 0;
      for (int k = 0; k < 4; ++k) {
        const int n = (int)((tf >> (24 + 8 * k)) & 0xFF);
        const int np = (n + 7) & ~7;
        sm.ccnt[k] = n;
        sm.pp0[k] = pp;
        sm.sbase[k] = sb;
        pp += np;
        sb += np * (2 << k);
      }
      sm.pp0[4] = pp;
      sm.sbase[4] = sb;
    }
    for (int i = t; i < kKSt; i += kDcThreads) sm.srcw[i] = 0;
    for (int i = t; i < kPPMax; i += kDcThreads) {
      sm.ppch[i] = -1;
      sm.ppslot[i] = -1;
    }
    if (t < RP) sm.lim[t] = t < R ? (causal ? N - Nq + shift + t % (int)Nq : N - 1) : -1;
    if (t < 4) sm.zrow[t] = hp[5 + t];
    __syncthreads();
    if (t < D && cls < 4) {
      const int rank = (int)((ef >> (24 + 8 * cls)) & 0xFF);
      const int pp = sm.pp0[cls] + rank;
      const int P = sm.pp0[cls + 1] - sm.pp0[cls];
      const int off = (int)(ef & 0xFFFF);
      sm.ppch[pp] = (int16_t)t;
      if (cls < 3) sm.ppslot[pp] = (int16_t)((ef >> 16) & 0xFF);
      for (int wi = 0; wi < (int)b; ++wi) sm.srcw[sm.sbase[cls] + wi * P + rank] = (int16_t)(off + wi);
    }
    __syncthreads();
    for (int i = t; i < RP * kPPMax; i += kDcThreads) {
      const int r = i / kPPMax, pp = i % kPPMax;
      const int ch = sm.ppch[pp];
      sm.qb[r][pp] = (r < R && ch >= 0) ? q[dec_row_index(g, G, Nq, r) * D + ch] : (uint16_t)0;
    }
  }
  const int npp = sm.pp0[4], nkb = (npp + 31) >> 5, Ws = sm.sbase[4];
  // this lane's 8-position runs (block kb, positions 32 kb + 8 lg ..) for token t of each half, one
  // word each: staged address of the token's words | path << 12 | bit << 16 | byte (raw: half) << 20
  // | 2-bit << 22 | real positions of a raw run << 24
  uint32_t kd[2][kKBMax];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tt = 16 * h + ln;
#pragma unroll
    for (int kb = 0; kb < kKBMax; ++kb) {
      const int pp = 32 * kb + 8 * lg;
      kd[h][kb] = 0;
      if (pp < npp) {
        const int cls = pp >= sm.pp0[3] ? 3 : pp >= sm.pp0[2] ? 2 : pp >= sm.pp0[1] ? 1 : 0;
        const int lb = cls + 1;
        const int P = sm.pp0[cls + 1] - sm.pp0[cls];
        const int a = sm.sbase[cls] + (tt >> (5 - lb)) * P + (pp - sm.pp0[cls]);
        const int sh = (tt << lb) & 31;
        const int path = cls < 2 ? 1 : cls == 2 ? 2 : 3;
        const int byte = path == 3 ? (tt & 1) : (sh >> 3);
        const int nval = min(8, sm.pp0[cls] + sm.ccnt[cls] - pp);
        kd[h][kb] = (uint32_t)a | ((uint32_t)path << 12) | ((uint32_t)(sh & 7) << 16) | ((uint32_t)byte << 20) |
                    ((uint32_t)(cls == 0) << 22) | ((uint32_t)nval << 24);
      }
    }
  }
  // this lane's position pairs 2 lane + 128 i + e: their parameter slots and the query values
  int kslot[2][2];
  float qv[RP][2];                                // the query at the first pair (the second, positions
#pragma unroll                                    // 128.., is read from LDS where it is used)
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int pp = 2 * lane + 128 * i + e;
      kslot[i][e] = pp < npp ? sm.ppslot[pp] : -1;
      if (i == 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r) qv[r][e] = bf16_bits_to_f32(sm.qb[r][pp]);
      }
    }
  __syncthreads();

  // ---- this wave's groups j_begin + w + 4 k through a ring of NBK slots, each a group's staged
  // words, its (scale, zero) pairs, its token ids and V locations; filled NBK - 1 groups ahead
  // a group's staged words beyond what a slot holds (heads whose channels are mostly 16-bit) are
  // read from global memory where they are used
  const int ssp = 2 * Qk, ssp4 = (ssp + 3) & ~3;
  const int cap = Ws < ((kKRing - 64 - ssp4) & ~7) ? Ws : ((kKRing - 64 - ssp4) & ~7);   // staged words
  const int ssw = (cap + 3) & ~3;
  const int SS = ssw + ssp4 + 64;
  int NBK = kKRing / SS;
  NBK = NBK < kKMaxSlots ? NBK : kKMaxSlots;
  const int cg = (cap + 63) / 64 + (ssp + 63) / 64 + 1;  // copies per group
  if (NBK > 2 && (NBK - 2) * cg > 63) NBK = 2 + 63 / cg;  // the wait count field holds 63
  const int64_t nblk = j_end - j_begin;
  const int nw = nblk > w ? (int)((nblk - w + kDcWaves - 1) / kDcWaves) : 0;
  const uint32_t* kwords = cache.k_words + kword0;
  const float* kparf = cache.k_par + 2 * kpar0;
  lds_u32* ring_l = (lds_u32*)&ring[w * kKRing];
  const uint32_t ring_b = lds_addr(&ring[w * kKRing]);
  const int r_col = ln % RP;
  constexpr int kIPL = RP >= 4 ? RP / 4 : 1;        // logits a lane stores per token half
  const int64_t lim_col = sm.lim[r_col];
  const uint32_t zrow32[4] = {(uint32_t)sm.zrow[0], (uint32_t)sm.zrow[1], (uint32_t)sm.zrow[2], (uint32_t)sm.zrow[3]};
  auto stage_group = [&](int k, int slot) {
    const int64_t j = j_begin + w + (int64_t)kDcWaves * k;
    lds_u32* dst = ring_l + slot * SS;
    const uint32_t* gw = kwords + j * Wk;
    for (int i0 = 0; 64 * i0 < cap; i0 += 4) {    // copy i moves staged words 64 i .. 64 i + 63
      int src[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int u = 64 * (i0 + b) + lane;
        src[b] = u < kKSt ? sm.srcw[u] : 0;        // read together, ahead of the copies
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = i0 + b;
        if (64 * i < cap && 64 * i + lane < cap) stage_dword(gw + src[b], dst + 64 * i);
      }
    }
    const float* gp = kparf + j * ssp;
    for (int i = 0; 64 * i < ssp; ++i)
      if (64 * i + lane < ssp) stage_dword(gp + 64 * i + lane, dst + ssw + 64 * i);
    const int64_t e = j * 32 + (lane & 31);       // token ids (lanes 0..31), V locations (32..63)
    if (e < Rg)
      stage_dword(lane < 32 ? (const void*)(cache.k_keep + slot0 + e) : (const void*)(cache.k_vloc + slot0 + e),
                  dst + ssw + ssp4);
  };
  const int npre = NBK > 1 ? (NBK - 1 < nw ? NBK - 1 : nw) : (nw > 0 ? 1 : 0);
  for (int k = 0; k < npre; ++k) stage_group(k, k);
  float mx = -INFINITY;
  for (int k = 0; k < nw; ++k) {
    const int slot = NBK > 1 ? k % NBK : 0;
    {
      const int ahead = NBK > 1 ? (NBK - 2 < nw - 1 - k ? NBK - 2 : nw - 1 - k) : 0;
      wait_vm((ahead > 0 ? ahead : 0) * cg);    // this group's copies have landed
    }
    if (NBK > 1 && k + NBK - 1 < nw) stage_group(k + NBK - 1, (k + NBK - 1) % NBK);
    const int64_t j = j_begin + w + (int64_t)kDcWaves * k;
    const uint32_t sb = ring_b + 4u * (uint32_t)(slot * SS);
    // q * scale (hi, lo) and the zeros of this group, two positions a lane per 32-bit store
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pp = 2 * lane + 128 * i;
      if (pp < 32 * nkb) {
        float sc[2] = {1.f, 1.f};
        uint32_t zb = 0u;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (kslot[i][e] >= 0) {
            const uint64_t pv = lds_rd_64(sb + 4u * (uint32_t)(ssw + 2 * kslot[i][e]));
            sc[e] = __uint_as_float((uint32_t)pv);
            zb |= ((uint32_t)(pv >> 48)) << (16 * e);   // the zero as bf16 bits (a bf16 value)
          }
        *reinterpret_cast<uint32_t*>(&sm.zbv[w][pp]) = zb;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          uint32_t hi = 0u, lo = 0u;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float v = (i == 0 ? qv[r][e] : bf16_bits_to_f32(sm.qb[r][pp + e])) * sc[e];
            const __bf16 hb = (__bf16)v;
            const __bf16 lb2 = (__bf16)(v - (float)hb);
            hi |= (uint32_t)__builtin_bit_cast(uint16_t, hb) << (16 * e);
            lo |= (uint32_t)__builtin_bit_cast(uint16_t, lb2) << (16 * e);
          }
          *reinterpret_cast<uint32_t*>(&sm.qah[w][r][pp]) = hi;
          *reinterpret_cast<uint32_t*>(&sm.qal[w][r][pp]) = lo;
        }
      }
    }
    wave_lds_sync();
    // both token halves per 32-position block: the block's B operands are read once, and the zero
    // term (the same for every token) is one product per block
    f32x4 s2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, sz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kKBMax; ++kb) {
      if (kb < nkb) {
        uint32_t dA0 = kd[0][kb], dA1 = kd[1][kb];
        asm volatile("" : "+v"(dA0), "+v"(dA1));   // derived selectors stay inside the loop
        const int path = (int)((dA0 >> 12) & 3);
        const int pk = 32 * kb + 8 * lg;
        const int ad0 = (int)(dA0 & 0xFFFu), ad1 = (int)(dA1 & 0xFFFu);
        const bool st0 = ad0 + 8 <= cap, st1 = ad1 + 8 <= cap;
        uint4 w00, w01, w10, w11, bh, bl, az, bq;
        lds_rd_kblock(sb + 4u * (uint32_t)(st0 ? ad0 : 0), sb + 4u * (uint32_t)(st1 ? ad1 : 0),
                       lds_addr(&sm.qah[w][r_col][pk]), lds_addr(&sm.qal[w][r_col][pk]), lds_addr(&sm.zbv[w][pk]),
                       lds_addr(&sm.qb[r_col][pk]), w00, w01, w10, w11, bh, bl, az, bq);
        if (path != 0 && (!st0 || !st1)) {       // past the slot: the group's words in global memory
          const uint32_t* gw = kwords + j * Wk;
          if (!st0) {
            uint32_t x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = gw[sm.srcw[ad0 + i]];
            w00 = make_uint4(x[0], x[1], x[2], x[3]);
            w01 = make_uint4(x[4], x[5], x[6], x[7]);
          }
          if (!st1) {
            uint32_t x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = gw[sm.srcw[ad1 + i]];
            w10 = make_uint4(x[0], x[1], x[2], x[3]);
            w11 = make_uint4(x[4], x[5], x[6], x[7]);
          }
        }
        const uint4 a0 = kcodes(dA0, w00, w01), a1 = kcodes(dA1, w10, w11);
        s2[0] = mfma16(a0, bh, s2[0]);
        s2[1] = mfma16(a1, bh, s2[1]);
        s2[0] = mfma16(a0, bl, s2[0]);
        s2[1] = mfma16(a1, bl, s2[1]);
        sz = mfma16(az, bq, sz);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 s;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = s2[h][i] + sz[i];
      // tokens 16 h + 4 lg + i of column ln (row ln % RP): the 16 / RP copies of a row's column share
      // its four tokens, so a lane stores the logits of IPL of them by V row
      if (ln % RP < R && (ln / RP) * kIPL < 4) {
        uint4 tk, vl;
        const uint32_t ta = sb + 4u * (uint32_t)(ssw + ssp4 + 16 * h + 4 * lg);
        lds_rd_128_pair(ta, ta + 128u, tk, vl);
#pragma unroll
        for (int ii = 0; ii < kIPL; ++ii) {
          const int i = (ln / RP) * kIPL + ii;
          if (j * 32 + 16 * h + 4 * lg + i < Rg) {
            const uint32_t tki = i == 0 ? tk.x : i == 1 ? tk.y : i == 2 ? tk.z : tk.w;
            const uint32_t vli = i == 0 ? vl.x : i == 1 ? vl.y : i == 2 ? vl.z : vl.w;
            const float si = i == 0 ? s[0] : i == 1 ? s[1] : i == 2 ? s[2] : s[3];
            const float v = (int64_t)(int32_t)tki <= lim_col ? si : -INFINITY;
            const uint32_t row = zrow32[vli >> 29] + (vli & ((1u << 29) - 1u));   // below 2^31
            logit[row * (uint32_t)RP + (uint32_t)(ln % RP)] = v;
            mx = fmaxf(mx, v);
          }
        }
      }
    }
    wave_lds_sync();                              // the slot and the q * scale buffers are read
    if (NBK == 1 && k + 1 < nw) stage_group(k + 1, 0);
  }
  wave_vm_sync();
#pragma unroll
  for (int o = RP; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));   // the copies of a row
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (lane < RP) sm.red[w][lane] = mx;
  __syncthreads();
  if (t < RP) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kDcWaves; ++k) m = fmaxf(m, sm.red[k][t]);
    bmax[((int64_t)g * nsplit + split) * RP + t] = m > -INFINITY ? m * c : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// attend_dec_values

template <int D, int RP>
struct VlSmem {
  alignas(16) float out[kDcWaves][RP][D];   // each wave's O per row
  float M[RP];                              // the head's maximum per row (base 2)
  float lred[kDcWaves][RP];
  int64_t zrow[4], vzw[4], vzp[4];          // per V zone: first logits row, first word, first pair
  int zcnt[4], zch[4];
  int64_t rowi[RP];
};

template <int D, int RP>
struct DecGeomV {
  static constexpr int GPR = D / 32;
  static constexpr int NGC = (16 / RP) < GPR ? (16 / RP) : GPR;   // channel groups per pass
  static constexpr int NPASS = (GPR + NGC - 1) / NGC;
};

// Logit, pair and word layout of a chunk slot: words and pairs in blocks of 64 words 66 apart
// (vpad), then the chunk's logits [row][RP].
template <int RP>
struct VSlot {
  static constexpr int WORDS = kVSlotWords + 32 * RP;
};

// One chunk of zone Z (rows row0 .. row0 + crows - 1 of the zone, staged at LDS byte address vb):
// the O^T tiles, the zero-term partial sums and the weight sum of this lane's column.
template <int D, int RP, int Z>
__device__ __forceinline__ void v_chunk(const float* Ms, uint32_t vb, int crows, int R, float c, int ln, int lg,
                                        f32x4 (&o)[D / 16], float (&ozp)[DecGeomV<D, RP>::NPASS], float& lsum) {
  using Gm = DecGeomV<D, RP>;
  constexpr int GPR = Gm::GPR, NGC = Gm::NGC, NPASS = Gm::NPASS;
  constexpr int NT = D / 16;
  constexpr int B = 2 << Z, LB = Z + 1;
  constexpr int RW = GPR * B;
  constexpr int CR = vchunk_rows(D, Z);
  constexpr int PATH = Z < 2 ? 1 : Z == 2 ? 2 : 3;
  constexpr uint32_t MASK = Z == 0 ? 0x03030303u : 0x0F0F0F0Fu;
  asm volatile("" : "+v"(ln), "+v"(lg));      // lane constants are rebuilt per chunk, not hoisted
  const int r_col = ln % RP;
  const bool lane_rows = 8 * lg < CR;          // this lane's 8 rows lie inside the chunk's staging
  const int sh = (ln << LB) & 31;              // bit of this lane's channel in its word
  const int wln = ln >> (5 - LB);              // word of this lane's channel within a tile's words
  const uint32_t sel_a = PATH == 3 ? ((ln & 1) ? 0x07060302u : 0x05040100u)
                                   : ((uint32_t)(sh >> 3) | ((uint32_t)((sh >> 3) + 4) << 8) | 0x0C0C0000u);
  const int bit = sh & 7;
  // word (8 lg + i) RW + ct B/2 + wln sits at vpad(8 lg RW) + wln + vpad(i RW + ct B/2): the lane's
  // part never carries into the next block of 64
  const uint32_t wbase = vb + 4u * (uint32_t)(vpad(8 * lg * RW) + wln);
  // the weights of this lane's rows (8 lg + i of the chunk) for its column's row
  float p[8];
  {
    const float m = Ms[r_col];
    uint32_t sv[8];
    if (lane_rows)
      lds_rd_8x32<0, 4 * RP, 8 * RP, 12 * RP, 16 * RP, 20 * RP, 24 * RP, 28 * RP>(
          vb + 4u * (uint32_t)(kVSlotWords + 8 * lg * RP + r_col), sv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = lane_rows ? __uint_as_float(sv[i]) : -INFINITY;
      const bool ok = lane_rows && 8 * lg + i < crows && r_col < R && x > -INFINITY && m > -INFINITY;
      p[i] = ok ? fast_exp2(fmaf(x, c, -m)) : 0.f;
    }
  }
  if (ln < RP) {                               // one column per row counts the weights
#pragma unroll
    for (int i = 0; i < 8; ++i) lsum += p[i];
  }
  static_for(std::make_integer_sequence<int, NPASS>{}, [&](auto psc) {
    constexpr int ps = decltype(psc)::value;
    const int grp = ps * NGC + ln / RP;
    const bool gok = (ln / RP) < NGC && grp < GPR;
    float x[8];
    float zs = 0.f;
    uint64_t pv[8];
    if (Z < 3 && lane_rows) {
      // pair (8 lg + i, grp) at word CR RW + 2 ((8 lg + i) GPR + grp): lane part + 8 i GPR bytes
      const int u0 = CR * RW + 2 * (8 * lg * GPR + (gok ? grp : 0));
      lds_rd_8x64<8 * GPR>(vb + 4u * (uint32_t)vpad(u0), pv);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = (uint64_t)__float_as_uint(1.f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sv = __uint_as_float((uint32_t)pv[i]), zv = __uint_as_float((uint32_t)(pv[i] >> 32));
      const bool ok = gok && p[i] != 0.f;      // stale parameters of rows past the chunk stay out
      x[i] = ok ? p[i] * sv : 0.f;
      zs = ok ? fmaf(p[i], zv, zs) : zs;
    }
    ozp[ps] += zs;
    uint4 bh, bl;
    hilo8(x, bh, bl);
    static_for(std::make_integer_sequence<int, NT / 2>{}, [&](auto cpc) {
      constexpr int ct = 2 * decltype(cpc)::value;   // tiles ct and ct + 1: one channel group
      if constexpr ((ct / 2) / NGC == ps) {    // the tiles of this pass's channel groups
        uint4 a0 = make_uint4(0u, 0u, 0u, 0u), a1 = a0;
        if (lane_rows) {
          uint32_t wv[16];
          lds_rd_tile2<RW, ct, B / 2>(wbase, wv);
          a0 = codes8<PATH>(make_uint4(wv[0], wv[1], wv[2], wv[3]), make_uint4(wv[4], wv[5], wv[6], wv[7]), sel_a,
                            bit, MASK);
          a1 = codes8<PATH>(make_uint4(wv[8], wv[9], wv[10], wv[11]), make_uint4(wv[12], wv[13], wv[14], wv[15]),
                            sel_a, bit, MASK);
          if (PATH == 3 && crows < CR) {       // raw rows past the chunk hold stale bit patterns
            uint32_t aa[4] = {a0.x, a0.y, a0.z, a0.w}, bb[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int k = 8 * lg + 2 * i;
              const uint32_t mk = (k < crows ? 0x0000FFFFu : 0u) | (k + 1 < crows ? 0xFFFF0000u : 0u);
              aa[i] &= mk;
              bb[i] &= mk;
            }
            a0 = make_uint4(aa[0], aa[1], aa[2], aa[3]);
            a1 = make_uint4(bb[0], bb[1], bb[2], bb[3]);
          }
        }
        o[ct] = mfma16(a0, bh, o[ct]);
        o[ct + 1] = mfma16(a1, bh, o[ct + 1]);
        o[ct] = mfma16(a0, bl, o[ct]);
        o[ct + 1] = mfma16(a1, bl, o[ct + 1]);
      }
    });
  });
}

template <int D, int RP>
__global__ void __launch_bounds__(kDcThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
attend_dec_values(kvc_packed_cache cache, const float* __restrict__ logit, const float* __restrict__ bmax,
                  float* __restrict__ part, int G, int Hkv, int64_t N, int64_t Nq, float c, int nsa, int nsplit,
                  int pstride) {
  using Gm = DecGeomV<D, RP>;
  constexpr int GPR = Gm::GPR, NGC = Gm::NGC, NPASS = Gm::NPASS;
  constexpr int NT = D / 16;
  constexpr int PSTRIDE = D + 2;
  constexpr int VS = VSlot<RP>::WORDS;
  __shared__ VlSmem<D, RP> sm;
  __shared__ uint32_t vring[kDcWaves * kVSlots * VS];   // copy buffers: written by global -> LDS loads only
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y;
  const int R = G * (int)Nq;
  const int64_t* H = cache.header;
  if (H[0] != Hkv || H[1] != D || H[2] != N) return;      // reported by the logits kernel
  const int64_t* hp = H + KVC_HDR_GLOBAL + g * KVC_HDR_PER_HEAD;
  if (t < RP) {
    float m = -INFINITY;
    for (int s2 = 0; s2 < nsa; ++s2) m = fmaxf(m, bmax[((int64_t)g * nsa + s2) * RP + t]);
    sm.M[t] = m;
    sm.rowi[t] = t < R ? dec_row_index(g, G, Nq, t) : 0;
  }
  if (t < 4) {
    sm.zrow[t] = hp[5 + t];
    sm.vzw[t] = hp[9 + t];
    sm.vzp[t] = hp[13 + t];
    const int cnt = (int)hp[t], cr = vchunk_rows(D, t);
    sm.zcnt[t] = cnt;
    sm.zch[t] = (cnt + cr - 1) / cr;
  }
  __syncthreads();
  const int nch0 = sm.zch[0], nch1 = sm.zch[1], nch2 = sm.zch[2], nch3 = sm.zch[3];
  const int nch = nch0 + nch1 + nch2 + nch3;
  const int cps = (nch + nsplit - 1) / nsplit;
  const int q0 = split * cps, q1 = q0 + cps < nch ? q0 + cps : nch;
  const int nwv = q1 - q0 > w ? (q1 - q0 - w + kDcWaves - 1) / kDcWaves : 0;   // this wave's chunks
  lds_u32* vr_l = (lds_u32*)&vring[w * kVSlots * VS];
  const uint32_t vr_b = lds_addr(&vring[w * kVSlots * VS]);
  auto chunk_of = [&](int qc, int& z, int& row0, int& crows) {
    const int nzc[4] = {nch0, nch1, nch2, nch3};
    z = 0;
    int qq = qc;
    while (z < 3 && qq >= nzc[z]) {
      qq -= nzc[z];
      ++z;
    }
    const int cr = vchunk_rows(D, z);
    row0 = qq * cr;
    crows = sm.zcnt[z] - row0 < cr ? sm.zcnt[z] - row0 : cr;
  };
  auto copies_of = [&](int k) {                 // copies of this wave's chunk k (wave-uniform)
    int z, row0, crows;
    chunk_of(q0 + w + kDcWaves * k, z, row0, crows);
    const int rw = GPR * (2 << z);
    return (crows * rw + 63) / 64 + (z < 3 ? (2 * crows * GPR + 63) / 64 : 0) + (crows * RP + 63) / 64;
  };
  auto stage_chunk = [&](int k, int slot) {
    int z, row0, crows;
    chunk_of(q0 + w + kDcWaves * k, z, row0, crows);
    const int rw = GPR * (2 << z);
    lds_u32* dst = vr_l + slot * VS;
    const uint32_t* src = cache.v_words + sm.vzw[z] + (int64_t)row0 * rw;
    const int n = crows * rw;
    for (int i = 0; 64 * i < n; ++i)
      if (64 * i + lane < n) stage_dword(src + 64 * i + lane, dst + 66 * i);
    if (z < 3) {
      const float* sp = cache.v_par + 2 * (sm.vzp[z] + (int64_t)row0 * GPR);
      const int np = 2 * crows * GPR;
      const int ib = vchunk_rows(D, z) * rw / 64;
      for (int i = 0; 64 * i < np; ++i)
        if (64 * i + lane < np) stage_dword(sp + 64 * i + lane, dst + 66 * (ib + i));
    }
    const float* lp = logit + (sm.zrow[z] + row0) * RP;
    const int nl = crows * RP;
    for (int i = 0; 64 * i < nl; ++i)
      if (64 * i + lane < nl) stage_dword(lp + 64 * i + lane, dst + kVSlotWords + 64 * i);
  };

  f32x4 o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ozp[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) ozp[i] = 0.f;
  float lsum = 0.f;
  const int npre = kVSlots - 1 < nwv ? kVSlots - 1 : nwv;
  for (int k = 0; k < npre; ++k) stage_chunk(k, k);
  for (int k = 0; k < nwv; ++k) {
    int outstanding = 0;                          // copies issued after chunk k
    for (int m = k + 1; m < nwv && m < k + kVSlots - 1; ++m) outstanding += copies_of(m);
    wait_vm(outstanding);
    if (k + kVSlots - 1 < nwv) stage_chunk(k + kVSlots - 1, (k + kVSlots - 1) % kVSlots);
    int z, row0, crows;
    chunk_of(q0 + w + kDcWaves * k, z, row0, crows);
    const uint32_t vbc = vr_b + 4u * (uint32_t)((k % kVSlots) * VS);
    if (z == 0) v_chunk<D, RP, 0>(sm.M, vbc, crows, R, c, ln, lg, o, ozp, lsum);
    else if (z == 1) v_chunk<D, RP, 1>(sm.M, vbc, crows, R, c, ln, lg, o, ozp, lsum);
    else if (z == 2) v_chunk<D, RP, 2>(sm.M, vbc, crows, R, c, ln, lg, o, ozp, lsum);
    else v_chunk<D, RP, 3>(sm.M, vbc, crows, R, c, ln, lg, o, ozp, lsum);
    wave_lds_sync();                              // this slot is refilled next
  }
  wave_vm_sync();

  // ---- the wave's O and l per row: column n holds row n % RP and its channel group n / RP
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    ozp[i] += __shfl_xor(ozp[i], 16, 64);
    ozp[i] += __shfl_xor(ozp[i], 32, 64);
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (lane < RP) sm.lred[w][lane] = lsum;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int gg = ct / 2, ps = gg / NGC;
    if (ln / RP == gg % NGC && ln / RP < NGC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.out[w][ln % RP][16 * ct + 4 * lg + i] = o[ct][i] + ozp[ps];
    }
  }
  __syncthreads();
  for (int idx = t; idx < R * D; idx += kDcThreads) {
    const int r = idx / D, cc = idx % D;
    float Or = 0.f;
#pragma unroll
    for (int k = 0; k < kDcWaves; ++k) Or += sm.out[k][r][cc];
    float* pr2 = part + (sm.rowi[r] * pstride + split) * PSTRIDE;
    if (cc == 0) {
      float L = 0.f;
#pragma unroll
      for (int k = 0; k < kDcWaves; ++k) L += sm.lred[k][r];
      pr2[0] = sm.M[r];
      pr2[1] = L;
    }
    pr2[2 + cc] = Or;
  }
}

}  // namespace

static int logits_nsplit(const Layer& L) {
  const int64_t groups = (L.n + 31) / 32;                 // K groups per head, at most
  int64_t want = (1024 + L.hkv - 1) / L.hkv;              // four blocks per compute unit, one round
  const int64_t cap = (groups + 3) / 4;                   // at least one group per wave
  if (want > cap) want = cap;
  if (want > 255) want = 255;
  if (want < 1) want = 1;
  return (int)want;
}

int decode_nsplit(const Layer& L) {                       // the values kernel's splits (partials per row)
  const int64_t chunks = (L.n + 31) / 32;                 // V chunks per head if most tokens sit below 16 bits
  int64_t want = (1024 + L.hkv - 1) / L.hkv;              // four blocks per compute unit, one round
  const int64_t cap = (chunks + 3) / 4;
  if (want > cap) want = cap;
  if (want > 255) want = 255;                             // one more split for the append buffer
  const int nsa = logits_nsplit(L);
  if (want < nsa) want = nsa;                             // the logits blocks' maxima fit the same array
  return (int)want;
}

static int decode_rows_padded(const Layer& L) {
  const int rows = L.G * (int)L.nq;
  return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16;
}

size_t decode_ws_bytes(const Layer& L) {
  const size_t rp = (size_t)decode_rows_padded(L);
  // logits of every retained token by V row, and the logits blocks' maxima
  return (size_t)L.hkv * (size_t)L.n * rp * sizeof(float) + 256 + (size_t)L.hkv * decode_nsplit(L) * rp * sizeof(float);
}

hipError_t launch_attend_decode(const Layer& L, const uint16_t* q, const kvc_packed_cache& cache, float* part,
                                int nsplit, int pstride, int64_t shift, int32_t* status, char* dws, hipStream_t s) {
  const int nsa = logits_nsplit(L);
  const dim3 grid((unsigned)nsa, (unsigned)L.hkv), gridv((unsigned)nsplit, (unsigned)L.hkv);
  const int rp = decode_rows_padded(L);
  float* logit = reinterpret_cast<float*>(dws);
  float* bm = reinterpret_cast<float*>(dws + (((size_t)L.hkv * (size_t)L.n * rp * sizeof(float) + 255) & ~size_t(255)));
#define KVC_DC(DD, RR)                                                                                          \
  do {                                                                                                          \
    attend_dec_logits<DD, RR><<<grid, kDcThreads, 0, s>>>(q, cache, logit, bm, L.G, L.hkv, L.n, L.nq, shift,     \
                                                          L.causal, L.c_log2, nsa, status);                     \
    attend_dec_values<DD, RR><<<gridv, kDcThreads, 0, s>>>(cache, logit, bm, part, L.G, L.hkv, L.n, L.nq,        \
                                                           L.c_log2, nsa, nsplit, pstride);                     \
  } while (0)
  if (L.d == 128) {
    if (rp == 1) KVC_DC(128, 1);
    else if (rp == 2) KVC_DC(128, 2);
    else if (rp == 4) KVC_DC(128, 4);
    else if (rp == 8) KVC_DC(128, 8);
    else KVC_DC(128, 16);
  } else {
    if (rp == 1) KVC_DC(64, 1);
    else if (rp == 2) KVC_DC(64, 2);
    else if (rp == 4) KVC_DC(64, 4);
    else if (rp == 8) KVC_DC(64, 8);
    else KVC_DC(64, 16);
  }
#undef KVC_DC
  return hipGetLastError();
}

}  // namespace kvc
