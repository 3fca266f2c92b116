// Scorer: pass 1 (row log-sum-exp) and pass 2 (per-token column reductions of the attention
// probabilities), plus the KVzip+ norm helpers.
//
// Pass 1 computes l_{h,i} = ln sum_{t visible} exp(s q.k) (KVSculpt summary §2, LSE term; the
// normaliser of RDKV's attention probabilities, RDKV summary §2.1).  Pass 2 recomputes
// a = exp(s q.k - l) and reduces it over query rows per key: the RDKV token weight (sum,
// RDKV summary §2.1) or the KVzip+ numerator max_j a_{j,t} ||h_j|| (KVzap summary §2.1).
//
// Both passes run QK^T on 32x32x16 bf16 matrix cores with fp32 accumulation, and handle the
// logits in the base-2 domain (x = s*log2(e) * q.k) so a probability is one exp2.
// Work item = (KV head g, 256-row tile, key chunk, query head of the group); a block of 4
// waves owns one item: each wave keeps the bf16 fragments of its 64 query rows in registers
// and the chunk's keys stream through LDS in 64-key tiles (double buffered).  The same
// register fragments serve both passes: pass 1 multiplies K x Q^T so a lane owns a query row
// (row max / sum-exp in-lane), pass 2 multiplies Q x K^T so a lane owns a key (column sums
// in-lane).  Blocks are mapped XCD-aware: the work items of one KV head run on one XCD so
// its keys stay in that XCD's L2.  Pass 1 writes per-chunk (max, sum) partials that a tiny
// kernel combines into l; pass 2 writes per-(head, row tile) column partials that a second
// kernel reduces in a fixed order, so every result is bitwise reproducible.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace kvc {

// Scratch of kvc_row_lse_noalloc: the per-chunk (max, sum) partials of pass 1, in a file-scope
// device array instead of a caller's workspace.  Each device that loads the library holds its
// own copy until the process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): row_lse_scratch() asks the runtime for the device address once per
// device and keeps it.
static __device__ __align__(256) char scratch[kLseScratchBytes];

namespace {
std::mutex g_scratch_mu;
char* g_scratch_dev[64] = {};
}  // namespace

hipError_t row_lse_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;   // 4 waves per block in both passes
constexpr int kRowsPerBlock = 256;
constexpr int kXcds = 8;        // MI355X: blocks are dealt round-robin to 8 XCDs

struct Decomp {
  int G, nRT, maxCh, KC;
  int64_t W;
};

// Work item of a block.  Items are ordered (g, chunk, row tile descending, head in group), and
// block b runs on XCD b % 8, so XCD x receives the x-th eighth of the items: the items that
// read one key chunk (every row tile and head of the group) run together on one XCD and share
// its L2, so each key is fetched from HBM about once.
// W < 2^31 (the launchers check it), so the index arithmetic is 32-bit.
__device__ __forceinline__ bool decode_work(const Decomp& dc, int& g, int& rt, int& ch, int& hl) {
  const uint32_t b = blockIdx.x, W = (uint32_t)dc.W;
  const uint32_t per = (W + kXcds - 1) / kXcds;
  uint32_t w = (b % kXcds) * per + b / kXcds;
  if (w >= W) return false;
  hl = (int)(w % (uint32_t)dc.G);
  w /= (uint32_t)dc.G;
  rt = dc.nRT - 1 - (int)(w % (uint32_t)dc.nRT);
  w /= (uint32_t)dc.nRT;
  ch = (int)(w % (uint32_t)dc.maxCh);
  g = (int)(w / (uint32_t)dc.maxCh);
  return true;
}

// Last key (exclusive) that any row of row tile rt can see.
__device__ __forceinline__ int64_t tile_kend(int rt, int64_t N, int64_t Nq, int causal) {
  if (!causal) return N;
  int64_t last = (int64_t)(rt + 1) * kRowsPerBlock;
  if (last > Nq) last = Nq;
  int64_t e = N - Nq + last;
  return e < N ? e : N;
}

// ---- K tile ring: 4 LDS slots of 64 keys x D bf16, filled by direct global->LDS loads -----
// Each slot is its own LDS object, so the compiler can tell an in-flight fill of one slot from
// reads of another and does not serialise them.  A key row occupies 2*D contiguous bytes; its
// 16-byte chunks are XOR-swizzled (slot s of row r holds chunk s ^ swz(r)) so that the 32 rows
// read by one matrix-core fragment load hit distinct banks without padding.
__shared__ __attribute__((aligned(16))) uint16_t g_kslot0[64 * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_kslot1[64 * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_kslot2[64 * 128];
__shared__ __attribute__((aligned(16))) uint16_t g_kslot3[64 * 128];

template <int S>
__device__ __forceinline__ uint16_t* kslot() {
  return S == 0 ? g_kslot0 : S == 1 ? g_kslot1 : S == 2 ? g_kslot2 : g_kslot3;
}

template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Global->LDS load instructions per wave for one 64-key tile (each moves 1 KB).
template <int D>
constexpr int tile_loads_per_wave() { return (64 * D * 2) / 1024 / 4; }

// Byte offset, inside a tile, of the 16 bytes lane `lane` of wave `wave` moves with its j-th
// load of every tile (constant across tiles).
template <int D>
__device__ __forceinline__ void tile_offsets(int (&voff)[4], int wave, int lane) {
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;          // rows per load instruction
  constexpr int L = tile_loads_per_wave<D>();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * L + j) * RPI + lane / CPR;
    voff[j] = j < L ? (row * D + 8 * ((lane % CPR) ^ swz<D>(row))) * 2 : 0;
  }
}

// Fill slot S with keys t0 .. t0+63 of head kh.  Buffer loads whose resource ends at key N:
// rows past the end read as zeros (their logits are masked), so a tile that starts at or past
// N issues its loads all the same and touches no memory.
template <int D, int S>
__device__ __forceinline__ void issue_tile(const uint16_t* kh, int t0, int N,
                                           const int (&voff)[4], int wave) {
  constexpr int L = tile_loads_per_wave<D>();
  constexpr int RPI = 64 / (D / 8);
  t0 = __builtin_amdgcn_readfirstlane(t0);   // block-uniform; keeps the resource scalar
  int rows = N - t0;
  rows = rows < 0 ? 0 : (rows > 64 ? 64 : rows);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kh + (int64_t)t0 * D), (short)0, __builtin_amdgcn_readfirstlane(rows * D * 2),
      0x00020000);
#pragma unroll
  for (int j = 0; j < L; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(kslot<S>() + (wave * L + j) * RPI * D), 16,
        voff[j], 0, 0, 0);
}

// Fragment of key row r, logical 16-byte chunk c, from slot S.
template <int D, int S>
__device__ __forceinline__ bf16x8 kfrag(int r, int c) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(kslot<S>() + r * D + 8 * (c ^ swz<D>(r))));
}

// Wait until at most `ahead` tiles of this wave's loads are in flight and every LDS operation
// has finished, then meet the other waves.  The empty asm statements keep the compiler from
// moving memory operations across the barrier.
template <int D>
__device__ __forceinline__ void ring_barrier(int ahead) {
  constexpr int L = tile_loads_per_wave<D>();
  asm volatile("" ::: "memory");
  // s_waitcnt immediate: vmcnt in [3:0] and [15:14], expcnt [6:4] (7 = no wait), lgkmcnt [11:8]
  if (ahead >= 2)
    __builtin_amdgcn_s_waitcnt(((2 * L) & 15) | (((2 * L) >> 4) << 14) | (7 << 4));
  else if (ahead == 1)
    __builtin_amdgcn_s_waitcnt((L & 15) | ((L >> 4) << 14) | (7 << 4));
  else
    __builtin_amdgcn_s_waitcnt(7 << 4);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier for ordinary LDS traffic that leaves the ring's loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// bf16 fragments of this wave's 64 query rows: qf[nb][ks] holds row 32*nb + lane%32,
// columns ks*16 + 8*(lane/32) .. +8.  Rows at or beyond Nq are zero.
template <int D>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[2][D / 16], const uint16_t* q, int h,
                                             int64_t Nq, int64_t row0, int hi, int lo) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t row = row0 + 32 * nb + lo;
    const bool ok = row < Nq;
    const uint16_t* qp = q + ((int64_t)h * Nq + (ok ? row : 0)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[nb][ks] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : make_uint4(0, 0, 0, 0));
  }
}

// Per-block geometry shared by both passes.
struct Geo {
  int g, rt, ch, hl, h, wave, lane, hi, lo;
  int off, i_block, i_wave, kend_wave, k0, k1;   // key / row positions (< 2^29)
  int ntiles;
};

// Decode the block's work item and key range; false for an empty item (uniform).
__device__ __forceinline__ bool geo_of(const Decomp& dc, int64_t N, int64_t Nq, int causal, Geo& o) {
  if (!decode_work(dc, o.g, o.rt, o.ch, o.hl)) return false;
  const int kend = (int)tile_kend(o.rt, N, Nq, causal);
  o.k0 = o.ch * dc.KC;
  if (o.k0 >= kend) return false;
  o.k1 = (o.k0 + dc.KC < kend) ? o.k0 + dc.KC : kend;
  o.lane = threadIdx.x & 63;
  o.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: keeps LDS bases scalar
  o.hi = o.lane >> 5;
  o.lo = o.lane & 31;
  o.h = o.g * dc.G + o.hl;
  o.off = (int)(N - Nq);
  o.i_block = o.rt * kRowsPerBlock;
  o.i_wave = o.i_block + 64 * o.wave;
  o.kend_wave = 0;
  if (o.i_wave < Nq) {
    const int lr = (o.i_wave + 63 < Nq) ? o.i_wave + 63 : (int)Nq - 1;
    o.kend_wave = causal ? ((o.off + lr + 1 < N) ? o.off + lr + 1 : (int)N) : (int)N;
  }
  o.ntiles = (int)((o.k1 - o.k0 + 63) / 64);
  return true;
}

// ---------------------------------------------------------------------------------------
// Both passes run a software pipeline over 32-key half tiles: while the matrix cores compute
// the products of one half, the VALU finishes the softmax work of the previous half.  Two
// accumulator sets (A, B) alternate; a half whose keys are not all visible to every row of
// the wave (the causal diagonal, the end of the cache, rows past Nq) is masked between the
// phases, outside the interleaved code.
// ---------------------------------------------------------------------------------------

// Scheduling fence between pipeline phases: the compiler interleaves matrix-core and VALU
// work inside a phase but moves nothing across except LDS reads (fragment prefetch), which
// bounds the registers live at once.
#define KVC_PHASE_FENCE() __builtin_amdgcn_sched_barrier(0x100)   // LDS reads may cross (prefetch)

// True if every key of the half [t0h, t0h + 32) is visible to every row of the wave.
__device__ __forceinline__ bool half_full(const Geo& G, int t0h, int N, int causal) {
  return (!causal || t0h + 31 <= G.off + G.i_wave) && (t0h + 32 <= N);
}

// ---------------------------------------------------------------------------------------
// Pass 1: per chunk, m = max_t x and l = sum_t 2^(x - m) for every row, x = c * q.k.
// h[nb] = K_half x Q^T block nb: element i of a lane is key 32kb + acc_row(i, hi), row
// 32nb + lo, so a lane holds one row and its softmax statistics stay in-lane.
// ---------------------------------------------------------------------------------------
template <int D, int S>
__device__ __forceinline__ void lse_mfma_half(f32x16 (&h)[2], const bf16x8 (&qf)[2][D / 16], int kb,
                                              int lo, int hi) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) h[nb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a = kfrag<D, S>(kb * 32 + lo, 2 * ks + hi);
    h[0] = mfma32(a, qf[0][ks], h[0]);
    h[1] = mfma32(a, qf[1][ks], h[1]);
  }
}

// Key t0h + acc_row(i, hi) is invisible to row pos iff it lies past min(pos, N - 1) (past
// N - 1 without the causal mask).  With acc_row(i, hi) = 4 hi + r_i, r_i = 8 (i / 4) + i % 4, the
// test is one compare of the constant r_i per element.
__device__ __forceinline__ void lse_mask_half(f32x16 (&h)[2], const Geo& G, int t0h, int N, int causal) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int pos = G.off + G.i_wave + 32 * nb + G.lo;
    const int lim = (causal && pos < N - 1) ? pos : N - 1;
    const int L = lim - t0h - 4 * G.hi;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + (i & 3);
      h[nb][i] = (r > L) ? -INFINITY : h[nb][i];
    }
  }
}

// sum_i 2^(c h_i + nm) over the 16 elements of a lane, in four chains that start from their
// first terms (a chain started from 0 would cost one more add per chain), then a fixed tree.
__device__ __forceinline__ float sum_exp2_16(const f32x16& h, float c, float nm) {
  float s0 = fast_exp2(fmaf(h[0], c, nm)), s1 = fast_exp2(fmaf(h[1], c, nm));
  float s2 = fast_exp2(fmaf(h[2], c, nm)), s3 = fast_exp2(fmaf(h[3], c, nm));
#pragma unroll
  for (int i = 4; i < 16; i += 4) {
    s0 += fast_exp2(fmaf(h[i], c, nm));
    s1 += fast_exp2(fmaf(h[i + 1], c, nm));
    s2 += fast_exp2(fmaf(h[i + 2], c, nm));
    s3 += fast_exp2(fmaf(h[i + 3], c, nm));
  }
  return (s0 + s1) + (s2 + s3);
}

// Online update of (m, l) with one half tile, the running max kept negated (nm_run = -m); no
// branches (an all-masked half leaves m, l).
__device__ __forceinline__ void lse_update_half(const f32x16 (&h)[2], float (&nm_run)[2],
                                                float (&l_run)[2], float c) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float t0 = max3_raw(h[nb][0], h[nb][1], h[nb][2]);
    float t1 = max3_raw(h[nb][3], h[nb][4], h[nb][5]);
#pragma unroll
    for (int i = 6; i < 14; i += 4) {
      t0 = max3_raw(t0, h[nb][i], h[nb][i + 1]);
      t1 = max3_raw(t1, h[nb][i + 2], h[nb][i + 3]);
    }
    t0 = max3_raw(t0, h[nb][14], h[nb][15]);
    const float tmax = half_max(max_raw(t0, t1));
    const float nmnew = fminf(nm_run[nb], -(tmax * c));   // -max(m, tmax c)
    const float nm = (nmnew == INFINITY) ? 0.f : nmnew;
    l_run[nb] = fmaf(l_run[nb], fast_exp2(nm - nm_run[nb]), sum_exp2_16(h[nb], c, nm));
    nm_run[nb] = nmnew;
  }
}

// Update for a half tile that every row sees in full.  The shift m is kept as it is while
// every term 2^(x - m) of the half stays small: the half's sums are added as they stand
// when both are at most 2^64 (so no term can overflow and l stays far below the float
// range), and the exact update above runs for the whole wave otherwise.  That covers the
// first tile (m = -inf makes every sum +inf, or NaN for the all -inf placeholder half,
// which the exact update folds in as zero) and a row whose maximum jumps by more than 60
// in the base-2 domain.  The log-sum-exp m + log2(l) is the same up to rounding for any m
// at or below the running maximum, so only the row max tree and the rescale are saved.
__device__ __forceinline__ void lse_update_half_lazy(const f32x16 (&h)[2], float (&nm_run)[2],
                                                     float (&l_run)[2], float c) {
  float s[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) s[nb] = sum_exp2_16(h[nb], c, nm_run[nb]);
  const bool redo = !(s[0] <= 0x1p64f) || !(s[1] <= 0x1p64f);   // also true for NaN
  if (__builtin_amdgcn_ballot_w64(redo) != 0) {
    lse_update_half(h, nm_run, l_run, c);
  } else {
    l_run[0] += s[0];
    l_run[1] += s[1];
  }
}

// Tiles [0, nfull) are visible in full to every row of the block; they run the pipelined
// step.  The rest (the causal diagonal band and a partial last tile: at most 5 tiles of an
// item) run a masked step without pipelining.
__device__ __forceinline__ int full_tiles(const Geo& G, int N, int causal) {
  int lim = N;                                   // keys [k0, lim) fully visible to all rows
  if (causal) {
    const int e = G.off + G.i_block + 1;         // keys <= first row's position
    lim = e < lim ? e : lim;
  }
  int nf = (lim - G.k0) / 64;
  nf = nf < 0 ? 0 : nf;
  return nf < G.ntiles ? nf : G.ntiles;
}

// One ring step: wait for tile J (two younger tiles may stay in flight), refill the slot the
// previous step freed with tile J + 3 (always issued: rows past the end read as zero and the
// slot is never read), then the two phases of tile J: the first half's products with the
// previous half's softmax update, then the second half's products with the first half's
// update.
#define KVC_LSE_STEP(S, J)                                                                  \
  {                                                                                         \
    ring_barrier<D>(2);                                                                     \
    issue_tile<D, ((S) + 3) & 3>(kh, G.k0 + 64 * ((J) + 3), n, voff, G.wave);               \
    KVC_PHASE_FENCE();                                                                      \
    lse_mfma_half<D, S>(A, qf, 0, G.lo, G.hi);                                              \
    lse_update_half_lazy(B, nm_run, l_run, c);                                               \
    KVC_PHASE_FENCE();                                                                      \
    lse_mfma_half<D, S>(B, qf, 1, G.lo, G.hi);                                              \
    lse_update_half_lazy(A, nm_run, l_run, c);                                               \
    KVC_PHASE_FENCE();                                                                      \
  }

// Masked step (no pipelining): both halves of tile J are masked and folded in.
template <int D, int S>
__device__ __forceinline__ void lse_masked_step(const Geo& G, const uint16_t* kh, int J, int n, int causal,
                                                const int (&voff)[4], const bf16x8 (&qf)[2][D / 16],
                                                float (&nm_run)[2], float (&l_run)[2], float c) {
  ring_barrier<D>(2);
  issue_tile<D, (S + 3) & 3>(kh, G.k0 + 64 * (J + 3), n, voff, G.wave);
  const int t0 = G.k0 + 64 * J;
  f32x16 h[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    lse_mfma_half<D, S>(h, qf, kb, G.lo, G.hi);
    lse_mask_half(h, G, t0 + 32 * kb, n, causal);
    lse_update_half(h, nm_run, l_run, c);
  }
}

// TAG does not change the code: it gives the launches made for another caller (the ridge
// fit's weights) their own kernel name, so that profiles keep the two apart.
template <int D, int TAG>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
lse_partial(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            float2* __restrict__ part, float* __restrict__ lse, Decomp dc, int64_t N, int64_t Nq,
            int causal, float c) {
  Geo G;
  if (!geo_of(dc, N, Nq, causal, G)) return;   // empty item: uniform for the block
  const uint16_t* kh = k + (int64_t)G.g * N * D;
  const int n = (int)N;
  bf16x8 qf[2][D / 16];
  load_q_frags<D>(qf, q, G.h, Nq, G.i_wave, G.hi, G.lo);
  int voff[4];
  tile_offsets<D>(voff, G.wave, G.lane);
  float nm_run[2] = {INFINITY, INFINITY};      // minus the running maxima
  float l_run[2] = {0.f, 0.f};
  // The first tiles are requested while the Q fragments are still in flight, so the two
  // latencies overlap.  Loads complete in issue order: the first ring wait (at most 2L loads
  // outstanding) also covers Q.
  issue_tile<D, 0>(kh, G.k0, n, voff, G.wave);
  issue_tile<D, 1>(kh, G.k0 + 64, n, voff, G.wave);
  issue_tile<D, 2>(kh, G.k0 + 128, n, voff, G.wave);
  const int nfull = full_tiles(G, n, causal);
  int j0 = 0;
  {
    f32x16 A[2], B[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) B[nb][i] = -INFINITY;   // "previous half" of the first step
    for (; j0 + 4 <= nfull; j0 += 4) {
      KVC_LSE_STEP(0, j0)
      KVC_LSE_STEP(1, j0 + 1)
      KVC_LSE_STEP(2, j0 + 2)
      KVC_LSE_STEP(3, j0 + 3)
    }
    if (j0 < nfull) KVC_LSE_STEP(0, j0)
    if (j0 + 1 < nfull) KVC_LSE_STEP(1, j0 + 1)
    if (j0 + 2 < nfull) KVC_LSE_STEP(2, j0 + 2)
    lse_update_half_lazy(B, nm_run, l_run, c);   // second half of the last pipelined tile
  }
  for (int j = nfull; j < G.ntiles; ++j) {
    switch (j & 3) {
      case 0: lse_masked_step<D, 0>(G, kh, j, n, causal, voff, qf, nm_run, l_run, c); break;
      case 1: lse_masked_step<D, 1>(G, kh, j, n, causal, voff, qf, nm_run, l_run, c); break;
      case 2: lse_masked_step<D, 2>(G, kh, j, n, causal, voff, qf, nm_run, l_run, c); break;
      default: lse_masked_step<D, 3>(G, kh, j, n, causal, voff, qf, nm_run, l_run, c); break;
    }
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);       // no LDS fill may outlive the block
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = half_sum(l_run[nb]);
    const int64_t row = G.i_wave + 32 * nb + G.lo;
    if (G.hi == 0 && row < Nq) {
      if (dc.maxCh == 1)   // one chunk covers the row: write l itself
        lse[(int64_t)G.h * Nq + row] = (nm_run[nb] < INFINITY) ? (log2f(lt) - nm_run[nb]) * kLn2 : -INFINITY;
      else
        part[((int64_t)G.h * Nq + row) * dc.maxCh + G.ch] = make_float2(-nm_run[nb], lt);
    }
  }
}

// l = (M + log2 sum_c l_c 2^(m_c - M)) * ln 2 over the chunks of the row's tile.  One wave per
// row: lane c takes chunks c, c + 64, ... (the row's partials are contiguous, so every load
// instruction reads 512 consecutive bytes), then fixed butterfly trees give M and the sum.
__global__ void __launch_bounds__(256)
lse_combine(const float2* __restrict__ part, float* __restrict__ lse, int Hq, int64_t N, int64_t Nq, int causal,
            int KC, int maxCh) {
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // h * Nq + row
  if (idx >= (int64_t)Hq * Nq) return;                                 // uniform per wave
  const int lane = threadIdx.x & 63;
  const int64_t row = idx % Nq;
  const int rt = (int)(row / kRowsPerBlock);
  const int nch = (int)((tile_kend(rt, N, Nq, causal) + KC - 1) / KC);
  const float2* p = part + idx * maxCh;
  float M = -INFINITY;
  for (int ch = lane; ch < nch; ch += 64) M = fmaxf(M, p[ch].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float L = 0.f;
  for (int ch = lane; ch < nch; ch += 64) {
    const float2 v = p[ch];
    if (v.x > -INFINITY) L += v.y * fast_exp2(v.x - M);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
  if (lane == 0) lse[idx] = (M > -INFINITY) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// Pass 2: column reductions.  h[mb] = Q block mb x K_half^T (operands swapped): element i of a
// lane is row 32mb + acc_row(i, hi), key 32kb + lo, so a lane holds one key and 16 rows of
// each 32-row block.  SUM: partial = sum_rows 2^(x - l'), l' = l*log2(e); MAX: partial =
// max_rows (x - l'), l' = l*log2(e) - log2||h||.  One partial per (query head, row tile,
// key), the four waves' rows combined in a fixed order.
// ---------------------------------------------------------------------------------------
template <int D, int S>
__device__ __forceinline__ void score_mfma_half(f32x16 (&h)[2], const bf16x8 (&qf)[2][D / 16], int kb,
                                                int lo, int hi) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) h[mb][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 b = kfrag<D, S>(kb * 32 + lo, 2 * ks + hi);
    h[0] = mfma32(qf[0][ks], b, h[0]);
    h[1] = mfma32(qf[1][ks], b, h[1]);
  }
}

// Row off + i_wave + 32 mb + 4 hi + r_i does not see key t = t0h + lo iff r_i < t - (off +
// i_wave + 32 mb + 4 hi) (causal), and no row sees a key t > N - 1: one compare per element.
__device__ __forceinline__ void score_mask_half(f32x16 (&h)[2], const Geo& G, int t0h, int N, int causal) {
  const int t = t0h + G.lo;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    int M = causal ? t - (G.off + G.i_wave + 32 * mb + 4 * G.hi) : -1;
    if (t > N - 1) M = 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + (i & 3);
      h[mb][i] = (r < M) ? -INFINITY : h[mb][i];
    }
  }
}

// Column value of one half tile for this wave's 64 rows, written to cbw[32 kb + lo].
template <bool MAXMODE>
__device__ __forceinline__ void score_reduce_half(const f32x16 (&h)[2], const float (&lv)[2][16],
                                                  float c, int hi, int lo, float* cbw) {
  float colv;
  if (MAXMODE) {
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        m0 = fmaxf(m0, fmaf(h[mb][i], c, -lv[mb][i]));
        m1 = fmaxf(m1, fmaf(h[mb][i + 1], c, -lv[mb][i + 1]));
      }
    colv = half_max(fmaxf(m0, m1));
  } else {
    float s0 = fast_exp2(fmaf(h[0][0], c, -lv[0][0])), s1 = fast_exp2(fmaf(h[0][1], c, -lv[0][1]));
    float s2 = fast_exp2(fmaf(h[1][0], c, -lv[1][0])), s3 = fast_exp2(fmaf(h[1][1], c, -lv[1][1]));
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      s0 += fast_exp2(fmaf(h[0][i], c, -lv[0][i]));
      s1 += fast_exp2(fmaf(h[0][i + 1], c, -lv[0][i + 1]));
      s2 += fast_exp2(fmaf(h[1][i], c, -lv[1][i]));
      s3 += fast_exp2(fmaf(h[1][i + 1], c, -lv[1][i + 1]));
    }
    colv = half_sum((s0 + s1) + (s2 + s3));
  }
  if (hi == 0) cbw[lo] = colv;
}

// Four waves' partials of one 64-key tile, combined in a fixed order.
template <bool MAXMODE>
__device__ __forceinline__ float combine4(const float* cp) {
  if (MAXMODE) return fmaxf(fmaxf(cp[0], cp[64]), fmaxf(cp[128], cp[192]));
  return (cp[0] + cp[64]) + (cp[128] + cp[192]);
}

// Ring step J (pipelined, tile J fully visible): tile J's halves are reduced in step J
// (first half) and step J + 1 (second half), so the LDS partials of tile J are complete at
// the barrier of step J + 2, where the first wave combines and stores them (three partial
// buffers rotate).  B holds the previous tile's second half (all -inf before the first step,
// which then writes zeros into a buffer that is rewritten before it is read).
#define KVC_SCORE_STEP(S, J)                                                                \
  {                                                                                         \
    ring_barrier<D>(2);                                                                     \
    if ((J) > 1 && threadIdx.x < 64)                                                        \
      out[G.k0 + 64 * ((J) - 2) + (int)threadIdx.x] = combine4<MAXMODE>(&cb[((J) + 1) % 3][0][threadIdx.x]); \
    issue_tile<D, ((S) + 3) & 3>(kh, G.k0 + 64 * ((J) + 3), n, voff, G.wave);               \
    KVC_PHASE_FENCE();                                                                      \
    score_mfma_half<D, S>(A, qf, 0, G.lo, G.hi);                                            \
    score_reduce_half<MAXMODE>(B, lv, c, G.hi, G.lo, &cb[((J) + 2) % 3][G.wave][32]);        \
    KVC_PHASE_FENCE();                                                                      \
    score_mfma_half<D, S>(B, qf, 1, G.lo, G.hi);                                            \
    score_reduce_half<MAXMODE>(A, lv, c, G.hi, G.lo, &cb[(J) % 3][G.wave][0]);               \
    KVC_PHASE_FENCE();                                                                      \
  }

// Masked step (no pipelining) for tiles that cross the causal diagonal or the end of the
// cache: both halves of tile J are masked and reduced in this step.
template <int D, bool MAXMODE, int S>
__device__ __forceinline__ void score_masked_step(const Geo& G, const uint16_t* kh, int J, int n, int causal,
                                                  const int (&voff)[4], const bf16x8 (&qf)[2][D / 16],
                                                  const float (&lv)[2][16], float c, float (&cb)[3][4][64],
                                                  float* out) {
  ring_barrier<D>(2);
  if (J > 1 && threadIdx.x < 64)
    out[G.k0 + 64 * (J - 2) + (int)threadIdx.x] = combine4<MAXMODE>(&cb[(J + 1) % 3][0][threadIdx.x]);
  issue_tile<D, (S + 3) & 3>(kh, G.k0 + 64 * (J + 3), n, voff, G.wave);
  const int t0 = G.k0 + 64 * J;
  f32x16 h[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    score_mfma_half<D, S>(h, qf, kb, G.lo, G.hi);
    score_mask_half(h, G, t0 + 32 * kb, n, causal);
    score_reduce_half<MAXMODE>(h, lv, c, G.hi, G.lo, &cb[J % 3][G.wave][32 * kb]);
  }
}

template <int D, bool MAXMODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
score_partial(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              const float* __restrict__ lse, const float* __restrict__ hlog2,
              float* __restrict__ part, Decomp dc, int64_t N, int64_t Nq, int causal, float c,
              int64_t Npad) {
  __shared__ float cb[3][4][64];
  __shared__ float lrow[kRowsPerBlock];
  Geo G;
  if (!geo_of(dc, N, Nq, causal, G)) return;
  const uint16_t* kh = k + (int64_t)G.g * N * D;
  const int n = (int)N;
  float* out = part + ((int64_t)G.h * dc.nRT + G.rt) * Npad;
  {
    const int64_t row = G.i_block + threadIdx.x;
    float v = INFINITY;                            // rows beyond Nq contribute nothing
    if (row < Nq) {
      v = lse[(int64_t)G.h * Nq + row] * kLog2e;
      if (MAXMODE) v -= hlog2[row];
    }
    lrow[threadIdx.x] = v;
  }
  bf16x8 qf[2][D / 16];
  load_q_frags<D>(qf, q, G.h, Nq, G.i_wave, G.hi, G.lo);
  int voff[4];
  tile_offsets<D>(voff, G.wave, G.lane);
  // The first tiles are requested while Q is in flight (loads complete in issue order, so the
  // first ring wait covers Q too).
  issue_tile<D, 0>(kh, G.k0, n, voff, G.wave);
  issue_tile<D, 1>(kh, G.k0 + 64, n, voff, G.wave);
  issue_tile<D, 2>(kh, G.k0 + 128, n, voff, G.wave);
  lds_barrier();
  float lv[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) lv[mb][i] = lrow[64 * G.wave + 32 * mb + acc_row(i, G.hi)];
  const int nfull = full_tiles(G, n, causal);
  int j0 = 0;
  {
    f32x16 A[2], B[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) B[mb][i] = -INFINITY;
    for (; j0 + 4 <= nfull; j0 += 4) {
      KVC_SCORE_STEP(0, j0)
      KVC_SCORE_STEP(1, j0 + 1)
      KVC_SCORE_STEP(2, j0 + 2)
      KVC_SCORE_STEP(3, j0 + 3)
    }
    if (j0 < nfull) KVC_SCORE_STEP(0, j0)
    if (j0 + 1 < nfull) KVC_SCORE_STEP(1, j0 + 1)
    if (j0 + 2 < nfull) KVC_SCORE_STEP(2, j0 + 2)
    if (nfull > 0) score_reduce_half<MAXMODE>(B, lv, c, G.hi, G.lo, &cb[(nfull - 1) % 3][G.wave][32]);
  }
  for (int j = nfull; j < G.ntiles; ++j) {
    switch (j & 3) {
      case 0: score_masked_step<D, MAXMODE, 0>(G, kh, j, n, causal, voff, qf, lv, c, cb, out); break;
      case 1: score_masked_step<D, MAXMODE, 1>(G, kh, j, n, causal, voff, qf, lv, c, cb, out); break;
      case 2: score_masked_step<D, MAXMODE, 2>(G, kh, j, n, causal, voff, qf, lv, c, cb, out); break;
      default: score_masked_step<D, MAXMODE, 3>(G, kh, j, n, causal, voff, qf, lv, c, cb, out); break;
    }
  }
  const int nt = G.ntiles;
  ring_barrier<D>(0);                        // also: no LDS fill may outlive the block
  if (threadIdx.x < 64) {
    if (nt > 1)
      out[G.k0 + 64 * (nt - 2) + (int)threadIdx.x] = combine4<MAXMODE>(&cb[(nt - 2) % 3][0][threadIdx.x]);
    out[G.k0 + 64 * (nt - 1) + (int)threadIdx.x] = combine4<MAXMODE>(&cb[(nt - 1) % 3][0][threadIdx.x]);
  }
}

// Column reductions of the pass-2 partials [H_q][nRT][Npad].  A block of 4 waves covers 64
// consecutive keys of one KV head (lane = key, so each load reads 256 consecutive bytes); wave
// w adds the row tiles rt = rt0 + w, rt0 + w + 4, ... of every head of the group (rt0 = the
// first tile whose rows see the key), and the four waves' values are combined in LDS in a fixed
// order, so every result is bitwise reproducible.
// SUM: scores[g][t] = sum over the group's heads and row tiles.
__global__ void __launch_bounds__(256)
score_reduce_sum(const float* __restrict__ part, float* __restrict__ scores, int Hkv, int G,
                 int nRT, int64_t N, int64_t Nq, int causal, int64_t Npad) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  const bool ok = t < N;
  int rt0 = 0;
  if (causal && ok) {
    const int64_t rel = t - (N - Nq);                 // first row index that sees t
    rt0 = rel > 0 ? (int)(rel / kRowsPerBlock) : 0;
  }
  float s = 0.f;
  if (ok) {
    // per row tile, the group's heads (at most 16) as independent loads, then added in head order
    const float* p = part + (int64_t)g * G * nRT * Npad + t;
    for (int rt = rt0 + w; rt < nRT; rt += 4) {
      float v[16];
#pragma unroll
      for (int hl = 0; hl < 16; ++hl) v[hl] = hl < G ? p[((int64_t)hl * nRT + rt) * Npad] : 0.f;
#pragma unroll
      for (int hl = 0; hl < 16; ++hl) s += v[hl];
    }
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && ok) scores[(int64_t)g * N + t] = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

// MAX: s+[g][t] = max over the group's heads h of 2^(max over row tiles of part) / ||W_O^h v_t||.
// The per-head maxima of the four waves are combined in LDS (max is exact in any order).
__global__ void __launch_bounds__(256)
score_reduce_max(const float* __restrict__ part, const float* __restrict__ won,
                 float* __restrict__ scores, int Hkv, int G, int nRT, int64_t N,
                 int64_t Nq, int causal, int64_t Npad) {
  __shared__ float red[4][16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  const bool ok = t < N;
  int rt0 = 0;
  if (causal && ok) {
    const int64_t rel = t - (N - Nq);
    rt0 = rel > 0 ? (int)(rel / kRowsPerBlock) : 0;
  }
  float m[16];
#pragma unroll
  for (int hl = 0; hl < 16; ++hl) m[hl] = -INFINITY;
  if (ok) {
    const float* p = part + (int64_t)g * G * nRT * Npad + t;
    for (int rt = rt0 + w; rt < nRT; rt += 4) {
#pragma unroll
      for (int hl = 0; hl < 16; ++hl)
        if (hl < G) m[hl] = fmaxf(m[hl], p[((int64_t)hl * nRT + rt) * Npad]);
    }
  }
#pragma unroll
  for (int hl = 0; hl < 16; ++hl)
    if (hl < G) red[w][hl][lane] = m[hl];
  __syncthreads();
  if (w != 0 || !ok) return;
  float best = 0.f;
  for (int hl = 0; hl < G; ++hl) {
    const int hh = g * G + hl;
    const float m = fmaxf(fmaxf(red[0][hl][lane], red[1][hl][lane]), fmaxf(red[2][hl][lane], red[3][hl][lane]));
    const float num = exp2f(m);
    const float den = won[(int64_t)hh * N + t];
    const float q = (num == 0.f && den == 0.f) ? 0.f : num / den;
    best = fmaxf(best, q);
  }
  scores[(int64_t)g * N + t] = best;
}

// log2 ||h_j||_2 per query row: one wave per row, 16-byte loads, float64 sums of the squares
// (bf16 squares are exact in fp32), a fixed-order wave reduction.
__global__ void __launch_bounds__(256)
hidden_log2_norm(const uint16_t* __restrict__ hidden, float* __restrict__ hlog2, int Dh, int64_t Nq) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= Nq) return;
  const uint16_t* hp = hidden + row * Dh;
  double ss = 0.0;
  if ((Dh & 7) == 0) {
    for (int i = 8 * lane; i < Dh; i += 512) {
      const uint4 w = *reinterpret_cast<const uint4*>(hp + i);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = bf16_bits_to_f32(ww[j] & 0xFFFFu), b = bf16_bits_to_f32(ww[j] >> 16);
        ss += (double)(a * a) + (double)(b * b);
      }
    }
  } else {
    for (int i = lane; i < Dh; i += 64) {
      const float a = bf16_bits_to_f32(hp[i]);
      ss += (double)(a * a);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) hlog2[row] = (float)(0.5 * log2(ss));
}

// Partial Gram matrices of each head's W_O slice on the matrix cores: gp[h][s][c1][c2] = sum over
// rows r of split s of S[r][c1] S[r][c2], S[r][c] = W_O[r][h*d + c] (bf16 products are exact;
// fp32 accumulation).  Rows are staged 64 at a time in LDS transposed, T[c][r], so both operands
// of D[m = c1][n = c2] read 8 consecutive rows of one column with one 16-byte load.  Wave w
// owns output row block c1 in [32w, 32w + 32) (D = 128; for D = 64 waves 2, 3 idle).
template <int D>
__global__ void __launch_bounds__(256)
wo_gram_partial(const uint16_t* __restrict__ w_o, float* __restrict__ gp, int Hq, int Dh,
                int rows_per_split) {
  constexpr int RB = 64;          // rows staged per step
  constexpr int NB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t T[D][RB + 8];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int r0 = s * rows_per_split;
  const int r1 = (r0 + rows_per_split < Dh) ? r0 + rows_per_split : Dh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const bool owner = wave < NB;
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[nb][i] = 0.f;
  const int64_t ld = (int64_t)Hq * D;
  for (int rb = r0; rb < r1; rb += RB) {
    __syncthreads();
    for (int e = threadIdx.x; e < RB * (D / 8); e += 256) {   // 16-byte loads along a row
      const int rr = e / (D / 8), c8 = e % (D / 8);
      const int r = rb + rr;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (r < r1) w = *reinterpret_cast<const uint4*>(w_o + (int64_t)r * ld + (int64_t)h * D + 8 * c8);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        T[8 * c8 + 2 * j][rr] = (uint16_t)(ww[j] & 0xFFFFu);
        T[8 * c8 + 2 * j + 1][rr] = (uint16_t)(ww[j] >> 16);
      }
    }
    __syncthreads();
    if (owner) {
#pragma unroll
      for (int ks = 0; ks < RB / 16; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&T[32 * wave + lo][16 * ks + 8 * hi]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(&T[32 * nb + lo][16 * ks + 8 * hi]));
          acc[nb] = mfma32(a, b, acc[nb]);
        }
      }
    }
  }
  if (!owner) return;
  float* out = gp + ((int64_t)h * gridDim.y + s) * D * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) out[(32 * wave + acc_row(i, hi)) * D + 32 * nb + lo] = acc[nb][i];
}

// Sum the Gram partials over splits in order: gram[h] = sum_s gp[h][s].
__global__ void wo_gram_reduce(const float* __restrict__ gp, float* __restrict__ gram, int Hq,
                               int splits, int DD) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Hq * DD) return;
  int h = (int)(idx / DD);
  int e = (int)(idx % DD);
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += gp[((int64_t)h * splits + sp) * DD + e];
  gram[idx] = s;
}

// ||W_O^h v_t||_2 = sqrt(v_t^T G_h v_t), G_h = W_O^h^T W_O^h, on the matrix cores: for 32 tokens
// at a time Y = G_h V^T (D[m = channel][n = token]; G_h split into bf16 hi + lo, so G_h = hi + lo
// to ~2^-17 and the bf16 values are exact operands), then each lane forms sum_c V[t][c] Y[c][t]
// for its token over its 16 channels per 32-channel block and the two lane halves are added.
// Block = (4 waves x kVnTiles token blocks of 32, query head h); G_h is staged in LDS once.
constexpr int kVnTiles = 4;
template <int D>
__global__ void __launch_bounds__(256)
value_out_norm(const uint16_t* __restrict__ v, const float* __restrict__ gram,
               float* __restrict__ won, int G, int64_t N) {
  constexpr int KS = D / 16, MB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t ghi[D][D + 8];
  __shared__ __attribute__((aligned(16))) uint16_t glo[D][D + 8];
  const int h = blockIdx.y;
  const int g = h / G;
  const float* gh = gram + (int64_t)h * D * D;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const float x = gh[e];
    const __bf16 hb = (__bf16)x;
    const __bf16 lb = (__bf16)(x - (float)hb);
    ghi[e / D][e % D] = __builtin_bit_cast(uint16_t, hb);
    glo[e / D][e % D] = __builtin_bit_cast(uint16_t, lb);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, lo = lane & 31;
  const uint16_t* vh = v + (int64_t)g * N * D;
  for (int tb = 0; tb < kVnTiles; ++tb) {
    const int64_t t0 = ((int64_t)blockIdx.x * kVnTiles + tb) * 128 + 32 * wave;
    if (t0 >= N) break;                       // uniform per wave
    const int64_t t = t0 + lo;
    const bool ok = t < N;
    const uint16_t* vr = vh + (ok ? t : 0) * D;
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 b = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(vr + 16 * ks + 8 * hi) : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 ah = as_bf16x8(*reinterpret_cast<const uint4*>(&ghi[32 * mb + lo][16 * ks + 8 * hi]));
        const bf16x8 al = as_bf16x8(*reinterpret_cast<const uint4*>(&glo[32 * mb + lo][16 * ks + 8 * hi]));
        acc[mb] = mfma32(ah, b, acc[mb]);
        acc[mb] = mfma32(al, b, acc[mb]);
      }
    }
    float qf = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // channels 32 mb + 8 q4 + 4 hi + (0..3) of this lane's token
        const uint2 w = ok ? *reinterpret_cast<const uint2*>(vr + 32 * mb + 8 * q4 + 4 * hi) : make_uint2(0, 0);
        qf = fmaf(bf16_bits_to_f32(w.x & 0xFFFFu), acc[mb][4 * q4 + 0], qf);
        qf = fmaf(bf16_bits_to_f32(w.x >> 16), acc[mb][4 * q4 + 1], qf);
        qf = fmaf(bf16_bits_to_f32(w.y & 0xFFFFu), acc[mb][4 * q4 + 2], qf);
        qf = fmaf(bf16_bits_to_f32(w.y >> 16), acc[mb][4 * q4 + 3], qf);
      }
    qf = half_sum(qf);
    if (hi == 0 && ok) won[(int64_t)h * N + t] = sqrtf(fmaxf(qf, 0.f));
  }
}

}  // namespace

ScorePlan score_plan(const Layer& L) {
  ScorePlan p;
  p.nRT = (int)((L.nq + kRowsPerBlock - 1) / kRowsPerBlock);
  p.Npad = ((L.n + 255) / 256) * 256;
  auto kend = [&](int rt) -> int64_t {
    if (!L.causal) return L.n;
    int64_t last = (int64_t)(rt + 1) * kRowsPerBlock;
    if (last > L.nq) last = L.nq;
    int64_t e = L.n - L.nq + last;
    return e < L.n ? e : L.n;
  };
  int64_t kmax = 0;
  for (int rt = 0; rt < p.nRT; ++rt) kmax = kend(rt) > kmax ? kend(rt) : kmax;
  // With >= 1024 (head, row tile) items one chunk per item balances well (longest items run
  // first); otherwise split the keys into chunks (<= 4096, >= 512 keys) until there are
  // >= 2048 non-empty items.
  int KC = (int)(((kmax + 63) / 64) * 64);
  if ((int64_t)p.nRT * L.hq < 1024) {
    KC = 4096;
    for (; KC > 512; KC /= 2) {
      int64_t items = 0;
      for (int rt = 0; rt < p.nRT; ++rt) items += (kend(rt) + KC - 1) / KC;
      if (items * L.hq >= 2048) break;
    }
  }
  p.KC = KC;
  p.maxCh = (int)((kmax + KC - 1) / KC);
  p.W = (int64_t)L.hkv * p.nRT * p.maxCh * L.G;
  return p;
}

static Decomp decomp_of(const Layer& L, const ScorePlan& p) {
  Decomp d;
  d.G = L.G;
  d.nRT = p.nRT;
  d.maxCh = p.maxCh;
  d.KC = p.KC;
  d.W = p.W;
  return d;
}

static unsigned grid_of(const ScorePlan& p) {
  return (unsigned)(((p.W + kXcds - 1) / kXcds) * kXcds);
}

static constexpr int kGramSplits = 14;

size_t lse_ws_bytes(const Layer& L) {
  const ScorePlan p = score_plan(L);
  WsPlan w;
  w.take((size_t)L.hq * L.nq * p.maxCh * sizeof(float2));
  return w.off;
}

size_t score_ws_bytes(const Layer& L, int mode, int hidden_dim) {
  (void)hidden_dim;
  const ScorePlan p = score_plan(L);
  WsPlan w;
  w.take((size_t)L.hq * p.nRT * p.Npad * sizeof(float));
  if (mode == KVC_SCORE_MAX) {
    w.take((size_t)L.nq * sizeof(float));                                  // log2 ||h||
    w.take((size_t)L.hq * kGramSplits * L.d * L.d * sizeof(float));        // gram partials
    w.take((size_t)L.hq * L.d * L.d * sizeof(float));                      // gram
    w.take((size_t)L.hq * L.n * sizeof(float));                            // ||W_O^h v||
  }
  return w.off;
}

hipError_t launch_row_lse(const Layer& L, const uint16_t* q, const uint16_t* k, float* lse,
                          char* ws, hipStream_t s, int tag) {
  const ScorePlan p = score_plan(L);
  if (p.W >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const Decomp dc = decomp_of(L, p);
  WsPlan w;
  float2* part = reinterpret_cast<float2*>(ws + w.take((size_t)L.hq * L.nq * p.maxCh * sizeof(float2)));
  if (L.d == 128 && tag == 0)
    lse_partial<128, 0><<<grid_of(p), kThreads, 0, s>>>(q, k, part, lse, dc, L.n, L.nq, L.causal, L.c_log2);
  else if (L.d == 128)
    lse_partial<128, 1><<<grid_of(p), kThreads, 0, s>>>(q, k, part, lse, dc, L.n, L.nq, L.causal, L.c_log2);
  else if (tag == 0)
    lse_partial<64, 0><<<grid_of(p), kThreads, 0, s>>>(q, k, part, lse, dc, L.n, L.nq, L.causal, L.c_log2);
  else
    lse_partial<64, 1><<<grid_of(p), kThreads, 0, s>>>(q, k, part, lse, dc, L.n, L.nq, L.causal, L.c_log2);
  if (p.maxCh > 1) {
    const int64_t rows = (int64_t)L.hq * L.nq;
    lse_combine<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(part, lse, L.hq, L.n, L.nq, L.causal, p.KC, p.maxCh);
  }
  return hipGetLastError();
}

hipError_t launch_score(const Layer& L, int mode, const uint16_t* q, const uint16_t* k,
                        const float* lse, const uint16_t* hidden, const uint16_t* w_o,
                        const uint16_t* v, int hidden_dim, float* scores, char* ws,
                        hipStream_t s) {
  const ScorePlan p = score_plan(L);
  if (p.W >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const Decomp dc = decomp_of(L, p);
  const bool mx = (mode == KVC_SCORE_MAX);
  WsPlan w;
  float* part = reinterpret_cast<float*>(ws + w.take((size_t)L.hq * p.nRT * p.Npad * sizeof(float)));
  float* hlog2 = nullptr;
  float* won = nullptr;
  if (mx) {
    hlog2 = reinterpret_cast<float*>(ws + w.take((size_t)L.nq * sizeof(float)));
    float* gp = reinterpret_cast<float*>(ws + w.take((size_t)L.hq * kGramSplits * L.d * L.d * sizeof(float)));
    float* gram = reinterpret_cast<float*>(ws + w.take((size_t)L.hq * L.d * L.d * sizeof(float)));
    won = reinterpret_cast<float*>(ws + w.take((size_t)L.hq * L.n * sizeof(float)));
    hidden_log2_norm<<<(unsigned)((L.nq + 3) / 4), 256, 0, s>>>(hidden, hlog2, hidden_dim, L.nq);
    const int rps = (hidden_dim + kGramSplits - 1) / kGramSplits;
    dim3 gg((unsigned)L.hq, kGramSplits);
    if (L.d == 128)
      wo_gram_partial<128><<<gg, 256, 0, s>>>(w_o, gp, L.hq, hidden_dim, rps);
    else
      wo_gram_partial<64><<<gg, 256, 0, s>>>(w_o, gp, L.hq, hidden_dim, rps);
    const int64_t ng = (int64_t)L.hq * L.d * L.d;
    wo_gram_reduce<<<(unsigned)((ng + 255) / 256), 256, 0, s>>>(gp, gram, L.hq, kGramSplits, L.d * L.d);
    dim3 gv((unsigned)((L.n + 128 * kVnTiles - 1) / (128 * kVnTiles)), (unsigned)L.hq);
    if (L.d == 128)
      value_out_norm<128><<<gv, 256, 0, s>>>(v, gram, won, L.G, L.n);
    else
      value_out_norm<64><<<gv, 256, 0, s>>>(v, gram, won, L.G, L.n);
  }
  const unsigned grid = grid_of(p);
  if (L.d == 128) {
    if (mx)
      score_partial<128, true><<<grid, kThreads, 0, s>>>(q, k, lse, hlog2, part, dc, L.n, L.nq, L.causal, L.c_log2, p.Npad);
    else
      score_partial<128, false><<<grid, kThreads, 0, s>>>(q, k, lse, nullptr, part, dc, L.n, L.nq, L.causal, L.c_log2, p.Npad);
  } else {
    if (mx)
      score_partial<64, true><<<grid, kThreads, 0, s>>>(q, k, lse, hlog2, part, dc, L.n, L.nq, L.causal, L.c_log2, p.Npad);
    else
      score_partial<64, false><<<grid, kThreads, 0, s>>>(q, k, lse, nullptr, part, dc, L.n, L.nq, L.causal, L.c_log2, p.Npad);
  }
  const dim3 gr((unsigned)((L.n + 63) / 64), (unsigned)L.hkv);
  if (mx)
    score_reduce_max<<<gr, 256, 0, s>>>(part, won, scores, L.hkv, L.G, p.nRT, L.n, L.nq, L.causal, p.Npad);
  else
    score_reduce_sum<<<gr, 256, 0, s>>>(part, scores, L.hkv, L.G, p.nRT, L.n, L.nq, L.causal, p.Npad);
  return hipGetLastError();
}

}  // namespace kvc
