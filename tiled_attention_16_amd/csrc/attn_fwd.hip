// Fused scaled-dot-product attention forward for MI355X (gfx950, CDNA4).
//
// Pages cited:
//   [PT2CUDA]  aiknowledge.cn, "4.5 注意力优化实战：从PyTorch到CUDA的完整流程".
//   [MEMWALL]  codechina.net, "GPU 内存墙 ... FlashAttention" article.
//   [PROFILE3] "Profiling in PyTorch (part 3): Attention is all you profile".
//
// What one launch computes is stated in include/attn.h. How:
//
// Work decomposition ([MEMWALL] §2.2, outer loop over query blocks, inner loop
// over key/value blocks): one workgroup of 4 wave64s owns a 128-row query tile
// of one (batch, head); each wave owns 32 of those rows for the whole launch.
// The workgroup walks the 64-key K/V tiles its rows can see; causal tiles above
// the diagonal and tiles past the batch's valid key length are never visited,
// and a wave skips the arithmetic of tiles that lie wholly above its own rows.
//
// Data movement ([MEMWALL] §4.3 double buffering; [PT2CUDA] step 5): K and V
// tiles go from global memory straight into LDS with the gfx950 16-byte
// global_load_lds copy, no register staging. K and V each have two LDS stages;
// the copies for K tile j+2 and V tile j+1 are in flight while tile j is
// computed, and one barrier per tile both publishes the landed tiles and frees
// the stages read in the previous step. Inside a stage, row r's 16-byte chunk c
// sits at chunk position c ^ swz(r): the MFMA operand reads (ds_read_b128 for K,
// the transposing ds_read_b64_tr_b16 for V) then touch distinct banks.
//
// Per K/V tile, per wave (the online softmax of [PT2CUDA] step 3.1 and
// [MEMWALL] §3.2, in the exp2 domain with c = |scale| * log2(e)):
//   S^T = K Q^T on MFMA 32x32x16 bf16 -> fp32. Computing the transpose puts one
//         query row in each lane (32 keys per lane, the other 32 keys of the
//         tile in lane ^ 32): the row max is an in-register max plus one
//         permlane32 swap, and the row sum needs no cross-lane step until the
//         very end.
//   mask  only on tiles that cross the causal diagonal, the valid key length or
//         the masked leading rows: the score becomes -inf.
//   m     running max of S*c per row. It is raised only when the tile's max
//         exceeds it by more than kTau; otherwise the stale max stays the
//         exponent's subtrahend. O / l does not depend on the subtrahend, so
//         this is the pages' recurrence in exact arithmetic; the exponentials
//         stay below 2^kTau. When m rises, l and O are scaled by
//         alpha = exp2(m_old - m_new) (O lazily, before the next P V).
//   P     = exp2(S*c - m) in fp32, summed into l in fp32, then rounded to bf16.
//         Its accumulator layout is already the B operand layout of the next
//         MFMA, so P never leaves registers.
//   O^T  += V^T P^T on MFMA 32x32x16 bf16 -> fp32, V^T read from LDS with the
//         transposing read.
// The loop is software pipelined inside each wave: while the MFMA unit
// computes S for tile j+1, the VALU exponentiates tile j; while it computes
// O += P V for tile j, the VALU takes the row max of tile j+1 and forms
// S*c - m. Two such waves share each SIMD.
// Epilogue ([PT2CUDA] step 4.1, one division per row at the end): O = O / l
// (0 when l = 0), LSE = ln2 * (m + log2 l) (-inf when l = 0), bf16 store.
//
// gfx950 MFMA 32x32x16 bf16 lane layouts:
//   A (M x K): lane L holds row L%32, k = 8*(L/32) + 0..7;
//   B (K x N): lane L holds column L%32, the same k;
//   C (M x N): lane L reg r holds row 8*(r/4) + 4*(L/32) + r%4, column L%32.
// ds_read_b64_tr_b16, per 16-lane group: lane 4j+k supplies 4 consecutive
// elements of row j; afterwards lane i holds element i of each of the 4 rows.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <type_traits>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kBN = 64;        // keys per K/V tile
constexpr int kWaves = 8;      // wave64s per workgroup (two per SIMD), 32 query rows each
constexpr int kStages = 4;     // LDS ring depth for K and V tiles: three tiles of copy lookahead
constexpr int kBM = 32 * kWaves;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;   // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
struct Tile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kBytes = kBN * kRowBytes;            // one K or V stage
  static constexpr int kLds = 2 * kStages * kBytes;         // K stages, then V stages
  static constexpr int kCopies = kBytes / 1024;             // 1 KB wave copies per stage
  static constexpr int kCopiesPerWave = kCopies / kWaves;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kLanesPerRow = 64 / kRowsPerCopy;
  static_assert(kCopies % kWaves == 0, "copies must split evenly over the waves");
  static_assert(kLds <= 160 * 1024, "the stages must fit the 160 KB LDS of a CU");
};

// Chunk position of 16-byte chunk c of row r is c ^ swz(r). For D = 128 a row
// is 256 bytes (one sweep of the banks): 16 consecutive rows get 16 distinct
// swizzles, and 4 consecutive rows x 2 adjacent chunks stay distinct too. For
// D = 64 two rows share a sweep, so row bit 0 picks the half and bits 1-3 the
// swizzle.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);   // v_cvt_pk_bf16_f32
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float lane_swap_max(float x) {
  // permlane32_swap(x, x) hands every lane both its own value and its partner's
  // (lane ^ 32), one in each result.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most N of this wave's copies are still in flight (copies
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int N_q, int N_k, float c, int neg_scale,
    int causal, const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_qt,
    int n_wg) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[T::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int grp = wave >> 2;   // waves w and w+4 share a SIMD: one of each group
  const int hf = lane >> 5;

  // ---- work decomposition: blockIdx -> (batch*head, pair of query tiles) ----
  // Consecutive workgroup ids are dealt round-robin over the 8 XCDs; regroup so
  // that each XCD gets a contiguous range of (head, tile) pairs and the K/V of a
  // head stay in one XCD's L2.
  int lin = blockIdx.x;
  if ((n_wg & 7) == 0) lin = (lin & 7) * (n_wg >> 3) + (lin >> 3);
  const int n_pairs = (n_qt + 1) / 2;
  const int bh = lin / n_pairs;
  const int pr = lin - bh * n_pairs;
  const int b = bh / H;
  const char* kg = (const char*)(K + (size_t)bh * N_k * D);
  const char* vg = (const char*)(V + (size_t)bh * N_k * D);

  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);

  // ---- K/V tile copies: global -> LDS, 1 KB per wave instruction ----
  // Copy q of this wave fills LDS bytes [1024*qi, 1024*qi + 1024) of a stage,
  // qi = wave * kCopiesPerWave + q: lane L lands at byte 16*L, which is row
  // qi*kRowsPerCopy + L / kLanesPerRow, chunk position L % kLanesPerRow, so it
  // fetches logical chunk (position ^ swz(row)) of that row.
  auto cp_row = [&](int q) __attribute__((always_inline)) {
    return (wave * T::kCopiesPerWave + q) * T::kRowsPerCopy + lane / T::kLanesPerRow;
  };
  int cp_off[T::kCopiesPerWave];
#pragma unroll
  for (int q = 0; q < T::kCopiesPerWave; ++q) {
    const int r = cp_row(q);
    cp_off[q] = r * T::kRowBytes + (((lane % T::kLanesPerRow) ^ swz<D>(r)) << 4);
  }
  // Copy the 64 rows starting at key k0 of a head's K or V into stage dst.
  // Rows outside [0, kv) are never read: those lanes fetch a clamped row whose
  // data the mask ignores (or that is multiplied by a zero probability).
  auto copy_tile = [&](const char* src, int k0, const char* dst) __attribute__((always_inline)) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)dst +
                          wave * T::kCopiesPerWave * 1024;
    const bool ragged = k0 < 0 || k0 + kBN > kv;
    const char* base = ragged ? src : src + (ptrdiff_t)k0 * T::kRowBytes;
    // (readfirstlane returns a signed int: widen through uint32_t so the low
    // half is zero-extended, never sign-extended into the high half)
    const uint32_t base_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
    const uint32_t base_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)base >> 32));
    const uint64_t sbase = ((uint64_t)base_hi << 32) | (uint64_t)base_lo;
#pragma unroll
    for (int q = 0; q < T::kCopiesPerWave; ++q) {
      uint32_t voff = (uint32_t)cp_off[q];
      if (ragged) {
        const int key = min(max(k0 + cp_row(q), 0), kv - 1);
        voff += (uint32_t)((key - cp_row(q)) * T::kRowBytes);
      }
      // The copy is issued as inline assembly so that the compiler does not
      // treat it as a pending write to every LDS address (it would then wait
      // for it before each LDS read); completion is awaited explicitly with
      // wait_copies() before the barrier that publishes the tile.
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(__builtin_amdgcn_readfirstlane(lds0 + q * 1024)), "v"(voff), "s"(sbase)
                   : "memory", "m0");
    }
  };
  // Stage st: K rows at kst(st), V rows at vst(st).
  auto kst = [&](int st) __attribute__((always_inline)) { return (const char*)smem + st * T::kBytes; };
  auto vst = [&](int st) __attribute__((always_inline)) { return (const char*)smem + (kStages + st) * T::kBytes; };

  // ---- per-lane LDS offsets of the MFMA operand reads ----
  // K (A operand of S^T = K Q^T): lane L reads row L%32 of a 32-key half
  // tile, logical chunk 2*kc + L/32, at byte r*kRowBytes + ((2kc + L/32) ^
  // swz(r))*16. The swizzle only flips chunk bits, so the offset for chunk
  // pair kc is k_off0 ^ (32*kc).
  // V (A operand of O^T += V^T P^T, via the transposing read): 16-key chunk cc,
  // half hi: lane L of group g = L/16 supplies row 16*cc + 8*hi + 4*(L/32) +
  // (L%16)/4, columns 32*db + 16*(g%2) + 4*(L%4) .. +3. After the transpose,
  // lane L holds column 32*db + L%32 of keys 16*cc + 8*hi + 4*(L/32) + 0..3,
  // which pairs with P's registers 8*(cc%2) + 4*hi + 0..3 of the half tile.
  // Its offset is v_off0 ^ (hi*(8*kRowBytes + 16)) ^ (64*db) (row +8 flips
  // swizzle bit 0), plus 16*cc rows as an immediate.
  // Every base these are added to is a multiple of 16 rows, so base + (off ^ x)
  // == (base + off) ^ x and the bases stay immediate offsets.
  int k_off0, v_off0;
  {
    const int r = lane & 31;
    k_off0 = r * T::kRowBytes + ((hf ^ swz<D>(r)) << 4);
    const int g = lane >> 4;
    const int rv = 4 * hf + ((lane & 15) >> 2);
    const int byte = 32 * (g & 1) + 8 * (lane & 3);
    v_off0 = rv * T::kRowBytes + (((byte >> 4) ^ swz<D>(rv)) << 4) + (byte & 15);
  }

  // A workgroup owns the pair of query tiles (n_qt-1-pr, pr): under a causal
  // mask their key counts add up to the same total for every pair, so all
  // workgroups carry equal work and none is left running alone at the end.
  // The tile with more keys goes first.
  const int n_mine = (n_qt - 1 - pr != pr) ? 2 : 1;
#pragma nounroll
  for (int it = 0; it < n_mine; ++it) {
  const int qt = it == 0 ? n_qt - 1 - pr : pr;
  const int q0 = qt * kBM;
  const int q_end = min(q0 + kBM, N_q);
  int kv_end = kv;                                 // keys this workgroup can see
  if (causal) kv_end = min(kv_end, q_end);
  if (qs >= q_end) kv_end = 0;                     // every row of the tile is masked

  const int row_lo = q0 + 32 * wave;               // this wave's rows: row_lo .. row_lo + 31
  const int row_hi = min(row_lo + 31, N_q - 1);
  const bool wave_live = row_lo < N_q && row_hi >= qs;
  const int my_row = row_lo + (lane & 31);
  const size_t q_base = (size_t)bh * N_q * D;

  // 32-key half tiles h (keys 32h .. 32h+31): nh_wg for the workgroup, nh (a
  // prefix) for this wave.
  const int nh_wg = (kv_end + 31) / 32;
  int nh = wave_live ? nh_wg : 0;
  if (causal) nh = min(nh, row_hi / 32 + 1);

  // ---- Q rows -> VGPRs as the B operand of S^T = K Q^T ----
  bf16x8 qreg[D / 16];
  {
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;   // negative scale: negate Q exactly
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (my_row < N_q) x = *(const u32x4*)(Q + q_base + (size_t)my_row * D + kc * 16 + hf * 8);
      x ^= flip;
      qreg[kc] = as_bf16x8(x);
    }
  }

  f32x16 o_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o_acc[db] = (f32x16){};
  float m_run = -INFINITY;   // running max of S*c for this lane's row (same in lane ^ 32)
  float l_run = 0.f;         // partial running sum over this lane's half of the keys
  f32x16 s = {};             // S^T of the current half tile (one query row per lane)
  bf16x8 pb[2] = {};         // P of the previous half tile, the B operand of P V

  // Key j is allowed for this lane's row iff j <= klim (klim folds the valid
  // length, the causal limit and the masked leading rows into one bound).
  const int klim = my_row < qs ? -1 : min(kv - 1, causal ? my_row : 0x7fffffff);
  // masking is needed only where the half tile crosses that bound for some row
  auto need_mask = [&](int h) __attribute__((always_inline)) {
    const int k0 = h * 32;
    return (k0 + 31 >= kv) || (causal && k0 + 31 > row_lo) || (row_lo < qs);
  };

  // K tile t holds keys 64t .. 64t+63 (K halves 2t, 2t+1); V tile t holds keys
  // 64t-32 .. 64t+31 (V halves 2t-1, 2t). Both live in stage t % kStages.
  // K half h: stage (h/2) % kStages, row 32*(h%2); V half h: stage
  // ((h+1)/2) % kStages, row 32*(1 - h%2). Callers pass h modulo 2*kStages as
  // a compile-time constant, so every LDS address is a per-lane offset plus an
  // immediate.
  auto k_half = [&](auto hm) __attribute__((always_inline)) {
    constexpr int h = decltype(hm)::value;
    return kst((h >> 1) % kStages) + (h & 1) * 32 * T::kRowBytes;
  };
  auto v_half = [&](auto hm) __attribute__((always_inline)) {
    constexpr int h = decltype(hm)::value;
    return vst(((h + 1) >> 1) % kStages) + (~h & 1) * 32 * T::kRowBytes;
  };

  // Operands of cluster C_h: K of half h (A operand of S^T = K Q^T) and V of
  // half h-1 (A operand of O^T += V^T P^T). They are read from LDS one cluster
  // ahead, during the softmax cluster of the same wave, so the MFMA cluster
  // itself never waits on LDS and the reads of one group overlap the other
  // group's MFMAs.
  u32x4 ka[D / 16];
  bf16x8 va[2][D / 32];
  auto load_ops = [&](auto hm) __attribute__((always_inline)) {
    constexpr int h = decltype(hm)::value;   // half index modulo 2*kStages
    const char* kb = k_half(std::integral_constant<int, h>{});
    const char* vb = v_half(std::integral_constant<int, (h + 2 * kStages - 1) % (2 * kStages)>{});
    // (re-derive the offsets here instead of keeping 16 of them live)
    int ko = k_off0, vo = v_off0;
    asm volatile("" : "+v"(ko), "+v"(vo));
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) ka[kc] = *(const lds_u32x4*)(kb + (ko ^ (32 * kc)));
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int off_lo = vo ^ (64 * db);
      const int off_hi = off_lo ^ (8 * T::kRowBytes + 16);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const char* p0 = vb + 16 * cc * T::kRowBytes;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + off_lo));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + off_hi));
        va[cc][db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  // Cluster C_h (MFMA): S of half h (into s) and O += P V of half h-1 (P from
  // the previous softmax cluster; zero before the first).
  auto cluster_c = [&]() __attribute__((always_inline)) {
    s = (f32x16){};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kc]), qreg[kc], s, 0, 0, 0);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cc][db], pb[cc], o_acc[db], 0, 0, 0);
  };

  // Cluster S_h (VALU): the online softmax of half h on s.
  auto cluster_s = [&](int h) __attribute__((always_inline)) {
    if (need_mask(h)) {
      const int lim = klim - h * 32 - 4 * hf;   // key offset within the half tile must be <= lim
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3)) <= lim ? s[r] : -INFINITY;
    }
    const float a0 = fmaxf(fmaxf(s[0], s[1]), s[2]), a1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float a2 = fmaxf(fmaxf(s[6], s[7]), s[8]), a3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float a4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
    const float mx = lane_swap_max(fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), s[15])));
    const float tmax = mx * c;   // c > 0, so -inf stays -inf
    const bool grow = tmax > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // raise the subtrahend; rescale l and O (O holds P V up to half h-1)
      const float m_new = grow ? tmax : m_run;
      const float a = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;   // m_run = -inf gives 0
      m_run = m_new;
      l_run *= a;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o_acc[db] *= a;
    }
    const float msub = (m_run == -INFINITY) ? 0.f : m_run;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -msub));
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])) +
             (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 w = {pack2(p[8 * u + 0], p[8 * u + 1]), pack2(p[8 * u + 2], p[8 * u + 3]),
                       pack2(p[8 * u + 4], p[8 * u + 5]), pack2(p[8 * u + 6], p[8 * u + 7])};
      pb[u] = as_bf16x8(w);
    }
  };

  // Ping-pong: every SIMD holds one wave of each group. In iteration j group 0
  // runs C_j then S_j, group 1 runs S_{j-1} then C_j, with a workgroup barrier
  // between the halves ("slots" 2j and 2j+1), so one wave of each SIMD feeds
  // the MFMA unit while the other works on the VALU and reads the operands of
  // its next MFMA cluster from LDS. Tile t (K halves 2t, 2t+1; V halves 2t-1,
  // 2t) is read in slots 4t-1 .. 4t+2, so the workgroup waits for tile t at the
  // barrier before slot 4t-1 and, once every wave has passed that barrier
  // (the last reads of tile t-1 were in slot 4t-2), copies tile t+3 into tile
  // t-1's stage. Copies are issued for every tile step, also past the last
  // tile (clamped rows), so that the number in flight, and with it every wait
  // count, is the same each time.
  constexpr int kC = 2 * T::kCopiesPerWave;   // copies per wave per K+V tile
  auto copy_tiles = [&](int t) __attribute__((always_inline)) {
    const int st = t & (kStages - 1);
    copy_tile(kg, t * kBN, kst(st));
    copy_tile(vg, t * kBN - 32, vst(st));
  };
  auto slot_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nh_wg > 0) {
    if (it > 0) __syncthreads();   // every wave is done reading the previous tile's stages
#pragma unroll
    for (int t = 0; t < kStages - 1; ++t) copy_tiles(t);
    wait_copies<(kStages - 2) * kC>();
    __syncthreads();   // tile 0 has landed
    copy_tiles(kStages - 1);
    // One loop per group (the group decides the order of the clusters); both
    // pass the same barriers in the same order.
    auto run = [&](auto gm) __attribute__((always_inline)) {
      constexpr int G = decltype(gm)::value;
      // The operand reads of the next MFMA cluster are issued unconditionally
      // (always inside LDS) at the start of the wave's softmax slot, so the LDS
      // works while the VALU does the softmax.
      auto iter = [&](auto jm, int j) __attribute__((always_inline)) {
        constexpr int J = decltype(jm)::value;   // j % (2 * kStages)
        constexpr int J1 = (J + 1) % (2 * kStages);
        slot_barrier();
        if constexpr (G == 0) {
          if (j <= nh) cluster_c();
        } else {
          load_ops(jm);
          if (j >= 1 && j - 1 < nh) cluster_s(j - 1);
        }
        if constexpr (J & 1) {
          wait_copies<(kStages - 2) * kC>();
          __syncthreads();   // tile (j+1)/2 has landed; tile (j+1)/2 - 1 is no longer read
          copy_tiles((j + 1) / 2 + kStages - 1);
        } else {
          slot_barrier();
        }
        if constexpr (G == 0) {
          load_ops(std::integral_constant<int, J1>{});
          if (j < nh) cluster_s(j);
        } else {
          if (j <= nh) cluster_c();
        }
      };
      if constexpr (G == 0) load_ops(std::integral_constant<int, 0>{});
      static_assert(kStages == 4, "the loop below is unrolled over 2 * kStages half tiles");
      for (int j0 = 0; j0 <= nh_wg; j0 += 8) {
        iter(std::integral_constant<int, 0>{}, j0);
        if (j0 + 1 > nh_wg) break;
        iter(std::integral_constant<int, 1>{}, j0 + 1);
        if (j0 + 2 > nh_wg) break;
        iter(std::integral_constant<int, 2>{}, j0 + 2);
        if (j0 + 3 > nh_wg) break;
        iter(std::integral_constant<int, 3>{}, j0 + 3);
        if (j0 + 4 > nh_wg) break;
        iter(std::integral_constant<int, 4>{}, j0 + 4);
        if (j0 + 5 > nh_wg) break;
        iter(std::integral_constant<int, 5>{}, j0 + 5);
        if (j0 + 6 > nh_wg) break;
        iter(std::integral_constant<int, 6>{}, j0 + 6);
        if (j0 + 7 > nh_wg) break;
        iter(std::integral_constant<int, 7>{}, j0 + 7);
      }
    };
    if (grp == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
    wait_copies<0>();   // no copy may still be writing LDS when the next tile (or wave) starts
  }

  // ---- epilogue: O / l, LSE, bf16 store ----
  if (my_row < N_q) {
    const float l_tot = lane_swap_add(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = O + q_base + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack2(o_acc[db][4 * g + 0] * inv, o_acc[db][4 * g + 1] * inv),
                         pack2(o_acc[db][4 * g + 2] * inv, o_acc[db][4 * g + 3] * inv)};
        *(u32x2*)(orow + 32 * db + 8 * g + 4 * hf) = w;
      }
    }
    if (LSE && lane < 32)
      LSE[(size_t)bh * N_q + my_row] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
  }   // tiles of the pair
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                        int N_q, int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                        const int32_t* q_start, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if ((long long)B * H * N_q == 0) return ATTN_OK;
  if (!q || !o) return ATTN_ERR_NULL;
  if (N_k > 0 && (!k || !v)) return ATTN_ERR_NULL;
  const long long n_qt = (N_q + kBM - 1) / kBM;
  const long long n_wg = (long long)B * H * ((n_qt + 1) / 2);   // one workgroup per pair of query tiles
  if (n_wg > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((long long)B * H > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const size_t q_bytes = (size_t)B * H * N_q * d * 2;
  const size_t k_bytes = (size_t)B * H * N_k * d * 2;
  const size_t lse_bytes = (size_t)B * H * N_q * 4;
  if (((uintptr_t)q | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if (N_k > 0 && (((uintptr_t)k | (uintptr_t)v) & 15)) return ATTN_ERR_ALIGN;
  if (lse && ((uintptr_t)lse & 3)) return ATTN_ERR_ALIGN;
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, k_bytes) || overlaps(o, q_bytes, v, k_bytes))
    return ATTN_ERR_ALIAS;
  if (lse && (overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, k_bytes) ||
              overlaps(lse, lse_bytes, v, k_bytes) || overlaps(lse, lse_bytes, o, q_bytes)))
    return ATTN_ERR_ALIAS;

  // exp2 domain: exp(x) = exp2(x * log2 e). A zero scale is replaced by a tiny
  // positive one: every exponent then rounds to exactly 1 in fp32 (uniform
  // weights, as with scale 0), and 0 * -inf never arises.
  float c = fabsf(scale) * 1.44269504088896340736f;
  if (!(c >= 1e-30f)) c = 1e-30f;
  const int neg = scale < 0.f ? 1 : 0;

  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  const uint16_t* vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)o;
  int causal01 = causal ? 1 : 0, n_qt_i = (int)n_qt, n_wg_i = (int)n_wg;
  void* args[] = {(void*)&qp, (void*)&kp, (void*)&vp, (void*)&op, (void*)&lse, (void*)&H, (void*)&N_q,
                  (void*)&N_k, (void*)&c, (void*)&neg, (void*)&causal01,
                  (void*)&seqlens_k, (void*)&q_start, (void*)&n_qt_i, (void*)&n_wg_i};
  const void* fn = d == 128 ? (const void*)attn_fwd_kernel<128> : (const void*)attn_fwd_kernel<64>;
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)n_wg), dim3(kThreads), args, 0, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid or too large shape";
    case ATTN_ERR_HEAD_DIM: return "head dim must be 64 or 128";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_ALIGN: return "misaligned pointer (q, k, v, o need 16 bytes, lse 4)";
    case ATTN_ERR_ALIAS: return "output overlaps an input or the other output";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int attn_version(void) { return 100; }
