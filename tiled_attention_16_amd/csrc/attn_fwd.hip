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
// The workgroup walks the 64-key K/V tiles its rows can see. Causal tiles above
// the diagonal are never visited; tiles past the batch's valid key length are
// never visited.
//
// Per K/V tile, per wave (the online softmax of [PT2CUDA] step 3.1 and
// [MEMWALL] §3.2, in the exp2 domain with c = |scale| * log2(e)):
//   S^T = K Q^T on MFMA 32x32x16 bf16 -> fp32. Computing the transpose puts one
//         query row in each lane (32 keys per lane, the other 32 keys of the
//         tile in lane ^ 32), so the row max is an in-register max plus one
//         permlane32 swap, and the row sum needs no cross-lane step until the
//         very end.
//   mask  only on tiles that cross the causal diagonal, the valid key length or
//         the masked leading rows: the score becomes -inf.
//   m, l  running max (exp2 domain) and per-lane partial running sum. The
//         rescale of l and O by alpha = exp2(m_old - m_new) is taken only when
//         some row's max grew by more than kTau; otherwise the stale max keeps
//         serving as the subtrahend. O / l is unchanged by the choice of
//         subtrahend, so this is exactly the pages' recurrence in exact
//         arithmetic; the exponentials stay below 2^kTau, far from overflow.
//   P     = exp2(S*c - m) in fp32, summed into l in fp32, then rounded to bf16.
//         Its accumulator layout is already the B operand layout of the next
//         MFMA, so P never leaves registers.
//   O^T  += V^T P^T on MFMA 32x32x16 bf16 -> fp32, V^T fetched from LDS with
//         the gfx950 transposing read ds_read_b64_tr_b16.
// Epilogue ([PT2CUDA] step 4.1, one division per row at the end): O = O / l
// (0 when l = 0), LSE = ln2 * (m + log2 l) (-inf when l = 0), bf16 store.
//
// Data movement: Q is read once into VGPRs as MFMA operands. K and V tiles are
// prefetched into VGPRs one tile ahead and written into one of two LDS stages
// (double buffering, [MEMWALL] §4.3; [PT2CUDA] step 5), one barrier per tile.
// LDS rows are padded (K: +16 B, V: 352-byte stride) so that the K operand reads
// and the transposing V reads hit distinct banks.
//
// Everything is written for wave64 and the gfx950 MFMA lane layouts:
//   32x32x16 bf16, A (M x K): lane L holds row L%32, k = 8*(L/32) + 0..7;
//   B (K x N): lane L holds column L%32, the same k;
//   C (M x N): lane L reg r holds row 8*(r/4) + 4*(L/32) + r%4, column L%32.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

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

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kWaves = 4;      // wave64s per workgroup, 32 query rows each
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;   // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kKStride = 2 * D + 16;            // LDS bytes per K row
  static constexpr int kVStride = 352;                   // LDS bytes per V row (= 96 mod 256)
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kStage = kKBytes + kBN * kVStride;
  static constexpr int kLds = 2 * kStage;
  static constexpr int kRowsPerPass = kThreads / kChunks;  // rows one pass of 256 threads covers
  static constexpr int kPasses = kBN / kRowsPerPass;
  static_assert(kVStride >= 2 * D, "V row must fit its stride");
  static_assert(kLds <= 80 * 1024, "two workgroups must fit the 160 KB LDS of a CU");
};

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

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int N_q, int N_k, float c, int neg_scale,
    int causal, const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_qt,
    int n_wg) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[T::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- work decomposition: blockIdx -> (batch*head, query tile) ----
  // Consecutive workgroup ids are dealt round-robin over the 8 XCDs; regroup so
  // that each XCD gets a contiguous range of (head, tile) pairs and the K/V of a
  // head stay in one XCD's L2. Within a head, the tile with the most keys
  // (the last one, under a causal mask) starts first.
  int lin = blockIdx.x;
  if ((n_wg & 7) == 0) lin = (lin & 7) * (n_wg >> 3) + (lin >> 3);
  const int bh = lin / n_qt;
  const int qt = n_qt - 1 - (lin - bh * n_qt);
  const int b = bh / H;
  const int q0 = qt * kBM;

  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);

  int kv_end = kv;                                 // keys this workgroup can see
  if (causal) kv_end = min(kv_end, min(q0 + kBM, N_q));
  if (qs >= min(q0 + kBM, N_q)) kv_end = 0;         // every row of the tile is masked
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  const int row_lo = q0 + 32 * wave;                // this wave's rows: row_lo .. row_lo + 31
  const int row_hi = row_lo + 31;
  const bool wave_live = row_lo < N_q && row_hi >= qs;
  const int my_row = row_lo + (lane & 31);

  const size_t q_base = (size_t)bh * N_q * D;
  const size_t kv_base = (size_t)bh * N_k * D;

  // ---- Q tile -> VGPRs as the B operand of S^T = K Q^T ----
  bf16x8 qreg[D / 16];
  {
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;   // negative scale: negate Q exactly
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (my_row < N_q)
        x = *(const u32x4*)(Q + q_base + (size_t)my_row * D + kc * 16 + (lane >> 5) * 8);
      x ^= flip;
      qreg[kc] = as_bf16x8(x);
    }
  }

  // ---- K/V tile staging: global -> VGPRs -> LDS ----
  const int ld_row = tid / T::kChunks;   // row within a pass
  const int ld_chunk = tid % T::kChunks;
  u32x4 stage_k[T::kPasses], stage_v[T::kPasses];

  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < T::kPasses; ++p) {
      const int key = j * kBN + p * T::kRowsPerPass + ld_row;
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (key < kv) {   // keys past the valid length are never read
        const size_t off = kv_base + (size_t)key * D + ld_chunk * 8;
        xk = *(const u32x4*)(K + off);
        xv = *(const u32x4*)(V + off);
      }
      stage_k[p] = xk;
      stage_v[p] = xv;
    }
  };
  auto store_tile = [&](int s) {
    char* kb = smem + s * T::kStage;
    char* vb = kb + T::kKBytes;
#pragma unroll
    for (int p = 0; p < T::kPasses; ++p) {
      const int r = p * T::kRowsPerPass + ld_row;
      *(u32x4*)(kb + r * T::kKStride + ld_chunk * 16) = stage_k[p];
      *(u32x4*)(vb + r * T::kVStride + ld_chunk * 16) = stage_v[p];
    }
  };

  // per-lane LDS offsets of the MFMA operand reads
  const int k_lane_off = (lane & 31) * T::kKStride + (lane >> 5) * 16;
  // transposing V read: 16-lane group g, lane i in it: lanes 4j..4j+3 of a group
  // fetch row j, four consecutive 4-element pieces of 16 columns; after the
  // transpose lane i holds column i of those 4 rows.
  const int g16 = lane >> 4;
  const int v_lane_off = (4 * (lane >> 5) + ((lane & 15) >> 2)) * T::kVStride + (16 * (g16 & 1) + 4 * (lane & 3)) * 2;

  f32x16 o_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o_acc[db] = (f32x16){};
  float m_run = -INFINITY;   // running max of S*c for this lane's row (same in lane ^ 32)
  float l_run = 0.f;         // partial running sum over this lane's half of the keys

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int s = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int k_lo = j * kBN;
    const bool skip = !wave_live || (causal && k_lo > row_hi);
    if (!skip) {
      const char* kb = smem + s * T::kStage;
      const char* vb = kb + T::kKBytes;

      // S^T = K Q^T for two 32-key blocks
      f32x16 sc[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        sc[sb] = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const u32x4 a = *(const u32x4*)(kb + k_lane_off + sb * 32 * T::kKStride + kc * 32);
          sc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qreg[kc], sc[sb], 0, 0, 0);
        }
      }

      // mask: only where the tile crosses the key length, the diagonal or masked rows
      const bool need_mask = (k_lo + kBN > kv) || (causal && k_lo + kBN - 1 > row_lo) || (row_lo < qs);
      if (need_mask) {
        const bool row_ok = my_row >= qs;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k_lo + 32 * sb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const bool ok = row_ok && key < kv && (!causal || key <= my_row);
            sc[sb][r] = ok ? sc[sb][r] : -INFINITY;
          }
      }

      // row max over this lane's 32 keys, then over the partner lane's 32
      float mx = sc[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
      mx = lane_swap_max(mx);
      const float tmax = mx * c;   // c > 0, so -inf stays -inf

      if (__builtin_amdgcn_ballot_w64(tmax > m_run + kTau)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o_acc[db] *= alpha;
      }
      const float msub = (m_run == -INFINITY) ? 0.f : m_run;

      // P = exp2(S*c - m): fp32 into the row sum, bf16 into the PV operand
      bf16x8 pb[4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(sc[sb][r], c, -msub));
          l_run += p[r];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = {pack2(p[8 * h + 0], p[8 * h + 1]), pack2(p[8 * h + 2], p[8 * h + 3]),
                           pack2(p[8 * h + 4], p[8 * h + 5]), pack2(p[8 * h + 6], p[8 * h + 7])};
          pb[2 * sb + h] = as_bf16x8(w);
        }
      }

      // O^T += V^T P^T: 16-key chunk cc pairs with P registers 8*(cc%2).. of block cc/2
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const char* p0 = vb + v_lane_off + (16 * cc) * T::kVStride + 64 * db;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 8 * T::kVStride));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], o_acc[db], 0, 0, 0);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(s ^ 1);
    __syncthreads();
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
        *(u32x2*)(orow + 32 * db + 8 * g + 4 * (lane >> 5)) = w;
      }
    }
    if (LSE && lane < 32)
      LSE[(size_t)bh * N_q + my_row] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
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
  const long long n_wg = (long long)B * H * n_qt;
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
