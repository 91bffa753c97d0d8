// Fused scaled-dot-product attention backward for MI355X (gfx950, CDNA4).
//
// Page cited: [PT2CUDA] aiknowledge.cn, "4.5 注意力优化实战：从PyTorch到CUDA的完整流程",
// step 4.2 (backward kernel): dQ sweeps every K/V block, dK and dV sweep every
// Q block, and the softmax of the forward pass is recomputed from what the
// forward kept (its row statistics; here the log-sum-exp).
//
// What one call computes is stated in include/attn.h. Three launches:
//   delta  D_i = sum_d dO_id * O_id (fp32), the row sum of P * dP that the
//          softmax Jacobian needs (sum_j P_ij dP_ij = dO_i . O_i).
//   dq     one workgroup of 4 wave64s per 128 query rows; each wave keeps its
//          32 rows of Q and dO in registers and walks the 32-key blocks its
//          rows can see (K and V through double-buffered LDS):
//            S^T  = K Q^T          (MFMA, lane = query row, 16 keys per lane)
//            dP^T = V dO^T         (MFMA, same layout)
//            P    = exp2(S c - LSE log2 e), 0 where masked
//            dS   = P (dP - D)
//            dQ^T += K^T dS^T      (MFMA, K^T by the transposing LDS read)
//   dkdv   one workgroup of 4 wave64s per 128 keys; each wave keeps its 32
//          keys of K and V in registers and walks the 32-row Q blocks that
//          can see them (Q, dO, LSE, D through double-buffered LDS):
//            S  = Q K^T, dP = dO V^T   (lane = key, 16 query rows per lane)
//            P, dS as above
//            dV^T += dO^T P,  dK^T += Q^T dS   (dO^T, Q^T by the transposing read)
//   dQ = scale * dS K and dK = scale * dS^T Q.
//
// MFMA 32x32x16 bf16 lane layouts (gfx950):
//   A (M x K): lane L holds row L%32, k = 8*(L/32) + 0..7;
//   B (K x N): lane L holds column L%32, the same k;
//   C (M x N): lane L reg r holds row 8*(r/4) + 4*(L/32) + r%4, column L%32.
// An accumulator's 16 registers thus run over the M index; when it becomes
// the B operand of the next product (contracting over that index), register
// 8*cc + e pairs with the transposing LDS read that delivers rows
// 16*cc + 8*(e/4) + 4*(L/32) + e%4 of the other operand.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr int kBlk = 32;          // rows (or keys) per block and per wave
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = kBlk * kWaves;   // rows (or keys) per workgroup
constexpr float kLog2e = 1.44269504088896340736f;

// 16-byte chunk c of block row r sits at chunk position c ^ swz(r), which
// keeps both the row reads (ds_read_b128) and the transposing reads
// (ds_read_b64_tr_b16) free of bank conflicts; the pattern repeats every 16 rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);   // round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane LDS byte offsets into one [32 rows][D] block.
template <int D>
struct Offs {
  int row0;          // row L%32, chunk L/32 (ds_read_b128); chunk pair kc: row0 ^ (32*kc)
  int tr[2];         // transposing read, rows 4*(L/32) + (L%16)/4 (+8 for tr[1]); column block db: ^ (64*db)
  __device__ Offs(int lane) {
    const int hf = lane >> 5;
    const int r = lane & 31;
    row0 = r * 2 * D + ((hf ^ swz<D>(r)) << 4);
    const int g = lane >> 4;
    const int rv = 4 * hf + ((lane & 15) >> 2);
    const int byte = 32 * (g & 1) + 8 * (lane & 3);
    tr[0] = rv * 2 * D + (((byte >> 4) ^ swz<D>(rv)) << 4) + (byte & 15);
    tr[1] = (rv + 8) * 2 * D + (((byte >> 4) ^ swz<D>(rv + 8)) << 4) + (byte & 15);
  }
};

// A operand of a product contracting over the block's rows: lane L gets
// column 32*db + L%32 of rows 16*cc + 8*hi + 4*(L/32) + 0..3 (hi = 0, 1).
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* blk, const Offs<D>& o, int cc, int db) {
  const char* p = blk + 16 * cc * 2 * D;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + (o.tr[0] ^ (64 * db))));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + (o.tr[1] ^ (64 * db))));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// A operand of a product contracting over d: lane L gets row L%32, d = 16*kc + 8*(L/32) + 0..7.
template <int D>
__device__ __forceinline__ bf16x8 read_row(const char* blk, const Offs<D>& o, int kc) {
  return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(blk + (o.row0 ^ (32 * kc))));
}

// Stage rows [r0, r0 + 32) of a [N, D] bf16 matrix (rows >= lim read as 0)
// into registers: thread t holds chunks t and t + kThreads of the block.
template <int D>
struct Stage {
  static constexpr int kChunks = kBlk * D / 8;
  static constexpr int kPer = kChunks / kThreads;
  u32x4 x[kPer];
  __device__ void load(const uint16_t* base, int r0, int lim, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + i * kThreads;
      const int r = id / (D / 8), c = id % (D / 8);
      x[i] = (u32x4){0u, 0u, 0u, 0u};
      if (r0 + r < lim) x[i] = *(const u32x4*)(base + (size_t)(r0 + r) * D + c * 8);
    }
  }
  __device__ void store(char* blk, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + i * kThreads;
      const int r = id / (D / 8), c = id % (D / 8);
      *(lds_u32x4*)(blk + r * 2 * D + ((c ^ swz<D>(r)) << 4)) = x[i];
    }
  }
};

// ---------------------------------------------------------------- delta
// D_i = sum_d dO_id O_id for every row of [rows, D]; D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const uint16_t* __restrict__ O,
                                                             const uint16_t* __restrict__ dO,
                                                             float* __restrict__ delta, long long rows) {
  constexpr int kL = D / 8;
  const long long row = (long long)blockIdx.x * (256 / kL) + threadIdx.x / kL;
  const int c = threadIdx.x % kL;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + row * D + c * 8);
    const u32x4 b = *(const u32x4*)(dO + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
      s += __uint_as_float(a[i] & 0xffff0000u) * __uint_as_float(b[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int m = kL / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, kL);
  if (row < rows && c == 0) delta[row] = s;
}

// ---------------------------------------------------------------- dq
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    uint16_t* __restrict__ dQ, int H, int N_q, int N_k, float c, float scale, int causal,
    const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_qt) {
  constexpr int kBlkBytes = kBlk * 2 * D;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][kBlkBytes];   // [buffer][K, V]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
  const int bh = blockIdx.x / n_qt;
  const int qt = n_qt - 1 - (int)(blockIdx.x % n_qt);   // tiles with more keys first
  const int b = bh / H;
  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);
  const size_t q_base = (size_t)bh * N_q * D, k_base = (size_t)bh * N_k * D;
  const int q0 = qt * kTile;
  const int q_end = min(q0 + kTile, N_q);
  int kv_end = kv;
  if (causal) kv_end = min(kv_end, q_end);
  if (qs >= q_end) kv_end = 0;
  const int nblk = (kv_end + kBlk - 1) / kBlk;

  const int row = q0 + kBlk * wave + (lane & 31);
  const bool row_ok = row < N_q;
  // this row's Q and dO as B operands (lane = row, d = 16*kc + 8*(L/32) + 0..7)
  bf16x8 qr[D / 16], gr[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
    if (row_ok) {
      a = *(const u32x4*)(Q + q_base + (size_t)row * D + kc * 16 + hf * 8);
      g = *(const u32x4*)(dO + q_base + (size_t)row * D + kc * 16 + hf * 8);
    }
    qr[kc] = __builtin_bit_cast(bf16x8, a);
    gr[kc] = __builtin_bit_cast(bf16x8, g);
  }
  float lse2 = INFINITY, dl = 0.f;   // +inf: a row with no allowed key gets P = 0
  if (row_ok) {
    const float l = LSE[(size_t)bh * N_q + row];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dl = delta[(size_t)bh * N_q + row];
  }
  // key j is allowed for this row iff j <= klim
  const int klim = (!row_ok || row < qs) ? -1 : min(kv - 1, causal ? row : 0x7fffffff);

  const Offs<D> off(lane);
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = (f32x16){};

  Stage<D> sk, sv;
  if (nblk > 0) {
    sk.load(K + k_base, 0, kv_end, tid);
    sv.load(V + k_base, 0, kv_end, tid);
    sk.store(smem[0][0], tid);
    sv.store(smem[0][1], tid);
  }
  __syncthreads();
  for (int n = 0; n < nblk; ++n) {
    const int cur = n & 1;
    if (n + 1 < nblk) {   // next block into registers while this one is used
      sk.load(K + k_base, (n + 1) * kBlk, kv_end, tid);
      sv.load(V + k_base, (n + 1) * kBlk, kv_end, tid);
    }
    const char* kb = smem[cur][0];
    const char* vb = smem[cur][1];
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      s = mfma(read_row<D>(kb, off, kc), qr[kc], s);
      dp = mfma(read_row<D>(vb, off, kc), gr[kc], dp);
    }
    // P and dS; register r holds key n*32 + 8*(r/4) + 4*hf + r%4
    const int lim = klim - n * kBlk - 4 * hf;
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int j0 = 8 * (r >> 2) + (r & 3);
      const float p0 = j0 <= lim ? __builtin_amdgcn_exp2f(s[r] * c - lse2) : 0.f;
      const float p1 = j0 + 1 <= lim ? __builtin_amdgcn_exp2f(s[r + 1] * c - lse2) : 0.f;
      w[r >> 1] = pack2(p0 * (dp[r] - dl), p1 * (dp[r + 1] - dl));
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const bf16x8 bw = __builtin_bit_cast(bf16x8, (u32x4){w[4 * cc], w[4 * cc + 1], w[4 * cc + 2], w[4 * cc + 3]});
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma(read_tr<D>(kb, off, cc, db), bw, acc[db]);
    }
    // The other buffer was last read in the previous iteration, before its
    // barrier: it can be refilled now, and one barrier publishes it.
    if (n + 1 < nblk) {
      sk.store(smem[cur ^ 1][0], tid);
      sv.store(smem[cur ^ 1][1], tid);
    }
    __syncthreads();
  }
  // dQ = scale * dQ^T: register r of block db holds d = 32*db + 8*(r/4) + 4*hf + r%4
  if (row_ok) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 x = {pack2(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale),
                         pack2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale)};
        *(u32x2*)(dQ + q_base + (size_t)row * D + 32 * db + 8 * g + 4 * hf) = x;
      }
  }
}

// ---------------------------------------------------------------- dk, dv
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int H, int N_q, int N_k, float c, float scale,
    int causal, const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_kt) {
  constexpr int kBlkBytes = kBlk * 2 * D;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][kBlkBytes];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float sstat[2][2][kBlk];         // [buffer][LSE*log2e, D]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
  const int bh = blockIdx.x / n_kt;
  const int kt = (int)(blockIdx.x % n_kt);   // under a causal mask, early keys have the most rows
  const int b = bh / H;
  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);
  const size_t q_base = (size_t)bh * N_q * D, k_base = (size_t)bh * N_k * D;
  const int k0 = kt * kTile;
  // query rows that can see a key of this tile: [r_begin, N_q)
  int r_begin = max(qs, causal ? k0 : 0);
  if (k0 >= kv) r_begin = N_q;                  // every key of the tile is masked
  const int blk0 = r_begin / kBlk;
  const int nblk = r_begin < N_q ? (N_q + kBlk - 1) / kBlk - blk0 : 0;

  const int key = k0 + kBlk * wave + (lane & 31);
  const bool key_ok = key < N_k;
  bf16x8 kr[D / 16], vr[D / 16];   // this key's K and V as B operands
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
    if (key_ok) {
      a = *(const u32x4*)(K + k_base + (size_t)key * D + kc * 16 + hf * 8);
      g = *(const u32x4*)(V + k_base + (size_t)key * D + kc * 16 + hf * 8);
    }
    kr[kc] = __builtin_bit_cast(bf16x8, a);
    vr[kc] = __builtin_bit_cast(bf16x8, g);
  }
  const bool key_live = key < kv;

  const Offs<D> off(lane);
  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) adk[db] = adv[db] = (f32x16){};

  Stage<D> sq, sg;
  float st = 0.f;   // thread t < 64 stages one LSE or D value
  auto load_stat = [&](int r0) {
    if (tid < 2 * kBlk) {
      const int r = r0 + (tid & (kBlk - 1));
      if (tid < kBlk) {
        st = INFINITY;
        if (r < N_q) {
          const float l = LSE[(size_t)bh * N_q + r];
          st = l == -INFINITY ? INFINITY : l * kLog2e;
        }
      } else {
        st = r < N_q ? delta[(size_t)bh * N_q + r] : 0.f;
      }
    }
  };
  auto store_stat = [&](int buf) {
    if (tid < 2 * kBlk) sstat[buf][tid / kBlk][tid & (kBlk - 1)] = st;
  };
  if (nblk > 0) {
    const int r0 = blk0 * kBlk;
    sq.load(Q + q_base, r0, N_q, tid);
    sg.load(dO + q_base, r0, N_q, tid);
    load_stat(r0);
    sq.store(smem[0][0], tid);
    sg.store(smem[0][1], tid);
    store_stat(0);
  }
  __syncthreads();
  for (int n = 0; n < nblk; ++n) {
    const int cur = n & 1;
    const int r0 = (blk0 + n) * kBlk;
    if (n + 1 < nblk) {
      sq.load(Q + q_base, r0 + kBlk, N_q, tid);
      sg.load(dO + q_base, r0 + kBlk, N_q, tid);
      load_stat(r0 + kBlk);
    }
    const char* qb = smem[cur][0];
    const char* gb = smem[cur][1];
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      s = mfma(read_row<D>(qb, off, kc), kr[kc], s);
      dp = mfma(read_row<D>(gb, off, kc), vr[kc], dp);
    }
    // register r holds query row r0 + 8*(r/4) + 4*hf + r%4 of this lane's key
    uint32_t wp[8], wd[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l2 = *(const lds_f32x4*)&sstat[cur][0][8 * g + 4 * hf];
      const f32x4 dd = *(const lds_f32x4*)&sstat[cur][1][8 * g + 4 * hf];
      float p[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const int qrow = r0 + 8 * g + 4 * hf + e;
        const bool ok = key_live && qrow >= qs && (!causal || key <= qrow);
        p[e] = ok ? __builtin_amdgcn_exp2f(s[r] * c - l2[e]) : 0.f;
        ds[e] = p[e] * (dp[r] - dd[e]);
      }
      wp[2 * g] = pack2(p[0], p[1]);
      wp[2 * g + 1] = pack2(p[2], p[3]);
      wd[2 * g] = pack2(ds[0], ds[1]);
      wd[2 * g + 1] = pack2(ds[2], ds[3]);
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const bf16x8 bp = __builtin_bit_cast(bf16x8, (u32x4){wp[4 * cc], wp[4 * cc + 1], wp[4 * cc + 2], wp[4 * cc + 3]});
      const bf16x8 bd = __builtin_bit_cast(bf16x8, (u32x4){wd[4 * cc], wd[4 * cc + 1], wd[4 * cc + 2], wd[4 * cc + 3]});
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        adv[db] = mfma(read_tr<D>(gb, off, cc, db), bp, adv[db]);
        adk[db] = mfma(read_tr<D>(qb, off, cc, db), bd, adk[db]);
      }
    }
    if (n + 1 < nblk) {   // the other buffer was last read before the previous barrier
      sq.store(smem[cur ^ 1][0], tid);
      sg.store(smem[cur ^ 1][1], tid);
      store_stat(cur ^ 1);
    }
    __syncthreads();
  }
  // register r of block db holds d = 32*db + 8*(r/4) + 4*hf + r%4 of this lane's key
  if (key_ok) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const size_t at = k_base + (size_t)key * D + 32 * db + 8 * g + 4 * hf;
        const u32x2 xk = {pack2(adk[db][4 * g] * scale, adk[db][4 * g + 1] * scale),
                          pack2(adk[db][4 * g + 2] * scale, adk[db][4 * g + 3] * scale)};
        const u32x2 xv = {pack2(adv[db][4 * g], adv[db][4 * g + 1]), pack2(adv[db][4 * g + 2], adv[db][4 * g + 3])};
        *(u32x2*)(dK + at) = xk;
        *(u32x2*)(dV + at) = xv;
      }
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N_q,
                        int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                        const int32_t* q_start, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  const long long bh = (long long)B * H;
  if (bh == 0 || (N_q == 0 && N_k == 0)) return ATTN_OK;
  const bool has_q = N_q > 0, has_k = N_k > 0;
  if (has_q && (!q || !o || !dout || !lse || !dq || !delta)) return ATTN_ERR_NULL;
  if (has_k && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (bh > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const long long n_qt = (N_q + kTile - 1) / kTile, n_kt = (N_k + kTile - 1) / kTile;
  if (bh * n_qt > 0x7fffffffLL || bh * n_kt > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const size_t qb = (size_t)bh * N_q * d * 2, kb = (size_t)bh * N_k * d * 2, rb = (size_t)bh * N_q * 4;
  if (((uintptr_t)q | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq) & 15) return ATTN_ERR_ALIGN;
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)dk | (uintptr_t)dv) & 15) return ATTN_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)delta) & 3) return ATTN_ERR_ALIGN;
  const void* ins[] = {q, k, v, o, dout, lse};
  const size_t in_n[] = {qb, kb, kb, qb, qb, rb};
  void* outs[] = {dq, dk, dv, delta};
  const size_t out_n[] = {qb, kb, kb, rb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return ATTN_ERR_ALIAS;
  }

  const float c = scale * kLog2e;
  int causal01 = causal ? 1 : 0, Hi = H, Nq = N_q, Nk = N_k;
  float cc = c, sc = scale;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v,
                 *op = (const uint16_t*)o, *gp = (const uint16_t*)dout;
  uint16_t *dqp = (uint16_t*)dq, *dkp = (uint16_t*)dk, *dvp = (uint16_t*)dv;
  hipError_t e = hipSuccess;
  if (has_q) {
    long long rows = bh * N_q;
    const long long per = 256 / (d / 8);
    const long long nb = (rows + per - 1) / per;
    if (nb > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    void* a0[] = {(void*)&op, (void*)&gp, (void*)&delta, (void*)&rows};
    const void* f0 = d == 128 ? (const void*)attn_bwd_delta_kernel<128> : (const void*)attn_bwd_delta_kernel<64>;
    e = hipLaunchKernel(f0, dim3((unsigned)nb), dim3(256), a0, 0, stream);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
    int nqt = (int)n_qt;
    void* a1[] = {(void*)&qp, (void*)&kp, (void*)&vp, (void*)&gp, (void*)&lse, (void*)&delta, (void*)&dqp,
                  (void*)&Hi, (void*)&Nq, (void*)&Nk, (void*)&cc, (void*)&sc, (void*)&causal01,
                  (void*)&seqlens_k, (void*)&q_start, (void*)&nqt};
    const void* f1 = d == 128 ? (const void*)attn_bwd_dq_kernel<128> : (const void*)attn_bwd_dq_kernel<64>;
    e = hipLaunchKernel(f1, dim3((unsigned)(bh * n_qt)), dim3(kThreads), a1, 0, stream);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  if (has_k) {
    int nkt = (int)n_kt;
    void* a2[] = {(void*)&qp, (void*)&kp, (void*)&vp, (void*)&gp, (void*)&lse, (void*)&delta, (void*)&dkp,
                  (void*)&dvp, (void*)&Hi, (void*)&Nq, (void*)&Nk, (void*)&cc, (void*)&sc, (void*)&causal01,
                  (void*)&seqlens_k, (void*)&q_start, (void*)&nkt};
    const void* f2 = d == 128 ? (const void*)attn_bwd_dkdv_kernel<128> : (const void*)attn_bwd_dkdv_kernel<64>;
    e = hipLaunchKernel(f2, dim3((unsigned)(bh * n_kt)), dim3(kThreads), a2, 0, stream);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}
