// Fused scaled-dot-product attention backward for MI355X (gfx950, CDNA4).
//
// Page cited: [PT2CUDA] aiknowledge.cn, "4.5 注意力优化实战：从PyTorch到CUDA的完整流程",
// step 4.2 (backward kernel): dQ sweeps every K/V block, dK and dV sweep every
// Q block, and the softmax of the forward pass is recomputed from what the
// forward kept (its row statistics; here the log-sum-exp).
//
// What one call computes is stated in include/attn.h. Three launches:
//   delta  per row (LSE * log2 e, D_i) with D_i = sum_d dO_id * O_id (fp32), the
//          row sum of P * dP that the softmax Jacobian needs
//          (sum_j P_ij dP_ij = dO_i . O_i).
//   dq     one workgroup of 8 wave64s per 256 query rows; each wave keeps its
//          32 rows of Q and dO in registers and walks the 32-key blocks its
//          rows can see (K and V copied straight into a 4-deep LDS ring):
//            S^T  = K Q^T          (MFMA, lane = query row, 16 keys per lane)
//            dP^T = V dO^T         (MFMA, same layout)
//            P    = exp2(S c - LSE log2 e), 0 where masked
//            dS   = P (dP - D)
//            dQ^T += K^T dS^T      (MFMA, K^T by the transposing LDS read)
//   dkdv   (d = 128) one workgroup of 8 wave64s per 256 keys; each wave keeps
//          its 32 keys of K in registers and of V in an LDS block, and walks
//          the 32-row Q blocks that can see them (Q, dO and the rows' (LSE, D)
//          through the LDS ring); (d = 64) 4 wave64s per 128 keys, K and V in
//          registers, software pipelined across blocks:
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
#include <mutex>
#include <type_traits>

#include "attn.h"
#include "launch.h"

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
typedef __attribute__((address_space(3))) float lds_f32;

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

// ---- the LDS ring: blocks copied from global memory straight into LDS ----
// A block is 32 rows of a [N, D] bf16 matrix (one head). Copy number ci of a
// block moves 1 KB: lane L brings the 16 bytes that belong at byte 16*L of
// that KB, i.e. row ci*kRowsPerKB + L/kLanesPerRow, chunk position
// L%kLanesPerRow, which holds logical chunk (position ^ swz(row)).
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kDepth = 4;   // ring depth in blocks: copies run three blocks ahead

template <int D, int W = kWaves>   // W: waves of the workgroup that share the copies
struct Ring {
  static constexpr int kBlkBytes = kBlk * 2 * D;
  static constexpr int kKB = kBlkBytes / 1024;        // copies per matrix block
  static constexpr int kRowsPerKB = 1024 / (2 * D);
  static constexpr int kLanesPerRow = 64 / kRowsPerKB;
  static constexpr int kCpw = 2 * kKB / W;            // copies per wave per block (two matrices)
  static_assert((2 * kKB) % W == 0, "copies must split evenly over the waves");
};

// Raw buffer descriptor over [base, base + bytes): lanes whose offset is at
// or past `bytes` fetch nothing.
__device__ __forceinline__ i32x4 rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);                 // num_records
  r[3] = 0x00020000;                                                 // 32-bit data format
  return r;
}

// One 1 KB global -> LDS copy: 16 bytes per lane from rs at byte offset
// off + soff, written to LDS byte lds + 16*lane. Completion is awaited with
// wait_copies; the compiler does not see the LDS write (inline assembly), so
// every read of a copied block follows an explicit wait and a barrier.
__device__ __forceinline__ void copy_kb(const i32x4& rs, uint32_t soff, uint32_t off, uint32_t lds) {
  uint32_t v;
  // (the add after the M0 write is the wait state the LDS copy needs)
  asm volatile("s_mov_b32 m0, %1\n\tv_add_u32 %0, %2, %3\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
               : "=&v"(v) : "s"(lds), "s"(soff), "v"(off), "s"(rs) : "memory", "m0");
}

// copy_kb with lane offset 16*lane, computed from the lane id inside the
// block, so that no register has to hold it across a loop.
__device__ __forceinline__ void copy_kb_lane16(const i32x4& rs, uint32_t soff, uint32_t lds) {
  uint32_t v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 4, %0\n\t"
               "s_mov_b32 m0, %1\n\tv_add_u32 %0, %2, %0\n\tbuffer_load_dwordx4 %0, %3, 0 offen lds"
               : "=&v"(v) : "s"(lds), "s"(soff), "s"(rs) : "memory", "m0");
}

// vmcnt(0) as a builtin the compiler sees: the register loads issued before
// the ring starts are complete, so it places no wait of its own (which would
// also drain the ring) inside the loop.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One 4-byte-per-lane global -> LDS copy (256 bytes at LDS byte lds + 4*lane).
__device__ __forceinline__ void copy_dw(const i32x4& rs, uint32_t soff, uint32_t off, uint32_t lds) {
  uint32_t v;
  asm volatile("s_mov_b32 m0, %1\n\tv_add_u32 %0, %2, %3\n\tbuffer_load_dword %0, %4, 0 offen lds"
               : "=&v"(v) : "s"(lds), "s"(soff), "v"(off), "s"(rs) : "memory", "m0");
}

// Bit-packed dense mask (the layout of attn_fwd_masked): bit t of word w of
// row i set means row i may attend to key 32*w + t; rows of mrw words,
// matrix (b, h) at word b*msb + h*msh.
struct DenseMask {
  const uint32_t* bits;
  long long sb, sh;
  int rw;
};

// Block mask of attn_fwd_block_sparse: a byte per (256-row query tile,
// 128-key block), rows of n_ks bytes, matrix (b, h) at byte b*sb + h*sh.
struct BlockMask {
  const uint8_t* flags;
  long long sb, sh;
  int n_ks;
};
constexpr int kMaxSparse = 1024;   // list entries (key slices, or 32-row query blocks) on the sparse path
constexpr int kListPad = 16;       // sentinel entries past a list (the copies look up to 4 ahead)

template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Lane offset of copy ci (0 .. 2*kKB-1) of a block pair: matrix ci / kKB,
// KB ci % kKB; returned relative to that matrix's block start.
template <int D>
__device__ __forceinline__ int copy_lane_off(int ci, int lane) {
  using R = Ring<D>;
  const int r = (ci % R::kKB) * R::kRowsPerKB + lane / R::kLanesPerRow;
  return r * 2 * D + (((lane % R::kLanesPerRow) ^ swz<D>(r)) << 4);
}

// ---------------------------------------------------------------- delta
// Per row: stats = (LSE * log2 e, D) with D = sum_d dO_id O_id, and +inf in
// place of LSE * log2 e for a row with no allowed key (LSE = -inf), so that
// exp2(S c - stats.x) is 0 there. D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const uint16_t* __restrict__ O,
                                                             const uint16_t* __restrict__ dO,
                                                             const float* __restrict__ LSE,
                                                             f32x2* __restrict__ stats, long long rows) {
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
  if (row < rows && c == 0) {
    const float l = LSE[row];
    stats[row] = (f32x2){l == -INFINITY ? INFINITY : l * kLog2e, s};
  }
}

// ---------------------------------------------------------------- dq
// Dense: a bit-packed mask is intersected with the rules; each wave copies
// its 32 rows' words of the block with the block (one more copy per block).
// Mode 2 (Sparse): the key slices the block mask keeps for the tile's
// 256-row block-mask tile are compacted into an LDS list that the ring walks.
// Waves per dQ workgroup (32 query rows each). Eight waves (256 rows, one
// workgroup per CU) share one K/V ring: half the copies and LDS writes per
// flop of two 4-wave workgroups per CU, and measured +0.3 to +2.3 % over them.
constexpr int waves_q(int) { return 8; }

template <int D, int Mode>   // 0: rules only; 1: dense mask (Dense); 2: block-sparse (Sparse)
__global__ __launch_bounds__(64 * waves_q(D)) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const f32x2* __restrict__ stats, uint16_t* __restrict__ dQ, int H, int N_q,
    int N_k, float c, float scale, int causal, int coff, const int32_t* __restrict__ seqlens_k,
    const int32_t* __restrict__ q_start, int n_qt, DenseMask dm, BlockMask bmk) {
  constexpr bool Dense = Mode == 1, Sparse = Mode == 2;
  constexpr int kWQ = waves_q(D), kThreadsQ = 64 * kWQ, kTileQ = kBlk * kWQ;
  using R = Ring<D, kWQ>;
  constexpr int kMaskBytes = Dense ? kWQ * 256 : 0;
  constexpr int kStage = 2 * R::kBlkBytes + kMaskBytes;   // [K block][V block][mask words of each wave]
  constexpr int kCpb = R::kCpw + (Dense ? 1 : 0);         // copies per wave per block
  constexpr int kListBytes = Sparse ? 4 * (kMaxSparse + kListPad + 4) : 0;
  __shared__ __attribute__((aligned(1024))) char smem[kDepth * kStage + kListBytes];
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  // Under a causal mask a tile's work grows with its index: launch the tiles
  // heaviest first across all heads (tile-major), so that the light ones fill
  // in at the end. Without it, head-major order keeps a head's tiles together
  // (they read the same K and V).
  const int n_bh = (int)(gridDim.x / n_qt);
  const int bh = causal ? (int)(blockIdx.x % n_bh) : (int)(blockIdx.x / n_qt);
  const int qt = causal ? n_qt - 1 - (int)(blockIdx.x / n_bh) : (int)(blockIdx.x % n_qt);
  const int b = bh / H;
  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);
  const size_t q_base = (size_t)bh * N_q * D, k_base = (size_t)bh * N_k * D;
  const int q0 = qt * kTileQ;
  const int q_end = min(q0 + kTileQ, N_q);
  int kv_end = kv;
  if (causal) kv_end = min(kv_end, max(q_end + coff, 0));   // row i sees keys <= i + coff
  if (qs >= q_end) kv_end = 0;
  int nblk = (kv_end + kBlk - 1) / kBlk;
  // Sparse: list of the kept slices below kv_end (ring position -> slice),
  // padded with the slice nblk, whose copies fetch nothing
  [[maybe_unused]] int* lst = (int*)(smem + kDepth * kStage);
  if constexpr (Sparse) {
    if (wave == 0) {
      const uint8_t* fl = bmk.flags + (size_t)b * bmk.sb + (size_t)(bh - b * H) * bmk.sh +
                          (size_t)(q0 / 256) * bmk.n_ks;
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int sl = 16 * lane + i;
        if (sl < nblk && fl[sl >> 2] != 0) bits |= 1u << i;   // a flag covers 4 slices (128 keys)
      }
      const int cnt = __builtin_popcount(bits);
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      int pos = incl - cnt;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((bits >> i) & 1u) lst[pos++] = 16 * lane + i;
      const int total = __shfl(incl, 63, 64);
      if (lane < kListPad) lst[total + lane] = nblk;
      if (lane == 0) lst[kMaxSparse + kListPad] = total;
    }
    __syncthreads();
    nblk = __builtin_amdgcn_readfirstlane(lst[kMaxSparse + kListPad]);
  }
  // key slice of ring position n
  auto slice_of = [&](int n) __attribute__((always_inline)) {
    if constexpr (Sparse) return __builtin_amdgcn_readfirstlane(lst[n]);
    else return n;
  };

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
    const f32x2 st = stats[(size_t)bh * N_q + row];
    lse2 = st[0];
    dl = st[1];
  }
  // key j is allowed for this row iff j <= klim
  const int klim = (!row_ok || row < qs) ? -1 : min(kv - 1, causal ? row + coff : 0x7fffffff);
  // Blocks n < full_below need no mask for any row of this wave: all its rows
  // exist and are past q_start, and every key of the block is below kv and
  // (causal) at or below the wave's first row.
  const int wrow0 = q0 + kBlk * wave;
  int full_below = 0;
  if (wrow0 + kBlk <= N_q && wrow0 >= qs) full_below = min(kv, causal ? max(wrow0 + 1 + coff, 0) : kv) / kBlk;
  full_below = __builtin_amdgcn_readfirstlane(full_below);

  wait_loads();
  // Keys past kv_end fetch nothing, so a stage keeps rows no copy wrote: zero
  // the ring once, then such rows hold zeros or keys of an earlier block, all
  // finite, and their probabilities are 0.
  for (int i = tid; i < kDepth * kStage / 16; i += kThreadsQ) *(lds_u32x4*)(smem + 16 * i) = (u32x4){0u, 0u, 0u, 0u};
  __syncthreads();
  const i32x4 k_rs = rsrc(K + k_base, (uint32_t)kv_end * 2 * D), v_rs = rsrc(V + k_base, (uint32_t)kv_end * 2 * D);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  int cpoff[R::kCpw];
#pragma unroll
  for (int i = 0; i < R::kCpw; ++i) cpoff[i] = copy_lane_off<D>(wave * R::kCpw + i, lane);
  // Dense: lane L < 32 brings the word of row wrow0 + L for the block
  [[maybe_unused]] i32x4 m_rs = {0, 0, 0, 0};
  [[maybe_unused]] uint32_t m_off = 0;
  if constexpr (Dense) {
    m_rs = rsrc(dm.bits + (size_t)b * dm.sb + (size_t)(bh - b * H) * dm.sh, (uint32_t)N_q * dm.rw * 4);
    m_off = lane < 32 ? (uint32_t)(wrow0 + lane) * dm.rw * 4 : 0x40000000u;
  }
  auto issue = [&](int n) {   // the block of ring position n into stage n % kDepth
    const uint32_t st = lds0 + (uint32_t)(n % kDepth) * kStage;
    const uint32_t soff = (uint32_t)slice_of(n) * R::kBlkBytes;
#pragma unroll
    for (int i = 0; i < R::kCpw; ++i) {
      const int ci = wave * R::kCpw + i;
      const bool is_v = ci >= R::kKB;
      copy_kb(is_v ? v_rs : k_rs, soff, cpoff[i], st + (uint32_t)ci * 1024);
    }
    if constexpr (Dense) copy_dw(m_rs, (uint32_t)n * 4, m_off, st + 2 * R::kBlkBytes + wave * 256);
  };

  const Offs<D> off(lane);
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = (f32x16){};
#pragma unroll
  for (int n = 0; n < kDepth - 1; ++n) issue(n);
  for (int n = 0; n < nblk; ++n) {
    wait_copies<(kDepth - 2) * kCpb>();   // block n has landed (this wave's copies)
    __syncthreads();                          // everyone's copies; block n-1's stage is free
    issue(n + kDepth - 1);
    const int sl = slice_of(n);
    const char* kb = smem + (n % kDepth) * kStage;
    const char* vb = kb + R::kBlkBytes;
    f32x16 s = {}, dp = {};
    {
      bf16x8 ka[2], va[2];   // operands read one step ahead of their MFMAs
      ka[0] = read_row<D>(kb, off, 0);
      va[0] = read_row<D>(vb, off, 0);
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        if (kc + 1 < D / 16) {
          ka[(kc + 1) & 1] = read_row<D>(kb, off, kc + 1);
          va[(kc + 1) & 1] = read_row<D>(vb, off, kc + 1);
        }
        s = mfma(ka[kc & 1], qr[kc], s);
        dp = mfma(va[kc & 1], gr[kc], dp);
      }
    }
    // P and dS; register r holds key n*32 + 8*(r/4) + 4*hf + r%4
    uint32_t w[8];
    if (!Dense && sl < full_below) {   // every key of the block is allowed for every row of the wave
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        w[r >> 1] = pack2(__builtin_amdgcn_exp2f(s[r] * c - lse2) * (dp[r] - dl),
                          __builtin_amdgcn_exp2f(s[r + 1] * c - lse2) * (dp[r + 1] - dl));
    } else if constexpr (Dense) {
      // the row's word for the block, ANDed with the rules' prefix of allowed
      // keys and shifted so that bit e is the lane's key offset e (+ 4*hf)
      uint32_t mw = *(const __attribute__((address_space(3))) uint32_t*)(kb + 2 * R::kBlkBytes + wave * 256 +
                                                                          4 * (lane & 31));
      const int lim0 = klim - sl * kBlk;
      const uint32_t pre = lim0 >= 31 ? 0xffffffffu : (lim0 < 0 ? 0u : ((2u << lim0) - 1u));
      mw = (mw & pre) >> (4 * hf);
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int j0 = 8 * (r >> 2) + (r & 3);
        const float d0 = (mw >> j0) & 1u ? __builtin_amdgcn_exp2f(s[r] * c - lse2) * (dp[r] - dl) : 0.f;
        const float d1 = (mw >> (j0 + 1)) & 1u ? __builtin_amdgcn_exp2f(s[r + 1] * c - lse2) * (dp[r + 1] - dl) : 0.f;
        w[r >> 1] = pack2(d0, d1);
      }
    } else {
      const int lim = klim - sl * kBlk - 4 * hf;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int j0 = 8 * (r >> 2) + (r & 3);
        const float d0 = j0 <= lim ? __builtin_amdgcn_exp2f(s[r] * c - lse2) * (dp[r] - dl) : 0.f;
        const float d1 = j0 + 1 <= lim ? __builtin_amdgcn_exp2f(s[r + 1] * c - lse2) * (dp[r + 1] - dl) : 0.f;
        w[r >> 1] = pack2(d0, d1);
      }
    }
    {
      bf16x8 ta[2];
      ta[0] = read_tr<D>(kb, off, 0, 0);
#pragma unroll
      for (int i = 0; i < 2 * (D / 32); ++i) {   // i = cc * (D/32) + db
        const int cc = i / (D / 32), db = i % (D / 32);
        if (i + 1 < 2 * (D / 32)) ta[(i + 1) & 1] = read_tr<D>(kb, off, (i + 1) / (D / 32), (i + 1) % (D / 32));
        const bf16x8 bw = __builtin_bit_cast(bf16x8, (u32x4){w[4 * cc], w[4 * cc + 1], w[4 * cc + 2], w[4 * cc + 3]});
        acc[db] = mfma(ta[i & 1], bw, acc[db]);
      }
    }
  }
  wait_copies<0>();   // no copy may still be writing LDS when the workgroup ends
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

// ---------------------------------------------------------------- dk, dv (d = 64)
// At d = 64 a block carries half the MFMA work of d = 128 but the same
// softmax work, and this kernel's software pipeline (the next block's S and
// dP on the MFMA unit while the VALU turns this block's into P and dS)
// measured faster than two waves per SIMD without it (attn_bwd_dkdv_kernel).
// Dense: as in the dQ kernel; each wave copies, per block, the words of the
// block's 32 rows that hold its own 32 keys.
// Mode 2 (Sparse): the WG's 128 keys are one key block of the mask; it walks
// the 32-row query blocks of the 256-row tiles that keep that block. Each
// list entry carries the query block and a mask of the waves that take part
// (all of them: the key block is the WG's).
template <int D, int Mode>   // 0: rules only; 1: dense mask (Dense); 2: block-sparse (Sparse)
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_pipe_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const f32x2* __restrict__ stats, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int H, int N_q, int N_k, float c, float scale, int causal, int coff,
    const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_kt, DenseMask dm,
    BlockMask bmk) {
  constexpr bool Dense = Mode == 1, Sparse = Mode == 2;
  using R = Ring<D>;
  constexpr int kMaskBytes = Dense ? kWaves * 256 : 0;
  // [Q block][dO block][stats of the 32 rows][mask words of each wave]
  constexpr int kStage = 2 * R::kBlkBytes + 1024 + kMaskBytes;
  constexpr int kCpb = R::kCpw + (Dense ? 1 : 0);   // copies per wave per block (wave 0: one more)
  constexpr int kListBytes = Sparse ? 4 * (kMaxSparse + kListPad + 4) : 0;
  __shared__ __attribute__((aligned(1024))) char smem[(kDepth + 1) * kStage + kListBytes];
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  // Under a causal mask early key tiles have the most rows: tile-major order,
  // heaviest first across all heads (see the dq kernel).
  const int n_bh = (int)(gridDim.x / n_kt);
  const int bh = causal ? (int)(blockIdx.x % n_bh) : (int)(blockIdx.x / n_kt);
  const int kt = causal ? (int)(blockIdx.x / n_bh) : (int)(blockIdx.x % n_kt);
  const int b = bh / H;
  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);
  const size_t q_base = (size_t)bh * N_q * D, k_base = (size_t)bh * N_k * D;
  const int k0 = kt * kTile;
  // query rows that can see a key of this tile: [r_begin, N_q)
  int r_begin = max(qs, causal ? max(k0 - coff, 0) : 0);   // row i sees keys <= i + coff
  if (k0 >= kv) r_begin = N_q;                  // every key of the tile is masked
  const int blk0 = r_begin / kBlk;
  int nblk = r_begin < N_q ? (N_q + kBlk - 1) / kBlk - blk0 : 0;
  // Sparse: list entries blk | (wave mask << 24) of the kept query blocks,
  // padded with the block past the last row (its copies fetch nothing)
  [[maybe_unused]] int* lst = (int*)(smem + (kDepth + 1) * kStage);
  if constexpr (Sparse) {
    const int nbq = (N_q + kBlk - 1) / kBlk;   // 32-row query blocks of the head
    if (wave == 0) {
      const uint8_t* fl = bmk.flags + (size_t)b * bmk.sb + (size_t)(bh - b * H) * bmk.sh;
      int base = 0;
      for (int t0 = blk0 / 8; t0 * 8 < nbq && nblk > 0; t0 += 64) {   // 256-row tiles, one per lane
        const int t = t0 + lane;
        // the WG's 128 keys are one block of the mask: all its waves take part or none
        uint32_t wm = 0;
        if (t * 8 < nbq && fl[(size_t)t * bmk.n_ks + kt] != 0) wm = (1u << kWaves) - 1;
        const int lo = max(8 * t, blk0), hi = min(8 * t + 8, nbq);
        const int cnt = (wm != 0 && hi > lo) ? hi - lo : 0;
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int x = __shfl_up(incl, o, 64);
          if (lane >= o) incl += x;
        }
        int pos = base + incl - cnt;
        for (int q = lo; q < lo + cnt; ++q) lst[pos++] = q | (int)(wm << 24);
        base += __shfl(incl, 63, 64);
      }
      if (lane < kListPad) lst[base + lane] = nbq;
      if (lane == 0) lst[kMaxSparse + kListPad] = base;
    }
    __syncthreads();
    nblk = __builtin_amdgcn_readfirstlane(lst[kMaxSparse + kListPad]);
  }
  // first query row of ring position n, and whether this wave's slice takes part
  auto row0_of = [&](int n) __attribute__((always_inline)) {
    if constexpr (Sparse) return (__builtin_amdgcn_readfirstlane(lst[n]) & 0xffffff) * kBlk;
    else return (blk0 + n) * kBlk;
  };
  auto wave_in = [&](int n) __attribute__((always_inline)) {
    if constexpr (Sparse) return ((__builtin_amdgcn_readfirstlane(lst[n]) >> (24 + wave)) & 1) != 0;
    else return true;
  };

  const int wkey0 = k0 + kBlk * wave;   // this wave's first key
  const int key = wkey0 + (lane & 31);
  const bool key_ok = key < N_k, key_live = key < kv;
  const bool wkey_live = wkey0 + kBlk <= kv;   // all 32 keys of the wave are valid
  bf16x8 kr[D / 16], vr[D / 16];   // this key's K and V as B operands (zeros past the valid length)
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
    if (key_live) {
      a = *(const u32x4*)(K + k_base + (size_t)key * D + kc * 16 + hf * 8);
      g = *(const u32x4*)(V + k_base + (size_t)key * D + kc * 16 + hf * 8);
    }
    kr[kc] = __builtin_bit_cast(bf16x8, a);
    vr[kc] = __builtin_bit_cast(bf16x8, g);
  }

  wait_loads();
  // Rows past N_q fetch nothing: zero the ring once, so such rows hold zeros
  // or rows of an earlier block (finite) and are masked out below.
  for (int i = tid; i < (kDepth + 1) * kStage / 16; i += kThreads) *(lds_u32x4*)(smem + 16 * i) = (u32x4){0u, 0u, 0u, 0u};
  __syncthreads();
  const uint32_t rows_bytes = (uint32_t)N_q * 2 * D;
  const i32x4 q_rs = rsrc(Q + q_base, rows_bytes), g_rs = rsrc(dO + q_base, rows_bytes);
  const i32x4 s_rs = rsrc(stats + (size_t)bh * N_q, (uint32_t)N_q * 8);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  int cpoff[R::kCpw];
#pragma unroll
  for (int i = 0; i < R::kCpw; ++i) cpoff[i] = copy_lane_off<D>(wave * R::kCpw + i, lane);
  // the stats copy (wave 0): lanes 0..15 bring the 256 bytes of the block's 32 rows
  const int soff_lane = lane < 16 ? 16 * lane : 0x40000000;
  // Ring of kDepthKV stages: while block n's dV/dK products run, block n+1's
  // S and dP are already computed, so two stages are being read and up to
  // three more blocks are in flight.
  constexpr int kDepthKV = kDepth + 1;
  // Dense: lane L < 32 brings, for row r0 + L, the word that holds this wave's keys
  [[maybe_unused]] i32x4 m_rs = {0, 0, 0, 0};
  [[maybe_unused]] uint32_t m_off = 0;
  if constexpr (Dense) {
    m_rs = rsrc(dm.bits + (size_t)b * dm.sb + (size_t)(bh - b * H) * dm.sh, (uint32_t)N_q * dm.rw * 4);
    m_off = lane < 32 ? (uint32_t)lane * dm.rw * 4 + (uint32_t)(wkey0 >> 5) * 4 : 0x40000000u;
  }
  auto issue = [&](int n) {   // the block of ring position n into stage n % kDepthKV
    const uint32_t st = lds0 + (uint32_t)(n % kDepthKV) * kStage;
    const uint32_t r0 = (uint32_t)row0_of(n);
#pragma unroll
    for (int i = 0; i < R::kCpw; ++i) {
      const int ci = wave * R::kCpw + i;
      const bool is_g = ci >= R::kKB;
      copy_kb(is_g ? g_rs : q_rs, r0 * 2 * D, cpoff[i], st + (uint32_t)ci * 1024);
    }
    if (wave == 0) copy_kb(s_rs, r0 * 8, soff_lane, st + 2 * R::kBlkBytes);
    if constexpr (Dense) copy_dw(m_rs, r0 * dm.rw * 4, m_off, st + 2 * R::kBlkBytes + 1024 + wave * 256);
  };
  // Block n has landed once at most the `ahead` newest blocks' copies of this
  // wave are in flight (wave 0 issues one copy more per block).
  auto wait_block = [&](auto ahead) {
    constexpr int A = decltype(ahead)::value;
    if (wave == 0) wait_copies<A * (kCpb + 1)>();
    else wait_copies<A * kCpb>();
  };
  auto stage_of = [&](int n) { return (const char*)smem + (n % kDepthKV) * kStage; };

  const Offs<D> off(lane);
  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) adk[db] = adv[db] = (f32x16){};
  // S = Q K^T and dP = dO V^T of the block in stage qb: all A operands are
  // read first (before the full/masked branch of the loop, so the MFMAs in
  // either branch only count the reads down), then the products
  using Rows = bf16x8[D / 16];
  auto sdp_read = [&](const char* qb, Rows& qa, Rows& ga) __attribute__((always_inline)) {
    const char* gb = qb + R::kBlkBytes;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qa[kc] = read_row<D>(qb, off, kc);
      ga[kc] = read_row<D>(gb, off, kc);
    }
  };
  auto sdp = [&](const Rows& qa, const Rows& ga, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    s = (f32x16){};
    dp = (f32x16){};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      s = mfma(qa[kc], kr[kc], s);
      dp = mfma(ga[kc], vr[kc], dp);
    }
  };
  // P and dS of block n from its S and dP, packed as the B operands of the
  // dV and dK products; register r holds query row r0 + 8*(r/4) + 4*hf + r%4.
  // no mask anywhere in block n for this wave: all its keys are valid, all
  // rows exist and are past q_start, and (causal) the block starts at or
  // after the wave's last key
  auto block_full = [&](int n) {
    const int r0 = row0_of(n);
    // one condition (bitwise, not short-circuit): a single branch lets the
    // operand reads placed before it stay there
    return wkey_live & (r0 + kBlk <= N_q) & (r0 >= qs) & (!causal | (r0 + coff >= wkey0 + kBlk - 1)) & wave_in(n);
  };
  auto softmax_grad = [&](auto full_t, int n, const f32x16& s, const f32x16& dp, uint32_t (&wp)[8],
                          uint32_t (&wd)[8]) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_t)::value;
    const int r0 = row0_of(n);
    [[maybe_unused]] const bool in = wave_in(n);
    const char* sb = stage_of(n) + 2 * R::kBlkBytes;
    [[maybe_unused]] const char* mb = sb + 1024 + wave * 256;   // Dense: word of row r0 + t at 4*t
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // stats of rows 8g + 4hf .. +3: (lse2, D) pairs, 32 bytes
      const f32x4 s01 = *(const lds_f32x4*)(sb + 8 * (8 * g + 4 * hf));
      const f32x4 s23 = *(const lds_f32x4*)(sb + 8 * (8 * g + 4 * hf) + 16);
      const float l2[4] = {s01[0], s01[2], s23[0], s23[2]};
      const float dd[4] = {s01[1], s01[3], s23[1], s23[3]};
      float p[4], ds[4];
      if constexpr (full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __builtin_amdgcn_exp2f(s[4 * g + e] * c - l2[e]);
          ds[e] = p[e] * (dp[4 * g + e] - dd[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const int qrow = r0 + 8 * g + 4 * hf + e;
          bool ok = key_live && qrow < N_q && qrow >= qs && (!causal || key <= qrow + coff);
          if constexpr (Sparse) ok = ok && in;
          if constexpr (Dense)
            ok = ok && ((*(const __attribute__((address_space(3))) uint32_t*)(mb + 4 * (8 * g + 4 * hf + e)) >>
                         (lane & 31)) & 1u);
          p[e] = ok ? __builtin_amdgcn_exp2f(s[r] * c - l2[e]) : 0.f;
          ds[e] = ok ? p[e] * (dp[r] - dd[e]) : 0.f;
        }
      }
      wp[2 * g] = pack2(p[0], p[1]);
      wp[2 * g + 1] = pack2(p[2], p[3]);
      wd[2 * g] = pack2(ds[0], ds[1]);
      wd[2 * g + 1] = pack2(ds[2], ds[3]);
    }
  };
  // Interleave the next block's S and dP MFMAs (16) with this block's
  // softmax VALU work and the LDS reads, one MFMA per group.
  auto interleave = [&](auto valu_t) __attribute__((always_inline)) {
    constexpr int kV = decltype(valu_t)::value;
#pragma unroll
    for (int i = 0; i < 2 * (D / 16); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);   // VALU
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS for the block in stage qb
  auto dvdk = [&](const char* qb, const uint32_t (&wp)[8], const uint32_t (&wd)[8]) __attribute__((always_inline)) {
    const char* gb = qb + R::kBlkBytes;
    bf16x8 ga[2], qa[2];
    ga[0] = read_tr<D>(gb, off, 0, 0);
    qa[0] = read_tr<D>(qb, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 2 * (D / 32); ++i) {   // i = cc * (D/32) + db
      const int cc = i / (D / 32), db = i % (D / 32);
      if (i + 1 < 2 * (D / 32)) {
        ga[(i + 1) & 1] = read_tr<D>(gb, off, (i + 1) / (D / 32), (i + 1) % (D / 32));
        qa[(i + 1) & 1] = read_tr<D>(qb, off, (i + 1) / (D / 32), (i + 1) % (D / 32));
      }
      const bf16x8 bp = __builtin_bit_cast(bf16x8, (u32x4){wp[4 * cc], wp[4 * cc + 1], wp[4 * cc + 2], wp[4 * cc + 3]});
      const bf16x8 bd = __builtin_bit_cast(bf16x8, (u32x4){wd[4 * cc], wd[4 * cc + 1], wd[4 * cc + 2], wd[4 * cc + 3]});
      adv[db] = mfma(ga[i & 1], bp, adv[db]);
      adk[db] = mfma(qa[i & 1], bd, adk[db]);
    }
  };

  // Software pipeline: step n computes S, dP of block n+1 on the MFMA unit
  // while the VALU turns block n's S, dP into P and dS, then runs block n's
  // dV and dK products.
  f32x16 s_cur, dp_cur;
  if (nblk > 0) {
#pragma unroll
    for (int n = 0; n < kDepthKV - 1; ++n) issue(n);
    wait_block(std::integral_constant<int, kDepthKV - 2>{});   // block 0
    __syncthreads();
    Rows qa, ga;
    sdp_read(stage_of(0), qa, ga);
    sdp(qa, ga, s_cur, dp_cur);
  }
  for (int n = 0; n < nblk; ++n) {
    wait_block(std::integral_constant<int, kDepthKV - 3>{});   // block n+1
    __syncthreads();   // everyone's copies of block n+1; block n-1's stage is free
    issue(n + kDepthKV - 1);
    // (past the last block, S and dP come from the stage of a copy that
    // fetched nothing: finite values, discarded)
    f32x16 s_nxt, dp_nxt;
    uint32_t wp[8], wd[8];
    Rows qa, ga;
    sdp_read(stage_of(n + 1), qa, ga);
    if (!Dense && block_full(n)) {
      sdp(qa, ga, s_nxt, dp_nxt);
      softmax_grad(std::true_type{}, n, s_cur, dp_cur, wp, wd);
      interleave(std::integral_constant<int, 6>{});
    } else {
      sdp(qa, ga, s_nxt, dp_nxt);
      softmax_grad(std::false_type{}, n, s_cur, dp_cur, wp, wd);
      interleave(std::integral_constant<int, 10>{});
    }
    dvdk(stage_of(n), wp, wd);
    s_cur = s_nxt;
    dp_cur = dp_nxt;
  }
  wait_copies<0>();   // no copy may still be writing LDS when the workgroup ends
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

// ---------------------------------------------------------------- dk, dv
// d = 128: one workgroup of 8 wave64s per 256 keys, 32 keys per wave. A wave keeps its
// keys' K in registers as B operands and the dK, dV accumulators; its keys'
// V stays in LDS (a 32-row block per wave, copied once) and is read as the B
// operand of dP. That keeps a wave within the 256 registers of two waves per
// SIMD, so one wave's softmax work and waits run under the other's MFMAs.
// Dense: as in the dQ kernel; each wave copies, per block, the words of the
// block's 32 rows that hold its own 32 keys.
// Mode 2 (Sparse): each group of 4 waves (128 keys) is one key block of the
// mask; the WG walks the 32-row query blocks of the 256-row tiles that keep
// any of its blocks. Each list entry carries the query block and a mask of
// the waves that take part.
constexpr int kWavesKV = 8;
constexpr int kTileKV = kBlk * kWavesKV;   // keys per dK/dV workgroup (d = 128)

template <int D, int Mode>   // 0: rules only; 1: dense mask (Dense); 2: block-sparse (Sparse)
__global__ __launch_bounds__(64 * kWavesKV) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const f32x2* __restrict__ stats, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int H, int N_q, int N_k, float c, float scale, int causal, int coff,
    const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_kt, DenseMask dm,
    BlockMask bmk) {
  constexpr bool Dense = Mode == 1, Sparse = Mode == 2;
  static_assert(D == 128, "d = 64 runs attn_bwd_dkdv_pipe_kernel");
  constexpr int kThreadsKV = 64 * kWavesKV;
  using R = Ring<D, kWavesKV>;
  constexpr int kMaskBytes = Dense ? kWavesKV * 256 : 0;
  // [Q block][dO block][stats of the 32 rows][mask words of each wave]
  constexpr int kStage = 2 * R::kBlkBytes + 1024 + kMaskBytes;
  constexpr int kCpb = R::kCpw + (Dense ? 1 : 0);   // copies per wave per block (wave 0: one more)
  constexpr int kVBytes = kWavesKV * R::kBlkBytes;   // the workgroup's V, a block per wave
  constexpr int kListBytes = Sparse ? 4 * (kMaxSparse + kListPad + 4) : 0;
  __shared__ __attribute__((aligned(1024))) char smem[kDepth * kStage + kVBytes + kListBytes];
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  // Under a causal mask early key tiles have the most rows: tile-major order,
  // heaviest first across all heads (see the dq kernel).
  const int n_bh = (int)(gridDim.x / n_kt);
  const int bh = causal ? (int)(blockIdx.x % n_bh) : (int)(blockIdx.x / n_kt);
  const int kt = causal ? (int)(blockIdx.x / n_bh) : (int)(blockIdx.x % n_kt);
  const int b = bh / H;
  int kv = N_k;
  if (seqlens_k) kv = min(max(seqlens_k[b], 0), N_k);
  int qs = 0;
  if (q_start) qs = min(max(q_start[b], 0), N_q);
  const size_t q_base = (size_t)bh * N_q * D, k_base = (size_t)bh * N_k * D;
  const int k0 = kt * kTileKV;
  // query rows that can see a key of this tile: [r_begin, N_q)
  int r_begin = max(qs, causal ? max(k0 - coff, 0) : 0);   // row i sees keys <= i + coff
  if (k0 >= kv) r_begin = N_q;                  // every key of the tile is masked
  const int blk0 = r_begin / kBlk;
  int nblk = r_begin < N_q ? (N_q + kBlk - 1) / kBlk - blk0 : 0;
  // Sparse: list entries blk | (wave mask << 24) of the kept query blocks,
  // padded with the block past the last row (its copies fetch nothing)
  [[maybe_unused]] int* lst = (int*)(smem + kDepth * kStage + kVBytes);
  if constexpr (Sparse) {
    const int nbq = (N_q + kBlk - 1) / kBlk;   // 32-row query blocks of the head
    if (wave == 0) {
      const uint8_t* fl = bmk.flags + (size_t)b * bmk.sb + (size_t)(bh - b * H) * bmk.sh;
      const int kb0 = kt * (kWavesKV / 4);     // the tile's 128-key blocks of the mask: 4 waves each
      int base = 0;
      for (int t0 = blk0 / 8; t0 * 8 < nbq && nblk > 0; t0 += 64) {   // 256-row tiles, one per lane
        const int t = t0 + lane;
        uint32_t wm = 0;
        if (t * 8 < nbq) {
#pragma unroll
          for (int kb = 0; kb < kWavesKV / 4; ++kb)
            if (kb0 + kb < bmk.n_ks && fl[(size_t)t * bmk.n_ks + kb0 + kb] != 0) wm |= 0x0fu << (4 * kb);
        }
        const int lo = max(8 * t, blk0), hi = min(8 * t + 8, nbq);
        const int cnt = (wm != 0 && hi > lo) ? hi - lo : 0;
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int x = __shfl_up(incl, o, 64);
          if (lane >= o) incl += x;
        }
        int pos = base + incl - cnt;
        for (int q = lo; q < lo + cnt; ++q) lst[pos++] = q | (int)(wm << 24);
        base += __shfl(incl, 63, 64);
      }
      if (lane < kListPad) lst[base + lane] = nbq;
      if (lane == 0) lst[kMaxSparse + kListPad] = base;
    }
    __syncthreads();
    nblk = __builtin_amdgcn_readfirstlane(lst[kMaxSparse + kListPad]);
  }
  // first query row of ring position n, and whether this wave's slice takes part
  auto row0_of = [&](int n) __attribute__((always_inline)) {
    if constexpr (Sparse) return (__builtin_amdgcn_readfirstlane(lst[n]) & 0xffffff) * kBlk;
    else return (blk0 + n) * kBlk;
  };
  [[maybe_unused]] auto row0_of_lane = [&](int i) __attribute__((always_inline)) {   // per-lane entry
    return (lst[i] & 0xffffff) * kBlk;
  };
  auto wave_in = [&](int n) __attribute__((always_inline)) {
    if constexpr (Sparse) return ((__builtin_amdgcn_readfirstlane(lst[n]) >> (24 + wave)) & 1) != 0;
    else return true;
  };

  const int wkey0 = k0 + kBlk * wave;   // this wave's first key
  const int key = wkey0 + (lane & 31);
  const bool key_ok = key < N_k, key_live = key < kv;
  const bool wkey_live = wkey0 + kBlk <= kv;   // all 32 keys of the wave are valid
  bf16x8 kr[D / 16];   // this key's K as B operands (zeros past the valid length)
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 a = {0u, 0u, 0u, 0u};
    if (key_live) a = *(const u32x4*)(K + k_base + (size_t)key * D + kc * 16 + hf * 8);
    kr[kc] = __builtin_bit_cast(bf16x8, a);
  }

  wait_loads();
  // Rows past N_q (and keys past kv) fetch nothing: zero the ring and the V
  // blocks once, so such rows hold zeros or rows of an earlier block (finite)
  // and are masked out below.
  for (int i = tid; i < (kDepth * kStage + kVBytes) / 16; i += kThreadsKV)
    *(lds_u32x4*)(smem + 16 * i) = (u32x4){0u, 0u, 0u, 0u};
  __syncthreads();
  const uint32_t rows_bytes = (uint32_t)N_q * 2 * D;
  const i32x4 q_rs = rsrc(Q + q_base, rows_bytes), g_rs = rsrc(dO + q_base, rows_bytes);
  const i32x4 s_rs = rsrc(stats + (size_t)bh * N_q, (uint32_t)N_q * 8);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  // this wave's 32 keys of V into its LDS block (keys past kv fetch nothing);
  // awaited by the first block's wait below (copies complete in issue order)
  const char* vblk = smem + kDepth * kStage + wave * R::kBlkBytes;
  {
    const i32x4 v_rs = rsrc(V + k_base, (uint32_t)kv * 2 * D);
    const uint32_t vl = lds0 + kDepth * kStage + wave * R::kBlkBytes;
#pragma unroll
    for (int ci = 0; ci < R::kKB; ++ci)
      copy_kb(v_rs, (uint32_t)wkey0 * 2 * D, copy_lane_off<D>(ci, lane), vl + ci * 1024);
  }
  int cpoff[R::kCpw];
#pragma unroll
  for (int i = 0; i < R::kCpw; ++i) cpoff[i] = copy_lane_off<D>(wave * R::kCpw + i, lane);
  // the stats copy (wave 0): lane L brings bytes 16L .. 16L+15 from the
  // block's first row on, into the stage's 1 KB stats area; the first 256
  // bytes are the block's 32 rows, the rest (later rows, or nothing past N_q)
  // is never read. Its lane offset is made inside the copy (kept in a
  // register across the loop, it was spilled and reloaded with a full vmcnt
  // wait).
  // Dense: lane L < 32 brings, for row r0 + L, the word that holds this wave's keys
  [[maybe_unused]] i32x4 m_rs = {0, 0, 0, 0};
  [[maybe_unused]] uint32_t m_off = 0;
  if constexpr (Dense) {
    m_rs = rsrc(dm.bits + (size_t)b * dm.sb + (size_t)(bh - b * H) * dm.sh, (uint32_t)N_q * dm.rw * 4);
    m_off = lane < 32 ? (uint32_t)lane * dm.rw * 4 + (uint32_t)(wkey0 >> 5) * 4 : 0x40000000u;
  }
  auto issue = [&](int n) {   // the block of ring position n into stage n % kDepth
    const uint32_t st = lds0 + (uint32_t)(n % kDepth) * kStage;
    const uint32_t r0 = (uint32_t)row0_of(n);
#pragma unroll
    for (int i = 0; i < R::kCpw; ++i) {
      const int ci = wave * R::kCpw + i;
      const bool is_g = ci >= R::kKB;
      copy_kb(is_g ? g_rs : q_rs, r0 * 2 * D, cpoff[i], st + (uint32_t)ci * 1024);
    }
    if (wave == 0) copy_kb_lane16(s_rs, r0 * 8, st + 2 * R::kBlkBytes);
    if constexpr (Dense) copy_dw(m_rs, r0 * dm.rw * 4, m_off, st + 2 * R::kBlkBytes + 1024 + wave * 256);
  };
  // Block n has landed once at most the `ahead` newest blocks' copies of this
  // wave are in flight (wave 0 issues one copy more per block).
  auto wait_block = [&](auto ahead) {
    constexpr int A = decltype(ahead)::value;
    if (wave == 0) wait_copies<A * (kCpb + 1)>();
    else wait_copies<A * kCpb>();
  };

  const Offs<D> off0(lane);
  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) adk[db] = adv[db] = (f32x16){};
  // Block n needs no mask for this wave when all its keys are valid, all
  // rows exist and are past q_start, and (causal) the block starts at or
  // after the wave's last key (block-sparse: and the wave's slice is kept).
  // The rows of the blocks increase with n, so these blocks are one range
  // [n_full0, n_full1) per wave; the loop runs in three parts (masked, no
  // mask, masked), each with one copy of the block code, which keeps the
  // accumulators' registers the same throughout.
  auto count_below = [&](int t) {   // ring positions n < nblk whose first row is below t
    if (t <= 0) return 0;
    if constexpr (Sparse) {
      int cnt = 0;
      for (int i = lane; i < nblk; i += 64) cnt += row0_of_lane(i) < t ? 1 : 0;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
      return __builtin_amdgcn_readfirstlane(cnt);
    } else {
      return min(max((t + kBlk - 1) / kBlk - blk0, 0), nblk);
    }
  };
  int n_full0 = nblk, n_full1 = nblk;
  if (!Dense && wkey_live) {
    n_full0 = count_below(max(qs, causal ? wkey0 + kBlk - 1 - coff : 0));
    n_full1 = max(count_below(N_q - kBlk + 1), n_full0);
  }

#pragma unroll
  for (int n = 0; n < kDepth - 1; ++n) issue(n);
  auto block = [&](int n, auto full_t) __attribute__((always_inline)) {
    wait_block(std::integral_constant<int, kDepth - 2>{});   // block n (and, before block 0, the V blocks)
    __syncthreads();   // everyone's copies of block n; block n-1's stage is free
    issue(n + kDepth - 1);
    if constexpr (Sparse && decltype(full_t)::value) {
      if (!wave_in(n)) return;   // the wave's slice is dropped: nothing to add
    }
    const int r0 = row0_of(n);
    // The block in an explicit order of slots, each one MFMA with the reads
    // and the arithmetic placed after it (scheduling fences between them), so
    // that a wave's softmax arithmetic overlaps its own MFMAs: P while the dP
    // products run, dS while the dV products run.
    auto step = [&](auto full_t) __attribute__((always_inline)) {
      constexpr bool F = decltype(full_t)::value;
      // The stage offset and the lane offsets pass through this marker, so
      // that every address is formed next to its read instead of two dozen
      // of them being held in registers across the loop.
      uint32_t so = (uint32_t)(n % kDepth) * kStage;
      Offs<D> off = off0;
      if constexpr (F)
        asm volatile("; dkdv block, no mask" : "+s"(so), "+v"(off.row0), "+v"(off.tr[0]), "+v"(off.tr[1]));
      else
        asm volatile("; dkdv block, masked" : "+s"(so), "+v"(off.row0), "+v"(off.tr[0]), "+v"(off.tr[1]));
      const char* qb = (const char*)smem + so;
      const char* gb = qb + R::kBlkBytes;
      // register r of S, dP (and P, dS) belongs to query row r0 + 8*(r/4) + 4*hf + r%4,
      // whose (LSE log2 e, D) pair sits at floats 16*(r/4) + 2*(r%4) + 0, 1 of st
      const lds_f32* st = (const lds_f32*)(qb + 2 * R::kBlkBytes + 32 * hf);
      auto sti = [](int r) { return 16 * (r / 4) + 2 * (r % 4); };
      auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
      [[maybe_unused]] const bool in = wave_in(n);
      [[maybe_unused]] const char* mb = qb + 2 * R::kBlkBytes + 1024 + wave * 256;   // Dense: row r0 + t at 4*t
      constexpr int kKC = D / 16;       // MFMAs of S (and of dP)
      constexpr int kJ = 4 * (D / 32);  // MFMAs of dV and dK
      static_assert(kKC == 8, "eight pairs of P elements, one per dP MFMA");

      // S = Q K^T (lane = key, 16 query rows per lane); operands are read two
      // slots ahead of their MFMA (dO and V one slot with a dense mask, whose
      // words take the registers)
      constexpr int kPF = Dense ? 1 : 2;
      f32x16 s = {}, dp = {};
      bf16x8 qa[3], ga[3], va[3], ta[3];
      float l2[2], dd[2];
      qa[0] = read_row<D>(qb, off, 0);
      qa[1] = read_row<D>(qb, off, 1);
      fence();
#pragma unroll
      for (int kc = 0; kc < kKC; ++kc) {
        if (kc + 2 < kKC) qa[(kc + 2) % 3] = read_row<D>(qb, off, kc + 2);
        if (kc + kPF >= kKC) {
          ga[kc + kPF - kKC] = read_row<D>(gb, off, kc + kPF - kKC);
          va[kc + kPF - kKC] = read_row<D>(vblk, off0, kc + kPF - kKC);
        }
        s = mfma(qa[kc % 3], kr[kc], s);
        fence();
      }
      // P of elements 2i, 2i+1 = exp2(S c - LSE log2 e), 0 where masked; packed
      // as a B operand of dV
      float p[16];
      uint32_t wp[8], wd[8];
      [[maybe_unused]] u32x4 mw[2] = {};   // Dense: the words of rows 8g + 4hf .. +3
      auto p_pair = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          const float x = s[r] * c - l2[e];
          if constexpr (F) {
            p[r] = __builtin_amdgcn_exp2f(x);
          } else {
            const int qrow = r0 + 8 * (r / 4) + 4 * hf + r % 4;
            bool ok = key_live && qrow < N_q && qrow >= qs && (!causal || key <= qrow + coff);
            if constexpr (Sparse) ok = ok && in;
            if constexpr (Dense) ok = ok && ((mw[(r / 4) & 1][r % 4] >> (lane & 31)) & 1u);
            p[r] = ok ? __builtin_amdgcn_exp2f(x) : 0.f;
          }
        }
        wp[i] = pack2(p[2 * i], p[2 * i + 1]);
      };
      // dS of elements 2i, 2i+1 = P (dP - D); a masked element has P = 0 and
      // gives 0 even where dP - D is not finite (rows before q_start hold
      // whatever the caller left there)
      auto ds_pair = [&](int i) __attribute__((always_inline)) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          ds[e] = p[r] * (dp[r] - dd[e]);
          if constexpr (!F) ds[e] = p[r] != 0.f ? ds[e] : 0.f;
        }
        wd[i] = pack2(ds[0], ds[1]);
      };
      // dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by the transposing read),
      // product j: dV for j < kJ/2, dK after; chunk (16 rows) m % 2, column block j % (D/32)
      auto tr_of = [&](int j) __attribute__((always_inline)) {
        const int m = j / (D / 32);
        return read_tr<D>(m >= 2 ? qb : gb, off, m & 1, j % (D / 32));
      };
      // dP = dO V^T. Slot kc: its MFMA; the next operands and the stats of pair
      // kc; then P of pair kc - 1 (pair 0 waits a slot for S to land).
#pragma unroll
      for (int kc = 0; kc < kKC; ++kc) {
        dp = mfma(ga[kc % 3], va[kc % 3], dp);
        fence();
        if (kc + kPF < kKC) {
          ga[(kc + kPF) % 3] = read_row<D>(gb, off, kc + kPF);
          va[(kc + kPF) % 3] = read_row<D>(vblk, off0, kc + kPF);
        }
        if (kc + 2 >= kKC) ta[kc + 2 - kKC] = tr_of(kc + 2 - kKC);
        if constexpr (Dense) {
          if (kc % 2 == 0) mw[(kc / 2) & 1] = *(const lds_u32x4*)(mb + 32 * (kc / 2) + 16 * hf);
        }
        float l2n[2] = {st[sti(2 * kc)], st[sti(2 * kc + 1)]};
        fence();
        if (kc > 0) p_pair(kc - 1);
        l2[0] = l2n[0];
        l2[1] = l2n[1];
        fence();
      }
      // Slot j: its MFMA; the next operand and the D values of pair j; then P
      // of pair 7 (j = 0) or dS of pair j - 1. The dV products use P of chunk
      // m % 2 (ready), the dK products from j = kJ/2 on find dS done.
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int m = j / (D / 32), cc = m & 1, db = j % (D / 32);
        if (m >= 2) {
          const bf16x8 bd =
              __builtin_bit_cast(bf16x8, (u32x4){wd[4 * cc], wd[4 * cc + 1], wd[4 * cc + 2], wd[4 * cc + 3]});
          adk[db] = mfma(ta[j % 3], bd, adk[db]);
        } else {
          const bf16x8 bp =
              __builtin_bit_cast(bf16x8, (u32x4){wp[4 * cc], wp[4 * cc + 1], wp[4 * cc + 2], wp[4 * cc + 3]});
          adv[db] = mfma(ta[j % 3], bp, adv[db]);
        }
        fence();
        if (j + 2 < kJ) ta[(j + 2) % 3] = tr_of(j + 2);
        float ddn[2];
        if (j < 8) {
          ddn[0] = st[sti(2 * j) + 1];
          ddn[1] = st[sti(2 * j + 1) + 1];
        }
        fence();
        if (j == 0) p_pair(kKC - 1);
        else if (j <= 8) ds_pair(j - 1);
        if (j < 8) {
          dd[0] = ddn[0];
          dd[1] = ddn[1];
        }
        fence();
      }
      if constexpr (F) asm volatile("; dkdv block end, no mask");
      else asm volatile("; dkdv block end, masked");
    };
    step(full_t);
  };
  int n = 0;
  for (; n < n_full0; ++n) block(n, std::false_type{});
  if constexpr (!Dense)
    for (; n < n_full1; ++n) block(n, std::true_type{});
  for (; n < nblk; ++n) block(n, std::false_type{});
  wait_copies<0>();   // no copy may still be writing LDS when the workgroup ends
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

// Device address of the allocation-free entry point's row-statistics array
// on the device of `stream` (declared below); looked up once per device.
int scratch_address(hipStream_t stream, float** out);

// delta == nullptr with own_delta: the row statistics go to the library's own
// array (attn_bwd_noalloc); its address is taken after every argument check.
int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N_q, int N_k, int d, float scale,
               int causal, const int32_t* seqlens_k, const int32_t* q_start, DenseMask dm, BlockMask bmk,
               hipStream_t stream, bool own_delta = false) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (causal < 0 || causal > 2) return ATTN_ERR_MASK;
  const long long bh = (long long)B * H;
  if (bh == 0 || (N_q == 0 && N_k == 0)) return ATTN_OK;
  const bool has_q = N_q > 0, has_k = N_k > 0;
  if (has_q && (!q || !o || !dout || !lse || !dq || (!delta && !own_delta))) return ATTN_ERR_NULL;
  if (has_k && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (bh > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const int tkv = d == 128 ? kTileKV : kTile;   // keys per dK/dV workgroup
  const int tq = kBlk * waves_q(d);   // query rows per dQ workgroup
  const long long n_qt = (N_q + tq - 1) / tq, n_kt = (N_k + tkv - 1) / tkv;
  if (bh * n_qt > 0x7fffffffLL || bh * n_kt > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  // per-head byte offsets of the copies are 32-bit
  if ((long long)(N_q + 256) * d * 2 > 0x7fffffffLL || (long long)(N_k + tkv) * d * 2 > 0x7fffffffLL)
    return ATTN_ERR_SHAPE;
  const size_t qb = (size_t)bh * N_q * d * 2, kb = (size_t)bh * N_k * d * 2, rb = (size_t)bh * N_q * 4;
  if (((uintptr_t)q | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq) & 15) return ATTN_ERR_ALIGN;
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)dk | (uintptr_t)dv) & 15) return ATTN_ERR_ALIGN;
  if (((uintptr_t)lse & 3) || ((uintptr_t)delta & 7)) return ATTN_ERR_ALIGN;
  const void* ins[] = {q, k, v, o, dout, lse};
  const size_t in_n[] = {qb, kb, kb, qb, qb, rb};
  void* outs[] = {dq, dk, dv, delta};
  const size_t out_n[] = {qb, kb, kb, 2 * rb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return ATTN_ERR_ALIAS;
  }

  if (own_delta && has_q) {
    const int st = scratch_address(stream, &delta);
    if (st != ATTN_OK) return st;
  }

  const float c = scale * kLog2e;
  int causal01 = causal ? 1 : 0, coff = causal == 2 ? N_k - N_q : 0, Hi = H, Nq = N_q, Nk = N_k;
  float cc = c, sc = scale;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v,
                 *op = (const uint16_t*)o, *gp = (const uint16_t*)dout;
  uint16_t *dqp = (uint16_t*)dq, *dkp = (uint16_t*)dk, *dvp = (uint16_t*)dv;
  f32x2* stp = (f32x2*)delta;
  hipError_t e = hipSuccess;
  if (has_q) {
    long long rows = bh * N_q;
    const long long per = 256 / (d / 8);
    const long long nb = (rows + per - 1) / per;
    if (nb > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    e = attn_launch::launch(d == 128 ? attn_bwd_delta_kernel<128> : attn_bwd_delta_kernel<64>, dim3((unsigned)nb),
                            dim3(256), stream, op, gp, lse, stp, rows);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
    const int mode = dm.bits ? 1 : bmk.flags ? 2 : 0;
    auto kq = d == 128 ? (mode == 1 ? attn_bwd_dq_kernel<128, 1> : mode == 2 ? attn_bwd_dq_kernel<128, 2>
                                                                             : attn_bwd_dq_kernel<128, 0>)
                       : (mode == 1 ? attn_bwd_dq_kernel<64, 1> : mode == 2 ? attn_bwd_dq_kernel<64, 2>
                                                                            : attn_bwd_dq_kernel<64, 0>);
    e = attn_launch::launch(kq, dim3((unsigned)(bh * n_qt)), dim3(64 * waves_q(d)), stream, qp, kp, vp, gp, (const f32x2*)stp,
                            dqp, Hi, Nq, Nk, cc, sc, causal01, coff, seqlens_k, q_start, (int)n_qt, dm, bmk);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  if (has_k) {
    const int mode = dm.bits ? 1 : bmk.flags ? 2 : 0;
    // d = 128: 8-wave workgroups of 256 keys; d = 64: the pipelined 4-wave kernel, 128 keys
    auto kk = d == 128 ? (mode == 1 ? attn_bwd_dkdv_kernel<128, 1> : mode == 2 ? attn_bwd_dkdv_kernel<128, 2>
                                                                               : attn_bwd_dkdv_kernel<128, 0>)
                       : (mode == 1 ? attn_bwd_dkdv_pipe_kernel<64, 1> : mode == 2 ? attn_bwd_dkdv_pipe_kernel<64, 2>
                                                                                   : attn_bwd_dkdv_pipe_kernel<64, 0>);
    e = attn_launch::launch(kk, dim3((unsigned)(bh * n_kt)), dim3(d == 128 ? 64 * kWavesKV : kThreads), stream, qp, kp,
                            vp, gp, (const f32x2*)stp, dkp, dvp, Hi, Nq, Nk, cc, sc, causal01, coff, seqlens_k, q_start,
                            (int)n_kt, dm, bmk);
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N_q,
                        int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                        const int32_t* q_start, hipStream_t stream) {
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start,
                    DenseMask{nullptr, 0, 0, 0}, BlockMask{nullptr, 0, 0, 0}, stream);
}

extern "C" int attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H,
                               int N_q, int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                               const int32_t* q_start, const uint32_t* mask_bits, long long mask_stride_b,
                               long long mask_stride_h, int mask_row_words, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  const bool work = (long long)B * H > 0 && (N_q > 0 || N_k > 0);
  if (!mask_bits) return work ? ATTN_ERR_NULL : ATTN_OK;
  if ((uintptr_t)mask_bits & 15) return ATTN_ERR_ALIGN;
  if (mask_row_words < (N_k + 31) / 32 || mask_row_words % 8 != 0 || mask_stride_b < 0 || mask_stride_h < 0)
    return ATTN_ERR_MASK;
  if ((long long)(N_q + 256) * mask_row_words * 4 > 0x7fffffffLL) return ATTN_ERR_SHAPE;   // 32-bit offsets
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start,
                    DenseMask{mask_bits, mask_stride_b, mask_stride_h, mask_row_words}, BlockMask{nullptr, 0, 0, 0},
                    stream);
}

extern "C" int attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                     const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H,
                                     int N_q, int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                                     const int32_t* q_start, const uint8_t* block_mask, long long block_stride_b,
                                     long long block_stride_h, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  const bool work = (long long)B * H > 0 && (N_q > 0 || N_k > 0);
  if (!block_mask) return work ? ATTN_ERR_NULL : ATTN_OK;
  if (block_stride_b < 0 || block_stride_h < 0) return ATTN_ERR_MASK;
  if ((N_k + kBlk - 1) / kBlk > kMaxSparse || (N_q + kBlk - 1) / kBlk > kMaxSparse) return ATTN_ERR_SHAPE;   // lists
  const int n_ks = (N_k + kTile - 1) / kTile;   // 128-key blocks per row of the block mask
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start,
                    DenseMask{nullptr, 0, 0, 0}, BlockMask{block_mask, block_stride_b, block_stride_h, n_ks}, stream);
}

// ---------------------------------------------------- allocation-free backward
// attn_bwd_noalloc is attn_bwd with the per-row (LSE * log2 e, Delta) pairs
// kept in `scratch`, a library-owned array of this size (one copy on every GPU
// the library runs on, resident until the process ends), for callers that
// cannot allocate device memory. On the host the array's name only stands in
// for the symbol: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is ever
// handed to a kernel. The delta kernel writes every row it covers before the
// dQ and dK/dV kernels read them, so nothing has to be cleared between calls.
// Two calls that overlap in time on one GPU share the array and race.
namespace {
constexpr long long kNoAllocRows = 1LL << 20;   // B * H * N_q at most: 8 MiB of float pairs
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) float scratch[2 * kNoAllocRows];

namespace {
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices];   // device address of `scratch` per device, null until looked up

int scratch_address(hipStream_t stream, float** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_LAUNCH;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return ATTN_ERR_LAUNCH;
    g_scratch[dev] = (float*)p;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}
}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N_q, int N_k,
                                int d, float scale, int causal, const int32_t* seqlens_k, const int32_t* q_start,
                                hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if ((long long)B * H * N_q > kNoAllocRows) return ATTN_ERR_SCRATCH;
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start,
                    DenseMask{nullptr, 0, 0, 0}, BlockMask{nullptr, 0, 0, 0}, stream, true);
}
