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
// over key/value blocks): one workgroup of 8 wave64s (two per SIMD) owns a
// pair of 256-row query tiles of one (batch, head), processed one after the
// other; each wave owns 32 rows of the tile. Under a causal mask the pair is
// (t, n-1-t), so every workgroup carries the same number of key slices;
// without a causal mask or per-batch lengths all tiles are equal and a
// workgroup owns a single tile, the tiles of a head going to workgroups that
// run at the same time on one XCD (one K/V read from HBM serves them). The
// workgroup walks the 32-key K/V slices its rows can see; slices above the
// causal diagonal and past the batch's valid key length are never visited,
// and a wave stops computing at the last slice its own rows can see. When a
// launch has more such slots than the GPU has CUs and all carry the same work
// (rules only, d = 128, no per-batch lengths), one workgroup per CU walks its
// share of them; a tile spanning whole turns of the ring then fetches the next
// tile's first K/V slices (the next head's included) during its last steps.
//
// Data movement ([MEMWALL] §4.3 double buffering, here an 8-deep ring;
// [PT2CUDA] step 5): K and V slices go from global memory straight into LDS
// with 16-byte buffer_load ... lds copies, no register staging. Each wave
// issues its share of the copy of slice h+7 during step h, into
// the stage slice h-1 used; one barrier per step publishes the landed slices
// and frees that stage. Inside a stage, row r's 16-byte chunk c sits at chunk
// position c ^ swz(r), so the MFMA operand reads (ds_read_b128 for K, the
// transposing ds_read_b64_tr_b16 for V) touch distinct banks.
//
// Per K/V slice, per wave (the online softmax of [PT2CUDA] step 3.1 and
// [MEMWALL] §3.2, in the exp2 domain with c = |scale| * log2(e)):
//   S^T = K Q^T on MFMA 32x32x16 bf16 -> fp32. Computing the transpose puts one
//         query row in each lane (16 keys per lane, the other 16 keys of the
//         slice in lane ^ 32): a row max is an in-register max plus one
//         permlane32 swap, and the row sum needs no cross-lane step until the
//         very end.
//   mask  only on slices that cross the causal diagonal (j <= i, or j <= i +
//         N_k - N_q when aligned bottom-right), the valid key length
//         or the masked leading rows: the score becomes -inf.
//   m     the exponent's subtrahend per row. The first slice sets it to that
//         slice's row max. After that it is a stale running max: it is raised
//         only when a lane's 16 exponentials of a slice add up to more than
//         kSumCap (2^8), and then to the slice's row max, with l and O scaled
//         by exp2(m_old - m_new) and the slice's exponentials redone. The sum
//         bounds every term, so the exponentials stay below 2^8 without
//         taking a row max per slice. O / l does not depend on the subtrahend,
//         so this is the pages' recurrence in exact arithmetic. A row whose m
//         is still -inf (no allowed key in the slices seen so far: under the
//         rule masks that means none at all, under a dense mask its first keys
//         may be masked) uses the subtrahend 0 until a rescale sets m, and its
//         LSE counts that 0.
//   P     = exp2(S*c - m) in fp32, summed into l in fp32, then rounded to bf16.
//         Its accumulator layout is already the B operand layout of the next
//         MFMA, so P never leaves registers.
//   O^T  += V^T P^T on MFMA 32x32x16 bf16 -> fp32, V^T read from LDS with the
//         transposing read.
// The loop is software pipelined inside each wave: while the MFMA unit
// computes S for slice h+1, the VALU exponentiates the second half of slice h;
// while it computes O += P V for slice h, the VALU forms S*c - m of slice h+1
// and exponentiates its first half. The two waves of a SIMD run the same
// phases at the same time (one barrier per slice keeps them in step) and
// interleave their MFMAs and VALU work.
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
#include <atomic>
#include <type_traits>
#include <utility>

#include "attn.h"
#include "launch.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kSlice = 32;     // keys per K/V slice (one LDS stage, one pipeline step)
constexpr int kRB = 1;         // 32-row MFMA blocks (query rows / 32) per wave
constexpr int kRows = 32 * kRB;           // query rows per wave
constexpr float kSumCap = 256.f;   // bound on a lane's 16 exponentials of one slice (2^8)
constexpr float kLn2 = 0.69314718055994530942f;

// Workgroup shape. W = 8: one workgroup of 8 waves (256 query rows) per CU,
// the two waves of each SIMD from the same workgroup. W = 4: 4 waves (128
// query rows) per workgroup and two workgroups per CU, each with its own ring
// in half the LDS: the two waves of a SIMD then belong to different
// workgroups and do not meet at the same barriers, so one workgroup's barrier
// and LDS waits, and its tile prologue and epilogue, run under the other's
// MFMAs. The ring is 8 slices deep either way, so W = 4 needs d = 64 (64 KB of
// stages per workgroup); at d = 128 the 80 KB per workgroup would allow only
// 5 stages, too shallow to cover the copy latency.
template <int D, int W>
struct Slice {
  static constexpr int kWaves = W;                           // wave64s per workgroup
  static constexpr int kBM = kRows * W;                      // query rows per workgroup (one tile)
  static constexpr int kThreads = 64 * W;
  static constexpr int kStages = 8;                          // LDS ring depth in slices
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kBytes = kSlice * kRowBytes;          // one K or V stage
  static constexpr int kLds = 2 * kStages * kBytes;          // K stages, then V stages
  static constexpr int kCopies = kBytes / 1024;              // 1 KB wave copies per stage
  static constexpr int kCopyWaves = kCopies < kWaves ? kCopies : kWaves;   // waves that copy
  static constexpr int kCopiesPerWave = kCopies / kCopyWaves;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kLanesPerRow = 64 / kRowsPerCopy;
  static_assert(kCopies % kCopyWaves == 0, "copies must split evenly over the copying waves");
  static_assert(kLds * (W == 4 ? 2 : 1) <= 160 * 1024, "the workgroups' stages must fit the 160 KB LDS of a CU");
};

// Workgroup shape of each kernel instance (see Slice): the rules-only forward
// at d = 64 runs two 4-wave workgroups per CU; the others keep 8-wave
// workgroups (the dense-mask and block-sparse instances lay out their mask
// words and block flags per 256-row tile).
constexpr int waves_of(int mode, int d) { return mode == 0 && d == 64 ? 4 : 8; }

// Chunk position of 16-byte chunk c of row r is c ^ swz(r). The banks sweep
// 256 bytes. Two read patterns must stay conflict-free:
//   K (ds_read_b128): 16 consecutive rows read the same logical chunk, so the
//     16 rows must land on 16 distinct chunk positions of a sweep;
//   V (ds_read_b64_tr_b16): each half-wave reads an aligned 64-byte group
//     (4 chunks) of 4 consecutive rows 4a..4a+3, so those 4 rows must land on
//     4 distinct 64-byte groups of a sweep.
// D = 128 (one row per sweep): swz = (r%4)*4 + (r/4)%4; bits 2-3 separate the
// 4 rows of a V group, and all 4 bits together separate 16 rows.
// D = 64 (two rows per sweep, row bit 0 picks the half): swz = bit 2 from
// row bit 1, bits 0-1 from row bits 2-3; within a half the 8 rows of the
// same parity get distinct swizzles, and rows 4a, 4a+2 (and 4a+1, 4a+3) differ
// in bit 2, the 64-byte group bit.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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

// MFMA 32x32x16 bf16 -> fp32, issued as inline assembly so that each
// operand's register class is fixed: every operand and accumulator in VGPRs.
// A kernel that uses no AGPRs gets the whole 256-register budget of two waves
// per SIMD as VGPRs; with the K, V and Q operands in AGPRs the budget was
// split 128/128 and spilled operand offsets cost a v_accvgpr_read each per step.
// The compiler does not know these are MFMAs, so the code itself places the
// wait states an MFMA result needs before anything else reads it
// (mfma_result_wait). An MFMA must also not read a register in the 2 wait
// states after a VALU write of it: the Pad forms begin with those wait states
// (used where the compiler materialises operands, in the prologue); in the
// loop no VALU instruction writes an MFMA operand, which the build verifies
// on the compiled code (tiled_attention_16_amd/hazards.py).
template <bool Pad>
__device__ __forceinline__ void mfma_v_init(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (Pad) asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
template <bool Pad>
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (Pad) asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// 24 wait states: more than a 32x32 MFMA result needs before another
// instruction may read it.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Wait until at most N of this wave's LDS reads are in flight (they complete
// in issue order); the compiler sees this wait and drops the ones it implies.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));   // vmcnt, expcnt at their maxima
}
// Wait until at most N of this wave's copies are still in flight (copies
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Dense: a bit-packed boolean mask is intersected with the rule masks. Bit
// j % 32 of word j / 32 of row i (rows of mrw words, mrw a multiple of 8;
// matrix (b, h) at word b*msb + h*msh) set means row i may attend to key j.
// Each wave copies its rows' words for the next 8 slices into LDS with one
// buffer_load ... lds per 8 steps; every slice is masked.
// Sparse (block-sparse attention, [MEMWALL] §7): a byte per (256-row query
// tile, 128-key block, i.e. 4 slices) says whether the block is computed for
// that tile at all (rows of n_ks bytes, n_ks = ceil(N_k / 128), matrix (b, h)
// at byte b*bsb + h*bsh). At each tile
// start wave 0 compacts the tile's set flags into a list of slice indices in
// LDS; the ring walks that list, so unset slices cost neither copies nor
// arithmetic. The rules still mask inside the slices that are computed.
constexpr int kMaxSparseSlices = 1024;   // keys per head up to 32768 on the sparse path
constexpr int kMaxRankedBatches = 64;    // batches ranked by work (one per lane) for the launch order
constexpr int kListPad = 80;             // sentinel entries past the list (the copies look 7 ahead)

template <int D, int Mode>   // Mode 0: rules only; 1: dense mask (Dense); 2: block-sparse (Sparse)
__global__ __launch_bounds__(64 * waves_of(Mode, D), waves_of(Mode, D) == 4 ? 2 : 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int N_q, int N_k, float c, int neg_scale,
    int causal, int coff, const int32_t* __restrict__ seqlens_k, const int32_t* __restrict__ q_start, int n_qt,
    int n_wg, const uint32_t* __restrict__ mbits, long long msb, long long msh, int mrw,
    const uint8_t* __restrict__ bmask, long long bsb, long long bsh, int n_ks) {
  constexpr bool Dense = Mode == 1, Sparse = Mode == 2;
  using T = Slice<D, waves_of(Mode, D)>;
  constexpr int kWaves = T::kWaves, kBM = T::kBM, kThreads = T::kThreads, kStages = T::kStages;
  constexpr int kMaskLds = Dense ? 2 * kWaves * 1024                              // two 8-slice blocks of mask words per wave
                                 : Sparse ? 4 * (kMaxSparseSlices + kListPad + 16)   // the slice list
                                          : 0;
  // Continuation (rules-only, d = 128): see the tile loop below
  constexpr bool kCont = Mode == 0 && D == 128;
  constexpr int kContLds = kCont ? 32 * 1024 : 0;   // with V stage 7: room to stage four waves' O rows
  __shared__ __attribute__((aligned(1024))) char smem[T::kLds + kMaskLds + kContLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int hf = lane >> 5;

  // ---- work decomposition: slots -> (batch*head, query tiles) ----
  // Slot s (0 <= s < n_wg) is a pair of query tiles of one head, or one tile
  // (below). A workgroup
  // takes slots blockIdx.x, blockIdx.x + gridDim.x, ...: one slot when the
  // grid has a workgroup per slot, several when it has one per CU (the host
  // does that only when every slot carries the same work).
  // Without a causal mask or per-batch lengths every tile has the same work:
  // a slot is then one tile, so that the tiles of a head are spread over
  // workgroups that run at the same time (consecutive ids, one XCD below) and
  // read its K/V from L2 once, instead of one workgroup reading it per tile.
  const bool single = !causal && !seqlens_k && !q_start;
  const int n_pairs = single ? n_qt : (n_qt + 1) / 2;   // slots of one head
  const int per_b = H * n_pairs;   // slots of one batch
  const int n_b = n_wg / per_b;    // the batch count
  // Per-batch valid lengths make batches unequal; the slots of one batch are
  // equal. Rank the batches by their work, valid keys times rows that attend
  // (ties by index), and order the slots heaviest batch first: the dispatcher
  // starts workgroups in id order and refills free slots in the same order,
  // so this is a longest-first schedule. Ids are dealt round-robin over the 8
  // XCDs; when the head count allows, whole heads are dealt that way (all
  // n_pairs slots of a head on one XCD, one after another, so its K/V is
  // fetched into one L2) while every XCD still gets the same mix of batches.
  const bool ranked = !causal && (seqlens_k || q_start) && n_b <= kMaxRankedBatches;
  int kv_l = N_k, qs_l = 0, rank = 0;   // lane l: batch l's valid keys, masked rows, rank
  if (ranked) {
    long long wl = -1;   // lane l: the work of batch l
    if (lane < n_b) {
      kv_l = seqlens_k ? min(max(seqlens_k[lane], 0), N_k) : N_k;
      qs_l = q_start ? min(max(q_start[lane], 0), N_q) : 0;
      wl = (long long)kv_l * (N_q - qs_l);
    }
    for (int j = 0; j < n_b; ++j) {
      const long long wj = ((long long)__builtin_amdgcn_readlane((int)(wl >> 32), j) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)wl, j);
      rank += (wj > wl || (wj == wl && j < lane)) ? 1 : 0;
    }
  }
  struct SlotW { int bh, pr, kv, qs; };   // head, tile pair, the batch's valid keys and masked rows (clamped)
  auto slot_of = [&](int sl) __attribute__((always_inline)) {
    SlotW r;
    if (ranked) {
      // j: position in the heaviest-first order (batch rank, head, tile pair)
      int j = sl;
      if (((n_b * H) & 7) == 0) {
        const int x = j & 7, sx = j >> 3;                 // XCD, position within it
        const int gx = sx / n_pairs;
        j = ((gx << 3) + x) * n_pairs + (sx - gx * n_pairs);
      }
      const int r0 = j / per_b;                          // the slot's batch rank
      const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < n_b && rank == r0);
      const int b_r = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
      const int rem = j - r0 * per_b;
      r.bh = b_r * H + rem / n_pairs;
      r.pr = rem % n_pairs;
      r.kv = __builtin_amdgcn_readlane(kv_l, b_r);
      r.qs = __builtin_amdgcn_readlane(qs_l, b_r);
    } else {
      // Consecutive ids are dealt round-robin over the 8 XCDs; regroup so that
      // each XCD gets a contiguous range of (head, tile) pairs and the K/V of
      // a head stay in one XCD's L2 (a grid of one workgroup per CU keeps
      // each workgroup on the XCD of its slots when the CU count is a
      // multiple of 8, which the host checks).
      int lin = sl;
      if ((n_wg & 7) == 0) lin = (lin & 7) * (n_wg >> 3) + (lin >> 3);
      r.bh = lin / n_pairs;
      r.pr = lin - r.bh * n_pairs;
      const int b = r.bh / H;
      r.kv = seqlens_k ? min(max(seqlens_k[b], 0), N_k) : N_k;
      r.qs = q_start ? min(max(q_start[b], 0), N_q) : 0;
    }
    return r;
  };
  // the current item (a query tile): its head, batch, the batch's key bounds
  int bh = 0, b = 0, kv = N_k, qs = 0;

  // ---- K/V slice copies: global -> LDS, 1 KB per wave instruction ----
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
  // Copy slice sl (keys kSlice*sl ..) of a head's K or V into stage dst, with
  // buffer_load_dwordx4 ... lds through a raw buffer descriptor that covers
  // the keys the current tile can see (set per tile, below): lanes whose row
  // is past them fall outside num_records and bring no data (such rows are
  // never used: the mask drops their scores and their probabilities are 0). The byte offset of a lane is
  // sl * kBytes + its fixed in-slice offset, so the head's K (or V) must span
  // less than 2 GB, which the host checks. The copy is issued as inline
  // assembly so that the compiler does not treat it as a pending write to
  // every LDS address (it would then wait for it before each LDS read);
  // completion is awaited explicitly with wait_copies() before the barrier
  // that publishes the slice.
  // LDS address of this wave's share of a stage at stage offset 0; a copy
  // writes M0 = lds_wave + the stage's offset (an immediate), one scalar add
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)smem + (uint32_t)(wave * T::kCopiesPerWave * 1024));
  // (readfirstlane returns a signed int: widen through uint32_t so the low
  // half is zero-extended, never sign-extended into the high half)
  auto sgpr64 = [&](const char* p) __attribute__((always_inline)) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)p >> 32));
    return ((uint64_t)hi << 32) | (uint64_t)lo;
  };
  // descriptor of a head's K or V whose byte 0 is `skip` bytes before `base`
  // and which covers `bytes` bytes from there
  auto rsrc_of = [&](const char* base, uint32_t skip, uint32_t bytes) __attribute__((always_inline)) {
    const uint64_t a = sgpr64(base) - skip;
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)(uint32_t)(a >> 32);   // base bits 32..47; stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);   // num_records, in bytes
    r[3] = 0x00020000;                  // 32-bit data format, no swizzle
    return r;
  };
  // the current item's descriptors, set per item (their empty asm makes them
  // opaque, so the compiler keeps each in its own four SGPRs instead of
  // rebuilding the shared words per copy)
  i32x4 k_rsrc = {0, 0, 0, 0}, v_rsrc = {0, 0, 0, 0};
  // Copy into the stage at byte offset `off` of smem (a compile-time
  // constant: the stage's address is an immediate added to lds_wave, so no
  // stage address is held in a register through the loop).
  auto copy_slice = [&](const i32x4& rs, int sl, auto off) __attribute__((always_inline)) {
    if (T::kCopyWaves < kWaves && wave >= T::kCopyWaves) return;
    constexpr uint32_t kOff = decltype(off)::value;
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)sl * (uint32_t)T::kBytes);
    const uint32_t lw = lds_wave;
#pragma unroll
    for (int q = 0; q < T::kCopiesPerWave; ++q) {
      // (the lane offset is added after the M0 write: that add is the wait
      // state the LDS copy needs after M0 changes)
      const int co = cp_off[q];
      uint32_t voff;
      asm volatile("s_add_u32 m0, %1, %5\n\tv_add_u32 %0, %2, %3\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
                   : "=&v"(voff)
                   : "s"(lw), "s"(soff), "v"(co), "s"(rs), "n"(kOff + q * 1024u)
                   : "memory", "m0", "scc");
    }
  };
  // Slice s lives in stage s % kStages: K rows at kst(st), V rows at vst(st);
  // kso / vso: their byte offsets in smem as compile-time constants.
  auto kst = [&](int st) __attribute__((always_inline)) { return (const char*)smem + st * T::kBytes; };
  auto vst = [&](int st) __attribute__((always_inline)) { return (const char*)smem + (kStages + st) * T::kBytes; };
  auto kso = [](auto st) { return std::integral_constant<uint32_t, (uint32_t)(decltype(st)::value % kStages) * T::kBytes>{}; };
  auto vso = [](auto st) {
    return std::integral_constant<uint32_t, (uint32_t)(kStages + decltype(st)::value % kStages) * T::kBytes>{};
  };
  // the V stage base relative to the folded-in kVBase (see v_off below)
  auto vst_rel = [&](int st) __attribute__((always_inline)) { return (const char*)smem + st * T::kBytes; };
  constexpr int kC = 2 * T::kCopiesPerWave;   // copies per wave per K+V slice
  // K and V of key slice sl into the stage of ring position s (a compile-time
  // std::integral_constant: only its value modulo kStages matters)
  auto copy_slices = [&](auto s, int sl) __attribute__((always_inline)) {
    copy_slice(k_rsrc, sl, kso(s));
    copy_slice(v_rsrc, sl, vso(s));
  };

  // ---- per-lane LDS offsets of the MFMA operand reads ----
  // K (A operand of S^T = K Q^T): lane L reads row L%32 of a slice, logical
  // chunk 2*kc + L/32, at byte r*kRowBytes + ((2kc + L/32) ^ swz(r))*16. The
  // swizzle only flips chunk bits, so the offset for chunk pair kc is
  // k_off0 ^ (32*kc).
  // V (A operand of O^T += V^T P^T, via the transposing read): 16-key chunk cc,
  // half hi: lane L of group g = L/16 supplies row 16*cc + 8*hi + 4*(L/32) +
  // (L%16)/4, columns 32*db + 16*(g%2) + 4*(L%4) .. +3. After the transpose,
  // lane L holds column 32*db + L%32 of keys 16*cc + 8*hi + 4*(L/32) + 0..3,
  // which pairs with P's registers 8*cc + 4*hi + 0..3. Its offset is
  // v_off0 (hi = 0) or v_off1 (hi = 1, row + 8), XORed with 64*db, plus 16*cc
  // rows as an immediate (the swizzle repeats every 16 rows).
  // Every base these are added to is a multiple of 16 rows, so base + (off ^ x)
  // == (base + off) ^ x and the bases stay immediate offsets.
  int k_off0, v_off0, v_off1;
  {
    const int r = lane & 31;
    k_off0 = r * T::kRowBytes + ((hf ^ swz<D>(r)) << 4);
    const int g = lane >> 4;
    const int rv = 4 * hf + ((lane & 15) >> 2);
    const int byte = 32 * (g & 1) + 8 * (lane & 3);
    v_off0 = rv * T::kRowBytes + (((byte >> 4) ^ swz<D>(rv)) << 4) + (byte & 15);
    v_off1 = (rv + 8) * T::kRowBytes + (((byte >> 4) ^ swz<D>(rv + 8)) << 4) + (byte & 15);
  }
  // All operand offsets, kept in registers. The V stages start at
  // kStages * kBytes (64 KB for d = 128), more than a DS immediate holds, so
  // that base is folded into the V offsets (it has no bits below 64 KB, so it
  // commutes with the XORs) and the immediates stay below it.
  constexpr int kVBase = kStages * T::kBytes;
  int k_off[D / 16], v_off[2][D / 32];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) k_off[kc] = k_off0 ^ (32 * kc);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    v_off[0][db] = (v_off0 ^ (64 * db)) + kVBase;
    v_off[1][db] = (v_off1 ^ (64 * db)) + kVBase;
  }

  // A slot is the pair of query tiles (n_qt-1-pr, pr) of a head: under a
  // causal mask their key counts add up to the same total for every pair, so
  // all slots carry equal work and no workgroup is left running alone at the
  // end. The tile with more keys goes first.
  // Lanes whose key row is past kv fetch nothing, so a stage can keep rows no
  // copy wrote. Zero the stages once: such rows then hold zeros or keys of an
  // earlier slice, always finite, and their zero probabilities keep them out.
  for (int i = tid; i < T::kLds / 16; i += kThreads)
    *(__attribute__((address_space(3))) u32x4*)(smem + 16 * i) = (u32x4){0u, 0u, 0u, 0u};
  __syncthreads();
  // keys the rows of query tile t can see (kv_, qs_: its batch's valid keys and masked rows)
  auto kv_end_of = [&](int t, int kv_, int qs_) __attribute__((always_inline)) {
    const int q_end_t = min(t * kBM + kBM, N_q);
    int e = kv_;
    if (causal) e = min(e, max(q_end_t + coff, 0));   // row i sees keys <= i + coff
    if (qs_ >= q_end_t) e = 0;                        // every row of the tile is masked
    return e;
  };
  // ---- Q rows -> VGPRs as the B operand of S^T = K Q^T ----
  // An item's Q rows are loaded once the previous item's last MFMA has read
  // qreg (the first item's before the item loop), so the loads overlap that
  // item's epilogue; nothing reads them until the item's first score product.
  // (Q is loaded at this one point only, so the compiler keeps one set of
  // registers for it and has no copy to make, which would wait for the loads.)
  // Lanes of rows past N_q load row N_q - 1, so every load is unconditional
  // and a load into registers still awaiting earlier loads needs no wait
  // (loads complete in order); such rows are given Q = 0 once the rows have
  // arrived (prep_q), as if they had been loaded as zeros.
  bf16x8 qreg[kRB][D / 16];
  auto load_q = [&](int bh_, int row_lo_t) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int row = min(row_lo_t + 32 * rb + (lane & 31), N_q - 1);
      const u32x4* src = (const u32x4*)(Q + (size_t)bh_ * N_q * D + (size_t)row * D + hf * 8);
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) qreg[rb][kc] = as_bf16x8(src[2 * kc]);
    }
  };
  // At the start of every item that computes, after q_read() (on every path
  // the compiler has then waited for the loads before the slice loop, never
  // inside it): a negative scale negates Q exactly (XOR with 0 otherwise), and
  // rows past N_q get Q = 0, so their scores are 0 whatever their mask words.
  const uint32_t qflip = neg_scale ? 0x80008000u : 0u;
  // a read of the Q registers that stays in order with the copies' asm
  auto q_read = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) asm volatile("" :: "v"(qreg[rb][kc]));
  };
  auto prep_q = [&](int row_lo_t) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const bool pad = row_lo_t + 32 * rb + (lane & 31) >= N_q;
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const u32x4 x = as_u32x4(qreg[rb][kc]) ^ qflip;
        qreg[rb][kc] = as_bf16x8(pad ? (u32x4){0u, 0u, 0u, 0u} : x);
      }
    }
  };
  // The workgroup's items are the tiles of its slots, in order. Continuation
  // (rules-only, d = 128): when a tile spans a whole number of ring turns and
  // another item follows, the tile's last seven steps copy the next item's
  // slices 0..6 into stages 0..6 (they would otherwise fetch nothing), the
  // next item's Q rows are loaded before this tile's epilogue, and that
  // epilogue stages O outside stages 0..6; the next item then starts without
  // refilling the ring, its K/V arriving while this tile still computes.
  // Only the slot and the tile index carry over from one item to the next
  // (the rest is recomputed per item, which keeps scalar registers free
  // through the slice loop).
  int slot = blockIdx.x;
  int it = 0;           // the item's tile in its slot: 0 the one with more keys, 1 the other
  {
    const SlotW s0 = slot_of(slot);
    load_q(s0.bh, (n_qt - 1 - s0.pr) * kBM + kRows * wave);
  }
  bool ahead = false;   // this item's Q and slices 0..6 were issued by the previous item
#pragma nounroll
  for (int item = 0;; ++item) {
  const SlotW cur = slot_of(slot);
  const int pr = cur.pr;
  bh = cur.bh;
  b = bh / H;
  kv = cur.kv;
  qs = cur.qs;
  const int n_mine = (!single && n_qt - 1 - pr != pr) ? 2 : 1;
  // the next item: the slot's other tile, else the first tile of the
  // workgroup's next slot; its head, query tile and visible keys
  const int slot_n = it + 1 < n_mine ? slot : slot + (int)gridDim.x;
  const int it_n = it + 1 < n_mine ? it + 1 : 0;
  const bool has_next = slot_n < n_wg;
  int nbh = 0, qt_n = 0, n_end = 0;
  if (has_next) {
    const SlotW nxt = it_n == 0 ? slot_of(slot_n) : cur;
    nbh = nxt.bh;
    qt_n = it_n == 0 ? n_qt - 1 - nxt.pr : nxt.pr;
    n_end = kv_end_of(qt_n, nxt.kv, nxt.qs);
  }
  const int qt = it == 0 ? n_qt - 1 - pr : pr;
  const int q0 = qt * kBM;
  const int q_end = min(q0 + kBM, N_q);
  const int kv_end = kv_end_of(qt, kv, qs);        // keys this workgroup can see
  // The copies only need the keys the tile can see: keys past kv_end (beyond
  // the causal limit of the tile's last row) come back as nothing.
  k_rsrc = rsrc_of((const char*)(K + (size_t)bh * N_k * D), 0u, (uint32_t)kv_end * T::kRowBytes);
  v_rsrc = rsrc_of((const char*)(V + (size_t)bh * N_k * D), 0u, (uint32_t)kv_end * T::kRowBytes);
  asm volatile("" : "+s"(k_rsrc), "+s"(v_rsrc));

  // This wave's rows: row_lo .. row_lo + 31, one MFMA block of 32 rows; lane L
  // holds row row_lo + L%32 (lanes L and L+32 split that row's keys).
  const int row_lo = q0 + kRows * wave;
  const int row_hi = min(row_lo + kRows - 1, N_q - 1);
  const bool wave_live = row_lo < N_q && row_hi >= qs;
  const size_t q_base = (size_t)bh * N_q * D;

  // slices: nh_wg for the workgroup, nh (a prefix) for this wave
  const int nsl = (kv_end + kSlice - 1) / kSlice;   // slices below kv_end
  int nh_wg = nsl;
  int nh = wave_live ? nh_wg : 0;
  if (causal) nh = min(nh, row_hi + coff < 0 ? 0 : (row_hi + coff) / kSlice + 1);
  nh = __builtin_amdgcn_readfirstlane(nh);
  // this tile's last steps copy the next item's first slices
  const bool cont = kCont && has_next && nsl > 0 && (nsl & (kStages - 1)) == 0;
  // Sparse: the list of the tile's computed slices (ring position -> slice),
  // then nh_wg = its length and nh = its entries at or below this wave's
  // last slice. Entries past the list are nsl: their copies fetch nothing.
  [[maybe_unused]] int* lst = (int*)(smem + T::kLds);
  [[maybe_unused]] int lst_v = 0;   // entries h0 .. h0+63 of the list, one per lane
  if constexpr (Sparse) {
    if (item > 0) __syncthreads();   // every wave is done with the previous tile's list
    if (wave == 0) {
      const uint8_t* fl = bmask + (size_t)b * bsb + (size_t)(bh - b * H) * bsh + (size_t)qt * n_ks;
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int sl = 16 * lane + i;
        if (sl < nsl && fl[sl >> 2] != 0) bits |= 1u << i;   // a flag covers 4 slices (128 keys)
      }
      const int cnt = __builtin_popcount(bits);
      int incl = cnt;   // inclusive prefix sum over the wave
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
      for (int i = lane; i < kListPad; i += 64) lst[total + i] = nsl;
      if (lane == 0) lst[kMaxSparseSlices + kListPad] = total;
    }
    __syncthreads();
    nh_wg = __builtin_amdgcn_readfirstlane(lst[kMaxSparseSlices + kListPad]);
    int lim_sl = 0x7fffffff;   // this wave's last slice
    if (causal) lim_sl = row_hi + coff < 0 ? -1 : (row_hi + coff) / kSlice;
    int cnt = 0;
    for (int base = 0; base < nh_wg; base += 64) {
      const int idx = base + lane;
      const bool in = idx < nh_wg && lst[idx] <= lim_sl;
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(in));
    }
    nh = wave_live ? __builtin_amdgcn_readfirstlane(cnt) : 0;
    lst_v = lst[lane];
  }
  // slice index of ring position h = h0 + j (Sparse: from the list; j < 64)
  auto slice_of = [&](int h, int j) __attribute__((always_inline)) {
    if constexpr (Sparse) return __builtin_amdgcn_readlane(lst_v, j);
    else return h;
  };


  f32x16 o_acc[kRB][D / 32];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o_acc[rb][db] = (f32x16){};
  float m_run[kRB], l_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -INFINITY;   // the exponent's subtrahend for the lane's row in block rb
    l_run[rb] = 0.f;         // partial running sum over this lane's half of the keys
  }

  // Key j is allowed for row i iff j <= klim (klim folds the valid length, the
  // causal limit and the masked leading rows into one bound).
  int klim[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int row = row_lo + 32 * rb + (lane & 31);
    klim[rb] = row < qs ? -1 : min(kv - 1, causal ? row + coff : 0x7fffffff);
  }
  // Masking is needed only where slice h crosses that bound for some row of
  // the wave: from the slice holding key kv-1 on (the first h with
  // kSlice*h + kSlice-1 >= kv), from the slice past the wave's first row's
  // diagonal on under a causal mask, and everywhere when masked leading rows
  // are in the wave.
  int mask_from = kv / kSlice;
  if (causal) mask_from = min(mask_from, max(row_lo + 1 + coff, 0) / kSlice);
  if (row_lo < qs) mask_from = 0;
  mask_from = __builtin_amdgcn_readfirstlane(mask_from);
  auto need_mask = [&](int h) __attribute__((always_inline)) { return h >= mask_from; };
  // slices mask_from .. nh-1 (this wave's) need the mask: h+1 is one of them
  // iff (unsigned)(h+1 - mask_from) < mask_span
  const int mask_span = max(nh, mask_from) - mask_from;
  auto mask = [&](int h, f32x16 (&s)[kRB]) __attribute__((always_inline)) {
    if constexpr (Dense) {
      // the row's word for slice h, ANDed with the rules' prefix of allowed
      // keys, shifted so that bit e is the lane's key offset e (+ 4*hf)
      const uint32_t* wb = (const uint32_t*)(smem + T::kLds) + ((h >> 3) & 1) * (kWaves * 256) + wave * 256;
      uint32_t w = wb[(lane & 31) * 8 + (h & 7)];
      const int lim = klim[0] - h * kSlice;   // rule-allowed key offsets within the slice: 0 .. lim
      const uint32_t pre = lim >= 31 ? 0xffffffffu : (lim < 0 ? 0u : ((2u << lim) - 1u));
      w = (w & pre) >> (4 * hf);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t t = (uint32_t)__builtin_amdgcn_sbfe((int)w, 8 * (r >> 2) + (r & 3), 1);   // 0 or ~0
        s[0][r] = __uint_as_float((t & __float_as_uint(s[0][r])) | (~t & 0xff800000u));
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int lim = klim[rb] - h * kSlice - 4 * hf;   // key offset within the slice must be <= lim
#pragma unroll
        for (int r = 0; r < 16; ++r) s[rb][r] = (8 * (r >> 2) + (r & 3)) <= lim ? s[rb][r] : -INFINITY;
      }
    }
  };
  // Dense: copy this wave's rows' mask words of slices 8*blk .. 8*blk+7 into
  // LDS buffer blk % 2 (lane L brings 16 bytes of row L/2).
  [[maybe_unused]] int m_off = 0;
  [[maybe_unused]] i32x4 m_rsrc = {0, 0, 0, 0};
  if constexpr (Dense) {
    m_off = (row_lo + (lane >> 1)) * mrw * 4 + (lane & 1) * 16;
    const uint32_t* mb = mbits + (size_t)b * msb + (size_t)(bh - b * H) * msh;
    const uint64_t a = sgpr64((const char*)mb);
    m_rsrc[0] = (int)(uint32_t)a;
    m_rsrc[1] = (int)(uint32_t)(a >> 32);
    m_rsrc[2] = __builtin_amdgcn_readfirstlane(N_q * mrw * 4);
    m_rsrc[3] = 0x00020000;
    asm volatile("" : "+s"(m_rsrc));
  }
  auto copy_mask = [&](int blk) __attribute__((always_inline)) {
    if constexpr (Dense) {
      const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(smem + T::kLds) +
                           (uint32_t)(((blk & 1) * kWaves + wave) * 1024);
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)blk * 32u);
      uint32_t voff;
      asm volatile("s_mov_b32 m0, %1\n\tv_add_u32 %0, %2, %3\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
                   : "=&v"(voff) : "s"(lds), "s"(soff), "v"(m_off), "s"(m_rsrc) : "memory", "m0");
    }
  };

  // Operand registers: K of the slice the next QK reads, V of the slice the
  // next PV reads. Each is read from LDS one phase before it is used.
  u32x4 ka[D / 16];
  bf16x8 va[2][D / 32];
  auto load_k = [&](auto sm) __attribute__((always_inline)) {
    const char* kb = kst(decltype(sm)::value);
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) ka[kc] = *(const lds_u32x4*)(kb + k_off[kc]);
  };
  // S^T = K Q^T for both row blocks, not interleaved (prologue only).
  auto qk = [&](f32x16 (&s)[kRB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        if (kc == 0) mfma_v_init<true>(s[rb], as_bf16x8(ka[kc]), qreg[rb][kc]);
        else mfma_v<true>(s[rb], as_bf16x8(ka[kc]), qreg[rb][kc]);
      }
    mfma_result_wait();
  };
  float negm[kRB];   // minus the exponent's subtrahend: -m_run, or 0 while m_run = -inf
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) negm[rb] = 0.f;
  // First slice of a tile: m = the slice's row max of S*c (-inf for a row with
  // no allowed key in it), then S <- S*c - m.
  auto first_max = [&](f32x16 (&s)[kRB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      f32x16& x = s[rb];
      float mx = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
      const float tmax = lane_swap_max(mx) * c;   // c > 0, so -inf stays -inf
      m_run[rb] = tmax;
      negm[rb] = (tmax == -INFINITY) ? 0.f : -tmax;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = fmaf(x[r], c, negm[rb]);
    }
  };
  // P = exp2(S*c - m), fp32 into the row sum, bf16 pairs into the PV operand
  // words. A slice's P is made in two halves: elements 0..7 (keys 0..15 of
  // the slice, the B operand of the first four PV MFMAs) in the phase before
  // the one that exponentiates elements 8..15, so that the exponentials are
  // spread over both phases. The first half is kept per slice parity,
  // because it is made while the previous slice's first half is still being
  // consumed.
  static_assert(kRB == 1, "the P halves below are laid out for one row block per wave");
  constexpr int kG = kRB * D / 16;      // MFMAs per phase
  uint32_t pbw_lo[2][4], pbw_hi[4];
  float lsum_lo[2], lsum_hi;
  float lsum[kRB];
  // exponential of element j of x; every second one completes a pair: packed
  // into words[(j % 8) / 2], its sum added to acc (started by the pair with j % 8 = 1)
  float p_even = 0.f;
  auto exp_one = [&](const f32x16& x, int j, uint32_t* words, float& acc) __attribute__((always_inline)) {
    const float p = __builtin_amdgcn_exp2f(x[j]);
    if ((j & 1) == 0) {
      p_even = p;
    } else {
      if ((j & 7) == 1) acc = p_even + p;
      else acc += p_even + p;
      words[(j & 7) >> 1] = pack2(p_even, p);
      asm volatile("" :: "v"(words[(j & 7) >> 1]), "v"(acc));
    }
  };
  // Per-group schedule (kG groups per phase) of the VALU work of the two
  // phases: phase A exponentiates elements 8..15 of slice h, phase B forms
  // S*c - m of slice h+1 (all 16 elements) and exponentiates its elements
  // 0..7, each after its own shift.
  struct Range { int lo, hi; };
  auto sched_a = [](int g) constexpr -> Range {   // elements of the second half
    return kG == 8 ? Range{8 + g, 9 + g} : Range{8 + 2 * g, 10 + 2 * g};
  };
  auto sched_b_shift = [](int g) constexpr -> Range {
    if (kG == 8) {
      constexpr Range r[8] = {{0, 4}, {4, 8}, {8, 10}, {10, 12}, {12, 14}, {14, 16}, {16, 16}, {16, 16}};
      return r[g];
    }
    constexpr Range r[4] = {{0, 8}, {8, 16}, {16, 16}, {16, 16}};
    return r[g];
  };
  auto sched_b_exp = [](int g) constexpr -> Range {
    if (kG == 8) {
      constexpr Range r[8] = {{0, 0}, {0, 1}, {1, 2}, {2, 3}, {3, 4}, {4, 5}, {5, 7}, {7, 8}};
      return r[g];
    }
    constexpr Range r[4] = {{0, 0}, {0, 2}, {2, 6}, {6, 8}};
    return r[g];
  };
  // S <- S*c - m for elements e0 .. e0+n-1 of block rb.
  auto shift_part = [&](f32x16 (&s)[kRB], int rb, int e0, int n) __attribute__((always_inline)) {
#pragma unroll
    for (int e = e0; e < e0 + n; ++e) s[rb][e] = fmaf(s[rb][e], c, negm[rb]);
#pragma unroll
    for (int e = e0; e < e0 + n; e += 2) asm volatile("" :: "v"(s[rb][e]), "v"(s[rb][e + 1]));
  };
  // Some lane's exponentials of the slice in s (already shifted by the current
  // m) add up to more than kSumCap: raise m to the slice's row max where that
  // max is above m, rescale l and O by exp2(m_old - m_new), and redo the
  // slice's exponentials. Rows whose max is not above m keep everything
  // (their shift d is 0). A row that has met no allowed key before this
  // slice still has m = -inf and the subtrahend 0; its new m is 0 + d.
  auto raise_max = [&](f32x16 (&s)[kRB], int par) __attribute__((always_inline)) {
    mfma_result_wait();   // o_acc is rescaled below
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      f32x16& x = s[rb];
      float mx = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
      mx = lane_swap_max(mx);                  // row max of S*c - m over the slice
      const float d = mx > 0.f ? mx : 0.f;     // 0 for -inf and NaN too
      const float a = __builtin_amdgcn_exp2f(-d);
      // the subtrahend in use is 0 while m is still -inf (a row that has met
      // no allowed key yet); from now on it is that plus d
      m_run[rb] = (m_run[rb] == -INFINITY ? 0.f : m_run[rb]) + d;
      negm[rb] = -m_run[rb];
      l_run[rb] *= a;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o_acc[rb][db] *= a;
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(x[e] - d);
        const float p1 = __builtin_amdgcn_exp2f(x[e + 1] - d);
        sum += p0 + p1;
        if (e < 8) pbw_lo[par][e >> 1] = pack2(p0, p1);
        else pbw_hi[(e - 8) >> 1] = pack2(p0, p1);
      }
      lsum[rb] = sum;
    }
  };
  auto pb = [&](int par, int cc) __attribute__((always_inline)) {
    const u32x4 w = cc == 0 ? (u32x4){pbw_lo[par][0], pbw_lo[par][1], pbw_lo[par][2], pbw_lo[par][3]}
                            : (u32x4){pbw_hi[0], pbw_hi[1], pbw_hi[2], pbw_hi[3]};
    return as_bf16x8(w);
  };
  // one transposing V read pair: va[cc][db] for PV
  auto load_v_one = [&](const char* vb, int cc, int db) __attribute__((always_inline)) {
    const char* p0 = vb + 16 * cc * T::kRowBytes;   // vb: vst_rel of the stage
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + v_off[0][db]));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + v_off[1][db]));
    va[cc][db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // Step h (slice h; S of slice h is in sc, already shifted):
  //   wait for slices <= h+2, barrier (slice h-1's stage is now free);
  //   phase A: QK(h+1) on the MFMA unit (K(h+1) was read last phase) while the
  //            VALU exponentiates elements 8..15 of slice h and the LDS reads
  //            V(h);
  //   check the exponential sums of slice h against kSumCap (rarely: raise m);
  //   copy this wave's share of K(h+7) into slice h-1's stage;
  //   mask slice h+1 if it crosses a bound;
  //   phase B: PV(h) on the MFMA unit while the VALU forms S*c - m of slice
  //            h+1 and exponentiates its elements 0..7, and the LDS reads
  //            K(h+2);
  //   copy this wave's share of V(h+7).
  // Each phase is written as kG groups of one MFMA, a share of the LDS reads
  // and a share of the VALU work, fenced so the scheduler keeps that order:
  // every MFMA overlaps the VALU work that follows it.
  // Slice h+1 may lie past this wave's last slice: its S is then computed from
  // whatever the stage holds and discarded, so no branch splits a phase.
  // Slice h-1's stage is free at step h: V(h-1) was read in step h-1 and
  // K(h-1) in step h-3. Copies are issued for every step, also past the
  // tile's last slice (where they fetch nothing), so the number in flight,
  // and with it the wait count, is the same each time: slices h+3 .. h+6 may
  // still be in flight.
  auto step = [&](auto hm, int h, f32x16 (&sc)[kRB], f32x16 (&sn)[kRB]) __attribute__((always_inline)) {
    constexpr int Hm = decltype(hm)::value;   // h % kStages
    wait_copies<4 * kC>();
    __syncthreads();   // slices <= h+2 have landed; slice h-1's stage is no longer read
    if (h >= nh) {   // this wave's rows are done; it still copies its share
      copy_slices(std::integral_constant<int, Hm + kStages - 1>{}, slice_of(h + kStages - 1, Hm + kStages - 1));
      return;
    }
    // ---- phase A ----
    {
      const char* vb = vst_rel(Hm);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const int kc = g / kRB, rb = g % kRB;
        // (for d = 64 the compiler moves the first K operand into AGPRs right
        // before this MFMA, so it gets the wait states)
        if (kc == 0) mfma_v_init<D == 64>(sn[rb], as_bf16x8(ka[kc]), qreg[rb][kc]);
        else mfma_v<false>(sn[rb], as_bf16x8(ka[kc]), qreg[rb][kc]);
        if (g % kRB == 0) {   // V reads for PV group g/kRB, (cc, db) in PV order
          const int pg = g / kRB;
          load_v_one(vb, pg / (D / 32), pg % (D / 32));
        }
        const Range ra = sched_a(g);   // second half of slice h's exponentials
#pragma unroll
        for (int j = ra.lo; j < ra.hi; ++j) exp_one(sc[0], j, pbw_hi, lsum_hi);
        // order inside the group (measured best of the orders tried): after
        // the MFMA the exponential, then the V reads, then the rest
        __builtin_amdgcn_sched_group_barrier(0x400, 4, 1);    // transcendental
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);    // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 24, 1);   // other VALU
        __builtin_amdgcn_sched_barrier(0);
      }
      // keep P and the sums in this phase (the compiler would otherwise sink
      // them past the mask branch, away from the MFMAs they overlap)
      asm volatile("" :: "v"(pbw_hi[0]), "v"(pbw_hi[1]), "v"(pbw_hi[2]), "v"(pbw_hi[3]), "v"(lsum_hi));
      lsum[0] = lsum_lo[Hm & 1] + lsum_hi;
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) over = over || !(lsum[rb] <= kSumCap);   // NaN counts as over
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) raise_max(sc, Hm & 1);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) l_run[rb] += lsum[rb];
    }
    // This wave's share of the K copy of slice h+7, into the stage the barrier
    // freed. The copies go out between the phases and at the end of the step,
    // where the waves arrive at different times, so the workgroup's copies
    // reach the address unit spread out rather than all at once.
    copy_slice(k_rsrc, slice_of(h + kStages - 1, Hm + kStages - 1), kso(std::integral_constant<int, Hm + kStages - 1>{}));
    // Dense: the next 8-slice block's mask words (used from step h+7 on; the
    // copies issued in between make the waits of those steps cover it).
    if constexpr (Dense && Hm == 0) copy_mask((h >> 3) + 1);
    // S of slice h+1 is read below. The mask reads it at once and needs the
    // wait states; for d = 128 the phase-B shifts come late enough without
    // them (the build's hazard check verifies that distance), for d = 64 not.
    bool msk;
    if constexpr (Sparse) msk = h + 1 < nh && slice_of(h + 1, Hm + 1) >= mask_from;
    else msk = Dense || (unsigned)(h + 1 - mask_from) < (unsigned)mask_span;
    if (D == 64 || msk) mfma_result_wait();
    if (msk) mask(slice_of(h + 1, Hm + 1), sn);
    // ---- phase B ----
    {
      const char* kb = kst((Hm + 2) % kStages);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const int pg = g / kRB, rb = g % kRB;
        const int cc = pg / (D / 32), db = pg % (D / 32);
        // V pairs were read in phase A in PV order, two reads per pair. Wait
        // for the first half before group 0 and for the second half before
        // group kG/2 (by then the K reads issued in between may still be in
        // flight; LDS reads complete in order), two waits instead of one per
        // group.
        static_assert(kRB == 1, "one V pair per group, in group order");
        if (g == 0) lgkm_wait<kG>();
        if (g == kG / 2) lgkm_wait<kG / 2>();
        mfma_a(o_acc[rb][db], va[cc][db], pb(Hm & 1, cc));
        if (g < D / 16) ka[g] = *(const lds_u32x4*)(kb + k_off[g]);
        // the shift S*c - m of slice h+1 and the first half of its exponentials
        const Range rs = sched_b_shift(g), rx = sched_b_exp(g);
        if (rs.hi > rs.lo) shift_part(sn, 0, rs.lo, rs.hi - rs.lo);
#pragma unroll
        for (int j = rx.lo; j < rx.hi; ++j) exp_one(sn[0], j, pbw_lo[(Hm + 1) & 1], lsum_lo[(Hm + 1) & 1]);
        // order inside the group: after the MFMA the K read, then the
        // exponentials, then the shifts, sums and packs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);    // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x400, 4, 1);    // transcendental
        __builtin_amdgcn_sched_group_barrier(0x002, 24, 1);   // other VALU
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    copy_slice(v_rsrc, slice_of(h + kStages - 1, Hm + kStages - 1), vso(std::integral_constant<int, Hm + kStages - 1>{}));   // the V share
  };

  f32x16 sa[kRB], sb[kRB];
  if (nh_wg > 0) {
    if (item > 0) __syncthreads();   // every wave is done reading the previous tile's stages
    // The item's Q rows are read here first, so the compiler's wait for their
    // loads comes before this tile's copies are issued and does not cover them
    // (vector memory operations complete in order).
    q_read();
    prep_q(row_lo);
    copy_mask(0);   // Dense: the first block's mask words, ahead of the copies the wait below covers
    if (!ahead) {
      static_for<kStages - 1>([&](auto s) { copy_slices(s, slice_of(decltype(s)::value, decltype(s)::value)); });
    }
    // A tile that was not continued waits for all of its first copies here
    // (slices 0..6 and the mask words); a wait for only the oldest of them let
    // rows of the first tiles of a cold launch see stale K/V or mask words
    // (measured, boolean-mask d = 64), and every build before that waited for
    // all of them anyway. After a continuation the copies of slices 0..6 are
    // older than the Q loads and the previous tile's O stores, so the partial
    // wait covers all of them.
    if (ahead) wait_copies<4 * kC>();
    else wait_copies<0>();
    __syncthreads();   // slices 0 .. 6 have landed
    if (nh > 0) {
      load_k(std::integral_constant<int, 0>{});
      qk(sa);
      if (Dense || need_mask(slice_of(0, 0))) mask(slice_of(0, 0), sa);
      first_max(sa);
#pragma unroll
      for (int j = 0; j < 8; ++j) exp_one(sa[0], j, pbw_lo[0], lsum_lo[0]);
      load_k(std::integral_constant<int, 1>{});
    }
    static_assert(kStages == 8, "the loop below is unrolled over kStages slices");
    for (int h0 = 0; h0 < nh_wg; h0 += 8) {
      if constexpr (Sparse) lst_v = lst[h0 + lane];   // list entries h0 .. h0+63
      step(std::integral_constant<int, 0>{}, h0, sa, sb);
      if (h0 + 1 >= nh_wg) break;
      // From here on the copies (ring positions h0 + 8 ..) are the next
      // item's: ring position nsl + s is stage s, where its slice s goes. They
      // use descriptors whose byte 0 lies nsl slices before the next item's K
      // (V), so position nsl + s addresses its slice s, and num_records bounds
      // it by the keys that item can see.
      if constexpr (kCont) {
        if (cont && h0 + kStages == nsl) {
          const uint32_t skip = (uint32_t)nsl * (uint32_t)T::kBytes;
          const uint32_t lim = skip + (uint32_t)n_end * T::kRowBytes;
          k_rsrc = rsrc_of((const char*)(K + (size_t)nbh * N_k * D), skip, lim);
          v_rsrc = rsrc_of((const char*)(V + (size_t)nbh * N_k * D), skip, lim);
          asm volatile("" : "+s"(k_rsrc), "+s"(v_rsrc));
        }
      }
      step(std::integral_constant<int, 1>{}, h0 + 1, sb, sa);
      if (h0 + 2 >= nh_wg) break;
      step(std::integral_constant<int, 2>{}, h0 + 2, sa, sb);
      if (h0 + 3 >= nh_wg) break;
      step(std::integral_constant<int, 3>{}, h0 + 3, sb, sa);
      if (h0 + 4 >= nh_wg) break;
      step(std::integral_constant<int, 4>{}, h0 + 4, sa, sb);
      if (h0 + 5 >= nh_wg) break;
      step(std::integral_constant<int, 5>{}, h0 + 5, sb, sa);
      if (h0 + 6 >= nh_wg) break;
      step(std::integral_constant<int, 6>{}, h0 + 6, sa, sb);
      if (h0 + 7 >= nh_wg) break;
      step(std::integral_constant<int, 7>{}, h0 + 7, sb, sa);
    }
  } else {
    // The rows loaded for this item go unused: read them here, so that on
    // every path the loads are complete before the next item's rows are
    // loaded into the same registers (that load then waits for nothing).
    q_read();
  }
  // No copy may still be writing LDS when the epilogue stages O or the next
  // tile starts (also when this tile computed nothing: a continued tile can
  // have issued its slices 0..6 all the same). A continuing tile's copies
  // write stages 0..6, which its epilogue leaves alone.
  if (!cont) wait_copies<0>();
  mfma_result_wait();   // the last P V MFMAs have written o_acc
  if (has_next) load_q(nbh, qt_n * kBM + kRows * wave);   // the next item's Q rows (qreg is no longer read)

  // ---- epilogue: O / l, LSE, bf16 store ----
  // In the accumulator layout a lane holds 8-byte pieces of 32 different rows,
  // so storing straight from it would touch 32 partial cache lines per store
  // instruction. The wave instead writes its normalised rows into LDS (row
  // stride 2*D + 16 bytes, which starts the rows of one write on different
  // banks), reads them back as 16-byte pieces of whole rows, and stores
  // kLanesPerORow lanes per row: each instruction writes complete rows.
  constexpr int kORow = 2 * D + 16;
  constexpr int kChunksPerRow = D / 8;                   // 16-byte pieces per row
  static_assert(kWaves * kRows * kORow <= T::kLds, "the O staging area must fit in the stages");
  static_assert(!kCont || (kWaves / 2) * kRows * kORow <= T::kBytes + kContLds, "half the waves' rows fit the spare room");
  __syncthreads();   // every wave is done with the K/V stages, which the staging area overlaps
  // A continued tile stages its rows in V stage 7 and the LDS past the ring
  // (stages 0..6 hold the next tile's first slices), half the waves at a time.
  char* const cont_area = smem + (2 * kStages - 1) * T::kBytes;
  char* ost = cont ? cont_area + (wave % (kWaves / 2)) * kRows * kORow : smem + wave * kRows * kORow;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
  if (half == 1 && !cont) break;
  if (half == 1) __syncthreads();   // the first half's rows have been read back
  if (cont && wave / (kWaves / 2) != half) continue;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int r = 32 * rb + (lane & 31);
    const int row = row_lo + r;
    const float l_tot = lane_swap_add(l_run[rb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack2(o_acc[rb][db][4 * g + 0] * inv, o_acc[rb][db][4 * g + 1] * inv),
                         pack2(o_acc[rb][db][4 * g + 2] * inv, o_acc[rb][db][4 * g + 3] * inv)};
        *(__attribute__((address_space(3))) u32x2*)(ost + r * kORow + 2 * (32 * db + 8 * g + 4 * hf)) = w;
      }
    }
    if (LSE && lane < 32 && row < N_q)
      LSE[(size_t)bh * N_q + row] =
          l_tot > 0.f ? ((m_run[rb] == -INFINITY ? 0.f : m_run[rb]) + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < kRows * kChunksPerRow / 64; ++i) {
    const int ci = 64 * i + lane;
    const int r = ci / kChunksPerRow, ch = ci % kChunksPerRow;
    const u32x4 x = *(const __attribute__((address_space(3))) u32x4*)(ost + r * kORow + 16 * ch);
    if (row_lo + r < N_q) *(u32x4*)(O + q_base + (size_t)(row_lo + r) * D + 8 * ch) = x;
  }
  }   // halves
  ahead = cont;
  if (!has_next) break;
  slot = slot_n;
  it = it_n;
  }   // items
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Bit-packed mask: pack rows of a byte mask (nonzero = may attend) into 32-bit
// words, bit j % 32 of word j / 32, rows of `row_words` words (the tail of a
// row past n_k is written as zeros). One thread per output word.
__global__ __launch_bounds__(256) void attn_mask_pack_kernel(const uint8_t* __restrict__ m, uint32_t* __restrict__ bits,
                                                            long long rows, int n_k, int row_words) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * row_words) return;
  const long long r = id / row_words;
  const int w = (int)(id - r * row_words);
  uint32_t x = 0;
  for (int t = 0; t < 32; ++t) {
    const int j = 32 * w + t;
    if (j < n_k && m[r * n_k + j] != 0) x |= 1u << t;
  }
  bits[id] = x;
}

// compute units of the current device, read once per device (0 if unknown)
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n > 0 ? n : 0;
}

int fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q, int N_k,
               int d, float scale, int causal, const int32_t* seqlens_k, const int32_t* q_start,
               const uint32_t* mbits, long long msb, long long msh, int mrw, const uint8_t* bmask, long long bsb,
               long long bsh, int n_ks, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (causal < 0 || causal > 2) return ATTN_ERR_MASK;
  if ((long long)B * H * N_q == 0) return ATTN_OK;
  if (!q || !o) return ATTN_ERR_NULL;
  if (N_k > 0 && (!k || !v)) return ATTN_ERR_NULL;
  const int mode = mbits ? 1 : bmask ? 2 : 0;
  const int waves = waves_of(mode, d), bm = kRows * waves;      // workgroup shape of the instance
  const long long n_qt = (N_q + bm - 1) / bm;
  // one slot per pair of query tiles, or per tile when all tiles are equal (as in the kernel)
  const bool single = !causal && !seqlens_k && !q_start;
  const long long n_wg = (long long)B * H * (single ? n_qt : (n_qt + 1) / 2);
  if (n_wg > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((long long)B * H > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((long long)N_k * d * 2 > 0x7fffffffLL) return ATTN_ERR_SHAPE;   // K/V copy offsets are 32-bit
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
  // causal mode 1: key j visible to row i iff j <= i; mode 2: iff j <= i + N_k - N_q
  int causal01 = causal ? 1 : 0, coff = causal == 2 ? N_k - N_q : 0, n_qt_i = (int)n_qt, n_wg_i = (int)n_wg;
  auto kern = d == 128 ? (mode == 1 ? attn_fwd_kernel<128, 1> : mode == 2 ? attn_fwd_kernel<128, 2> : attn_fwd_kernel<128, 0>)
                       : (mode == 1 ? attn_fwd_kernel<64, 1> : mode == 2 ? attn_fwd_kernel<64, 2> : attn_fwd_kernel<64, 0>);
  // One workgroup per slot (pair of query tiles), or, for rules-only d = 128
  // launches with equal slots (no per-batch lengths) and more slots than CUs,
  // one workgroup per CU that walks its share of them: each tile's last steps
  // then fetch the next one's first K/V slices and Q while it still computes.
  // (A multiple of 8 CUs keeps every workgroup's slots on its own XCD.)
  unsigned grid = (unsigned)n_wg;
  if (mode == 0 && d == 128 && !seqlens_k && !q_start) {
    const int n_cu = cu_count();
    if (n_cu > 0 && n_cu % 8 == 0 && n_wg > n_cu) grid = (unsigned)n_cu;
  }
  const hipError_t e = attn_launch::launch(kern, dim3(grid), dim3(64 * waves), stream, qp, kp, vp, op, lse, H, N_q,
                                           N_k, c, neg, causal01, coff, seqlens_k, q_start, n_qt_i, n_wg_i, mbits, msb,
                                           msh, mrw, bmask, bsb, bsh, n_ks);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                        int N_q, int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                        const int32_t* q_start, hipStream_t stream) {
  return fwd_launch(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start, nullptr, 0, 0, 0, nullptr,
                    0, 0, 0, stream);
}

extern "C" int attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                               int N_q, int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                               const int32_t* q_start, const uint32_t* mask_bits, long long mask_stride_b,
                               long long mask_stride_h, int mask_row_words, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if (!mask_bits) {
    if ((long long)B * H * N_q == 0) return fwd_launch(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, seqlens_k,
                                                       q_start, nullptr, 0, 0, 0, nullptr, 0, 0, 0, stream);
    return ATTN_ERR_NULL;
  }
  if ((uintptr_t)mask_bits & 15) return ATTN_ERR_ALIGN;
  if (mask_row_words < (N_k + 31) / 32 || mask_row_words % 8 != 0 || mask_stride_b < 0 || mask_stride_h < 0)
    return ATTN_ERR_MASK;
  if ((long long)N_q * mask_row_words * 4 > 0x7fffffffLL) return ATTN_ERR_SHAPE;   // 32-bit copy offsets
  return fwd_launch(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start, mask_bits,
                    mask_stride_b, mask_stride_h, mask_row_words, nullptr, 0, 0, 0, stream);
}

extern "C" int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                     int N_q, int N_k, int d, float scale, int causal, const int32_t* seqlens_k,
                                     const int32_t* q_start, const uint8_t* block_mask, long long block_stride_b,
                                     long long block_stride_h, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  const int n_ks = (N_k + 4 * kSlice - 1) / (4 * kSlice);   // 128-key blocks per row of the block mask
  if ((long long)B * H * N_q == 0)
    return fwd_launch(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start, nullptr, 0, 0, 0, nullptr,
                      0, 0, 0, stream);
  if (!block_mask) return ATTN_ERR_NULL;
  if ((N_k + kSlice - 1) / kSlice > kMaxSparseSlices) return ATTN_ERR_SHAPE;
  if (block_stride_b < 0 || block_stride_h < 0) return ATTN_ERR_MASK;
  return fwd_launch(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, seqlens_k, q_start, nullptr, 0, 0, 0,
                    block_mask, block_stride_b, block_stride_h, n_ks, stream);
}

extern "C" int attn_mask_pack(const uint8_t* mask, uint32_t* bits, long long rows, int N_k, int row_words,
                              hipStream_t stream) {
  if (rows < 0 || N_k < 0 || row_words < (N_k + 31) / 32) return ATTN_ERR_SHAPE;
  if (rows == 0 || row_words == 0) return ATTN_OK;
  if (!bits || (N_k > 0 && !mask)) return ATTN_ERR_NULL;
  if (((uintptr_t)bits & 3)) return ATTN_ERR_ALIGN;
  const long long n = rows * row_words;
  if ((n + 255) / 256 > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const hipError_t e = attn_launch::launch(attn_mask_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), stream,
                                           mask, bits, rows, N_k, row_words);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid or too large shape";
    case ATTN_ERR_HEAD_DIM: return "head dim must be 64 or 128";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_ALIGN: return "misaligned pointer (bf16 tensors need 16 bytes, lse and delta 4)";
    case ATTN_ERR_ALIAS: return "output overlaps an input or the other output";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_MASK: return "causal must be 0, 1 or 2; mask rows need >= ceil(N_k/32) words, a multiple of 8";
    case ATTN_ERR_SCRATCH: return "B*H*N_q exceeds the 1048576 rows of the allocation-free backward's own workspace";
    default: return "unknown status";
  }
}

extern "C" int attn_version(void) { return 10100; }
