// FP8 (OCP E4M3) fused attention forward for gfx950.
//
// The mixed-precision direction of the codechina.net "GPU memory wall ...
// FlashAttention" article (section 9, future directions): both matrix
// products of the tiled attention in FP8 with a wider accumulator, here the
// fp32 accumulator of the gfx950 FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4
// with unit block scales). The softmax is the online softmax of the bf16
// kernel (running max and sum per row, output rescaled when the max grows);
// the probabilities are rounded to E4M3 (times 2^8, so that small ones stay
// normal numbers) before the second product.
//
// Layout of one wave's work. The wave owns 32 query rows; lane L handles row
// L % 32 and half h = L / 32 of every operand. Scores are computed transposed,
// S^T = K Q^T (A = 32 keys, B = 32 queries, k = head dim), so that each lane's
// accumulator registers all belong to its own query row: the per-row max, sum
// and rescale need no cross-lane traffic except between the two halves. The
// output is O^T = V^T P^T: the score accumulator, rounded to FP8, is directly
// the B operand (k = 64 keys), and V^T rows (head-dim index d, keys fastest)
// are the A operand. An MFMA reads lane half h's byte i of A and of B as the
// same k index, whatever that index is; so any assignment of keys to
// (half, byte) works if both operands use it. A row of the S^T tile is chosen
// to be key sigma(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3) of the 32-key slice:
// then accumulator register r of half h holds key 16h + r, and lane half h
// needs V^T bytes of keys [16h, 16h+16) and [32+16h, 32+16h+16) of each 64 keys of a
// step: two 16-byte LDS reads.
#include <hip/hip_runtime.h>
#include <float.h>

#include <cmath>
#include <stdint.h>

#include "attn.h"
#include "launch.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kWaves = 8;            // waves per workgroup, 32 query rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWG = 32 * kWaves;
constexpr int kStep = 128;           // keys per step: 4 slices of 32 for S^T, 2 MFMAs of 64 for P V
constexpr int kSlices = kStep / 32, kVRowChunks = kStep / 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPLog2 = 8.f;        // P is rounded to E4M3 as P * 2^8

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // operand formats 0 = E4M3 for A and B; block scales 127 = 2^0 (E8M0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(const u32x4& lo, const u32x4& hi) {
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// 16-byte chunk c of K tile row r, XOR-swizzled so that the 16 lanes of one
// LDS pass (the rows sigma(m) of a slice) hit distinct bank groups
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) {
  if constexpr (D == 128) return c ^ (((r >> 1) & 3) | (((r >> 4) & 1) << 2));
  else return c ^ (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}
// 16-byte chunk c of V^T tile row d (kStep bytes), XOR-swizzled likewise
__device__ __forceinline__ int v_chunk(int d, int c) {
  if constexpr (kVRowChunks == 8) return c ^ ((d >> 1) & 7);
  else return c ^ ((d >> 2) & 3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  auto rn = [](float x) {
    uint32_t u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;   // round to nearest even (values are finite)
  };
  return rn(a) | (rn(b) << 16);
}

template <int D>
// one workgroup of eight waves per CU, two per SIMD: one wave's softmax runs while the
// other's MFMAs do, and each K / V^T tile staged in LDS serves 256 query rows
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ Vt,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int N_q, int N_k, long long ldv, float c,
    float o_scale, uint32_t q_sign, int causal, int coff, int n_qt) {
  constexpr int kKBytes = kStep * D, kStage = 2 * kKBytes;   // [K tile kStep x D][V^T tile D x kStep]
  constexpr int kKChunks = kKBytes / 16 / kThreads;          // 16-byte K chunks per thread per step
  constexpr int kVChunks = kKChunks;                         // same count for V^T
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, m = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_bh = (int)(gridDim.x / n_qt);
  // causal: tile-major, the tiles with the most keys first
  const int bh = causal ? (int)(blockIdx.x % n_bh) : (int)(blockIdx.x / n_qt);
  const int qt = causal ? n_qt - 1 - (int)(blockIdx.x / n_bh) : (int)(blockIdx.x % n_qt);
  const size_t q_base = (size_t)bh * N_q * D, k_base = (size_t)bh * N_k * D, v_base = (size_t)bh * D * ldv;
  const int q0 = qt * kRowsWG, q0w = q0 + 32 * wave, qrow = q0w + m;

  // keys any row of the workgroup may see
  int k_end = N_k;
  if (causal) k_end = max(0, min(N_k, min(q0 + kRowsWG, N_q) - 1 + coff + 1));
  const int n_steps = (k_end + kStep - 1) / kStep;

  // this lane's Q bytes: B operand of S^T, bytes [64c + 32h, +32) of its row
  i32x8 qop[D / 64];
#pragma unroll
  for (int cq = 0; cq < D / 64; ++cq) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = lo;
    if (qrow < N_q) {
      const uint8_t* p = Q + q_base + (size_t)qrow * D + 64 * cq + 32 * h;
      lo = *(const u32x4*)p;
      hi = *(const u32x4*)(p + 16);
      // a negative score factor is moved onto Q: flipping every sign bit negates
      // Q exactly, so c >= 0 and the max of the raw scores is the max of S * c
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] ^= q_sign;
        hi[w] ^= q_sign;
      }
    }
    qop[cq] = join(lo, hi);
  }

  // global -> register prefetch of one step's tiles, through buffer loads
  // bounded by the head's K (rows past N_k read as zeros) and V^T bytes (the
  // host keeps both below 2^31), so that no load sits behind a branch
  const __amdgpu_buffer_rsrc_t k_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + k_base), (short)0, N_k * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Vt + v_base), (short)0, (int)(D * ldv), 0x00020000);
  const int ldv_i = (int)ldv;
  u32x4 kbuf[kKChunks], vbuf[kVChunks];
  auto fetch = [&](int st) {
    const int k0 = st * kStep;
#pragma unroll
    for (int j = 0; j < kKChunks; ++j) {
      const int i = tid + kThreads * j, r = i / (D / 16), cc = i % (D / 16);
      kbuf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(k_rs, (k0 + r) * D + 16 * cc, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < kVChunks; ++j) {
      const int i = tid + kThreads * j, d = i / kVRowChunks, cc = i % kVRowChunks;
      const int kk = k0 + 16 * cc;
      // the row stride holds whole 16-byte chunks; bytes of keys >= N_k are cleared
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v_rs, d * ldv_i + kk, 0, 0));
      vbuf[j] = kk < N_k ? x : (u32x4){0u, 0u, 0u, 0u};
    }
    if (k0 + kStep > N_k) {   // the step holding key N_k: clear the keys past it in its chunk
#pragma unroll
      for (int j = 0; j < kVChunks; ++j) {
        const int i = tid + kThreads * j, cc = i % kVRowChunks;
        const int nv = N_k - (k0 + 16 * cc);
        if (nv > 0 && nv < 16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int keep = min(max(nv - 4 * w, 0), 4);
            vbuf[j][w] = keep == 4 ? vbuf[j][w] : (vbuf[j][w] & ((1u << (8 * keep)) - 1u));
          }
        }
      }
    }
  };
  auto store = [&](int stage) {
    uint8_t* sk = smem + stage * kStage;
    uint8_t* sv = sk + kKBytes;
#pragma unroll
    for (int j = 0; j < kKChunks; ++j) {
      const int i = tid + kThreads * j, r = i / (D / 16), cc = i % (D / 16);
      *(lds_u32x4*)(sk + r * D + 16 * k_chunk<D>(r, cc)) = kbuf[j];
    }
#pragma unroll
    for (int j = 0; j < kVChunks; ++j) {
      const int i = tid + kThreads * j, d = i / kVRowChunks, cc = i % kVRowChunks;
      *(lds_u32x4*)(sv + d * kStep + 16 * v_chunk(d, cc)) = vbuf[j];
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;   // running max (log2 units) and this half's sum of 2^8 p
  const int sig = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);   // key of S^T row m in its slice

  if (n_steps > 0) {
    fetch(0);
    store(0);
    __syncthreads();
  }
  for (int st = 0; st < n_steps; ++st) {
    const int stage = st & 1;
    if (st + 1 < n_steps) fetch(st + 1);
    const int k0 = st * kStep;
    // the wave has work unless every key of the step is past its last row's diagonal
    if (!causal || k0 <= min(q0w + 31, N_q - 1) + coff) {
      const uint8_t* sk = smem + stage * kStage;
      const uint8_t* sv = sk + kKBytes;
      f32x16 s[kSlices];
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        const int r = 32 * sl + sig;
        s[sl] = (f32x16){};
#pragma unroll
        for (int cq = 0; cq < D / 64; ++cq) {
          const u32x4 lo = *(const lds_u32x4*)(sk + r * D + 16 * k_chunk<D>(r, 4 * cq + 2 * h));
          const u32x4 hi = *(const lds_u32x4*)(sk + r * D + 16 * k_chunk<D>(r, 4 * cq + 2 * h + 1));
          s[sl] = mfma8(join(lo, hi), qop[cq], s[sl]);
        }
      }
      // register r of slice sl, half h: key k0 + 32*sl + 16*h + r of row qrow,
      // visible iff key <= lim (the last key, or the row's diagonal): one
      // compare against a per-slice threshold per score
      const bool full = k0 + kStep <= N_k && (!causal || k0 + kStep - 1 <= q0w + coff);
      if (!full) {
        const int lim = causal ? min(N_k - 1, qrow + coff) : N_k - 1;
#pragma unroll
        for (int sl = 0; sl < kSlices; ++sl) {
          const int thr = lim - (k0 + 32 * sl + 16 * h);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[sl][r] = r <= thr ? s[sl][r] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sl][r]);
      {   // with the other half of the row (lane ^ 32): permlane32_swap gives each lane both values
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_new = fmaxf(m_run, mx * c);
      // rescale only when some row's max grew
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
      }
      // p * 2^8 straight from the exponent; a row with no key yet: every p is 0
      const float msub = (m_run == -INFINITY ? 0.f : m_run) - kPLog2;
      int pw[4 * kSlices];
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(s[sl][4 * j + e] * c - msub);
            l_run += p[e];
          }
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          pw[4 * sl + j] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        }
      // keys [64kh, 64kh + 64) of the step: slices 2kh and 2kh + 1
#pragma unroll
      for (int kh = 0; kh < kSlices / 2; ++kh) {
        const i32x8 pop = {pw[8 * kh], pw[8 * kh + 1], pw[8 * kh + 2], pw[8 * kh + 3],
                           pw[8 * kh + 4], pw[8 * kh + 5], pw[8 * kh + 6], pw[8 * kh + 7]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = 32 * db + m;
          const u32x4 lo = *(const lds_u32x4*)(sv + d * kStep + 16 * v_chunk(d, 4 * kh + h));
          const u32x4 hi = *(const lds_u32x4*)(sv + d * kStep + 16 * v_chunk(d, 4 * kh + 2 + h));
          oacc[db] = mfma8(join(lo, hi), pop, oacc[db]);
        }
      }
    }
    if (st + 1 < n_steps) {
      // every wave is done with stage st - 1 (barrier at the end of the last
      // step), so the other stage may be overwritten
      store(stage ^ 1);
      __syncthreads();
    }
  }

  const float l = l_run + __shfl_xor(l_run, 32, 64);
  if (qrow < N_q) {
    const float inv = l > 0.f ? o_scale / l : 0.f;
    uint16_t* orow = O + q_base + (size_t)qrow * D;
    // register r of block db holds d = 32*db + 8*(r/4) + 4*h + r%4
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        const uint32_t a = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        const uint32_t b = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(uint2*)(orow + d) = make_uint2(a, b);
      }
    if (LSE && h == 0) LSE[(size_t)bh * N_q + qrow] = l > 0.f ? (m_run + __log2f(l) - kPLog2) / kLog2e : -INFINITY;
  }
}

bool spans_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int attn_fwd_fp8(const void* q, const void* k, const void* vt, long long vt_row_stride, void* o,
                            float* lse, int B, int H, int N_q, int N_k, int d, float scale, float q_descale,
                            float k_descale, float v_descale, int causal, hipStream_t stream) {
  if (B < 0 || H < 0 || N_q < 0 || N_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!std::isfinite(scale) || !std::isfinite(q_descale) || !std::isfinite(k_descale) || !std::isfinite(v_descale))
    return ATTN_ERR_SCALE;
  if (causal < 0 || causal > 2) return ATTN_ERR_MASK;
  const long long bh = (long long)B * H;
  if (bh == 0 || N_q == 0) return ATTN_OK;
  if (!q || !o) return ATTN_ERR_NULL;
  if (N_k > 0 && (!k || !vt)) return ATTN_ERR_NULL;
  if (vt_row_stride < (N_k + 15) / 16 * 16 || vt_row_stride % 16 != 0) return ATTN_ERR_SHAPE;
  if (bh > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  const long long n_qt = (N_q + kRowsWG - 1) / kRowsWG;
  if (bh * n_qt > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((long long)N_k * d > 0x7fffffffLL || (long long)d * vt_row_stride > 0x7fffffffLL) return ATTN_ERR_SHAPE;   // 32-bit load offsets
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)vt | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
  const size_t qn = (size_t)bh * N_q * d, kn = (size_t)bh * N_k * d, vn = (size_t)bh * d * vt_row_stride;
  const size_t on = qn * 2, ln = lse ? (size_t)bh * N_q * 4 : 0;
  const void* ins[] = {q, k, vt};
  const size_t in_n[] = {qn, kn, vn};
  for (int j = 0; j < 3; ++j)
    if (spans_overlap(o, on, ins[j], in_n[j]) || spans_overlap(lse, ln, ins[j], in_n[j])) return ATTN_ERR_ALIAS;
  if (spans_overlap(o, on, lse, ln)) return ATTN_ERR_ALIAS;

  // log2-domain factor of the raw scores; a negative factor negates Q instead,
  // and 0 becomes the smallest normal float: exp2 of a finite raw score times
  // it is exactly 1 in fp32, while a masked -inf stays -inf (0 * -inf would not)
  float c = scale * q_descale * k_descale * kLog2e;
  const uint32_t q_sign = c < 0.f ? 0x80808080u : 0u;
  c = fabsf(c);
  if (c < FLT_MIN) c = FLT_MIN;
  if (!std::isfinite(c)) return ATTN_ERR_SCALE;
  const float o_scale = v_descale;   // the sum l carries the same 2^8 as the rounded P
  const int coff = causal == 2 ? N_k - N_q : 0, causal01 = causal ? 1 : 0, nqt = (int)n_qt;
  const dim3 grid((unsigned)(bh * n_qt)), block(kThreads);
  const uint8_t *qp = (const uint8_t*)q, *kp = (const uint8_t*)k, *vp = (const uint8_t*)vt;
  uint16_t* op = (uint16_t*)o;
  const hipError_t e =
      d == 128 ? attn_launch::launch(attn_fwd_fp8_kernel<128>, grid, block, stream, qp, kp, vp, op, lse, H, N_q, N_k,
                                     vt_row_stride, c, o_scale, q_sign, causal01, coff, nqt)
               : attn_launch::launch(attn_fwd_fp8_kernel<64>, grid, block, stream, qp, kp, vp, op, lse, H, N_q, N_k,
                                     vt_row_stride, c, o_scale, q_sign, causal01, coff, nqt);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
