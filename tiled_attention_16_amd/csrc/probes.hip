// Microbenchmarks of the gfx950 instruction rates the attention kernels are
// designed around (measurement only; not part of the attention library's C
// ABI). Each probe kernel runs a fixed, bounded loop per wave and records,
// per workgroup, the shader-clock cycles (s_memtime) and the 100 MHz
// real-time counter (s_memrealtime) at its start and end, from which the host
// derives the clock and the per-instruction cost.
//
//   mfma     back-to-back v_mfma_f32_32x32x16_bf16 on four independent
//            accumulators, optionally with `nv` VALU instructions (v_fma_f32,
//            v_exp_f32, v_cvt_pk_bf16_f32 or v_add_f32) issued after each
//            MFMA: the MFMA-only rate and how much VALU work an MFMA hides;
//   valu     32 of one of those VALU instructions per loop step, no MFMA;
//   chain    v_mfma_f32_32x32x16_bf16 accumulating into one accumulator (a
//            dependent chain) or two in turn;
//   mfma16   back-to-back v_mfma_f32_16x16x32_bf16 on four independent
//            accumulators (half the flops of the 32x32x16 form per instruction);
//   lds      ds_read_b128 or ds_read_b64_tr_b16 streams over a 64 KB LDS
//            buffer, bank-conflict free, eight reads in flight per wave; the
//            buffer holds distinct words and the reads are summed, so no read
//            can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ void stamp(unsigned long long* t, int slot) {
  // one lane of wave 0 of each workgroup records (cycles, real time)
  const unsigned long long c = __builtin_amdgcn_s_memtime();
  const unsigned long long r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    t[4 * blockIdx.x + 2 * slot] = c;
    t[4 * blockIdx.x + 2 * slot + 1] = r;
  }
}

// Op: 0 v_fma_f32, 1 v_exp_f32, 2 v_cvt_pk_bf16_f32, 3 v_add_f32; each
// instruction reads and writes one of 8 registers in turn.
template <int NV, int Op>
__device__ __forceinline__ void valu_block(float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if constexpr (Op == 1) asm volatile("v_exp_f32 %0, %0" : "+v"(x[i & 7]));
    else if constexpr (Op == 2) asm volatile("v_cvt_pk_bf16_f32 %0, %0, %0" : "+v"(x[i & 7]));
    else if constexpr (Op == 3) asm volatile("v_add_f32 %0, %0, %0" : "+v"(x[i & 7]));
    else asm volatile("v_fma_f32 %0, %0, %0, %0" : "+v"(x[i & 7]));
  }
}

// iters steps of 4 MFMAs (4 independent accumulators), NV VALU instructions
// after each MFMA.
template <int NV, int Op>
__global__ __launch_bounds__(512) void probe_mfma_kernel(int iters, unsigned long long* t, float* sink) {
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = (f32x16){};
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x & 7));
    b[i] = (__bf16)(0.002f * i);
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 1e-3f * (i + 1);
  __syncthreads();
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc[j]) : "a"(a), "a"(b));
      valu_block<NV, Op>(x);
    }
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();
  stamp(t, 1);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][threadIdx.x & 15];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  if (s == 12345.f) sink[threadIdx.x] = s;   // never true for these inputs; keeps the work alive
}

// iters steps of 4 MFMAs that all accumulate into `Acc` independent
// accumulators in turn (Acc = 1: one dependent chain, each MFMA reads the
// previous one's result as its C operand; Acc = 2: two interleaved chains).
template <int Acc>
__global__ __launch_bounds__(512) void probe_mfma_chain_kernel(int iters, unsigned long long* t, float* sink) {
  f32x16 acc[Acc];
#pragma unroll
  for (int j = 0; j < Acc; ++j) acc[j] = (f32x16){};
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x & 7));
    b[i] = (__bf16)(0.002f * i);
  }
  __syncthreads();
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc[j % Acc]) : "a"(a), "a"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();
  stamp(t, 1);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < Acc; ++j) s += acc[j][threadIdx.x & 15];
  if (s == 12345.f) sink[threadIdx.x] = s;   // never true for these inputs; keeps the work alive
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(512) void probe_mfma16_kernel(int iters, unsigned long long* t, float* sink) {
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = (f32x4){};
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x & 7));
    b[i] = (__bf16)(0.002f * i);
  }
  __syncthreads();
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[j]) : "a"(a), "a"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();
  stamp(t, 1);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][threadIdx.x & 3];
  if (s == 12345.f) sink[threadIdx.x] = s;   // never true for these inputs; keeps the work alive
}

template <int NV, int Op>
__global__ __launch_bounds__(512) void probe_valu_kernel(int iters, unsigned long long* t, float* sink) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 1e-3f * (i + 1 + (threadIdx.x & 3));
  __syncthreads();
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) valu_block<NV, Op>(x);
  __syncthreads();
  stamp(t, 1);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  if (s == 12345.f) sink[threadIdx.x] = s;
}

// LDS read streams: every wave reads the same 64 KB buffer, 8 reads per step,
// lane offsets 16 * lane (b128) or 8 * lane (b64 transposing), which touch
// every bank equally.
template <bool Tr>
__global__ __launch_bounds__(512) void probe_lds_kernel(int iters, unsigned long long* t, float* sink) {
  __shared__ __attribute__((aligned(1024))) char buf[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += blockDim.x)
    *(lds_u32x4*)(buf + 16 * i) = (u32x4){4u * i + 1u, 4u * i + 2u, 4u * i + 3u, 4u * i + 4u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) {
    const int base = ((it + wave) & 7) * 8192;   // a different 8 KB block every step
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (Tr) {
        const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + base + j * 1024 + 8 * lane));
        acc[j & 3] += __builtin_bit_cast(uint2, v).x;
      } else {
        acc += *(const lds_u32x4*)(buf + base + j * 1024 + 16 * lane);
      }
    }
  }
  __syncthreads();
  stamp(t, 1);
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[threadIdx.x] = 1.f;   // keeps every read
}

template <typename K>
int run(K kern, int blocks, int threads, int iters, unsigned long long* t, float* sink, hipStream_t s) {
  if (blocks <= 0 || threads <= 0 || threads > 512 || threads % 64 != 0 || iters <= 0 || !t || !sink) return 1;
  void* args[] = {&iters, &t, &sink};
  return hipLaunchKernel((const void*)kern, dim3(blocks), dim3(threads), args, 0, s) == hipSuccess ? 0 : 2;
}

}  // namespace

// kind: 0 mfma, 1 valu, 2 lds, 3 mfma16 (op and nv 0), 4 dependent MFMA chains (op: 1 or 2 chains). op (mfma, valu): 0 v_fma_f32, 1 v_exp_f32,
// 2 v_cvt_pk_bf16_f32, 3 v_add_f32; (lds) 0 ds_read_b128, 1
// ds_read_b64_tr_b16. nv: VALU instructions after each MFMA (mfma: 0, 2, 4,
// 6, 8) or per loop step (valu: 32). t: device, 4 * blocks unsigned 64-bit
// words (per workgroup: start cycles, start real time, end cycles, end real
// time). sink: device, >= threads floats (never written for the inputs
// used). Returns 0, 1 for bad arguments, 2 for a failed launch.
template <int Op>
int run_mfma(int nv, int blocks, int threads, int iters, unsigned long long* t, float* sink, hipStream_t s) {
  switch (nv) {
    case 2: return run(probe_mfma_kernel<2, Op>, blocks, threads, iters, t, sink, s);
    case 4: return run(probe_mfma_kernel<4, Op>, blocks, threads, iters, t, sink, s);
    case 6: return run(probe_mfma_kernel<6, Op>, blocks, threads, iters, t, sink, s);
    case 8: return run(probe_mfma_kernel<8, Op>, blocks, threads, iters, t, sink, s);
    default: return 1;
  }
}

extern "C" int attn_probe(int kind, int op, int nv, int blocks, int threads, int iters, unsigned long long* t,
                          float* sink, hipStream_t stream) {
  if (kind == 0) {
    if (nv == 0) return run(probe_mfma_kernel<0, 0>, blocks, threads, iters, t, sink, stream);
    switch (op) {
      case 0: return run_mfma<0>(nv, blocks, threads, iters, t, sink, stream);
      case 1: return run_mfma<1>(nv, blocks, threads, iters, t, sink, stream);
      case 2: return run_mfma<2>(nv, blocks, threads, iters, t, sink, stream);
      case 3: return run_mfma<3>(nv, blocks, threads, iters, t, sink, stream);
      default: return 1;
    }
  }
  if (kind == 1) {
    if (nv != 32) return 1;
    switch (op) {
      case 0: return run(probe_valu_kernel<32, 0>, blocks, threads, iters, t, sink, stream);
      case 1: return run(probe_valu_kernel<32, 1>, blocks, threads, iters, t, sink, stream);
      case 2: return run(probe_valu_kernel<32, 2>, blocks, threads, iters, t, sink, stream);
      case 3: return run(probe_valu_kernel<32, 3>, blocks, threads, iters, t, sink, stream);
      default: return 1;
    }
  }
  if (kind == 2) return run(op == 1 ? probe_lds_kernel<true> : probe_lds_kernel<false>, blocks, threads, iters, t, sink,
                            stream);
  if (kind == 3) return run(probe_mfma16_kernel, blocks, threads, iters, t, sink, stream);
  if (kind == 4) return run(op == 2 ? probe_mfma_chain_kernel<2> : probe_mfma_chain_kernel<1>, blocks, threads, iters, t,
                            sink, stream);
  return 1;
}
