// Rate probes for gfx950 (not part of the attention library; they are built
// into libfa_probe.so and driven by `bench.py --mfma-rate` and
// `bench.py --lds-rate`).
//
// MFMA rate.
// Each wave issues `iters` rounds of NACC independent MFMAs (NACC separate
// accumulators, operands held in registers, no memory traffic inside the
// timed loop) and records its own elapsed shader cycles (s_memtime) and the
// elapsed ticks of the fixed 100 MHz counter (s_memrealtime). One workgroup
// per CU (the workgroup asks for more than half of the 160 KiB LDS), with
// `waves_per_simd` waves on each of the four SIMDs. Cycles per MFMA per wave
// then give the issue rate of the instruction: at the dense bf16/f16 peak of
// 2.5 PFLOP/s (256 CUs, 2.4 GHz) a SIMD retires 1024 FLOP per cycle, i.e.
// 32 cycles per 32x32x16 MFMA and 16 per 16x16x32 MFMA. The ratio of the two
// counters gives the shader clock the probe ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 96 * 1024;

// KIND: 0 = 32x32x16 bf16, 1 = 16x16x32 bf16, 2 = 32x32x16 f16, 3 = 16x16x32 f16
template <int KIND>
struct Acc {
  typedef typename std::conditional<(KIND & 1) == 0, f32x16_t, f32x4_t>::type type;
};

template <int KIND>
__device__ inline typename Acc<KIND>::type mfma(bf16x8_t a, bf16x8_t b, typename Acc<KIND>::type c) {
  if constexpr (KIND == 0) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else if constexpr (KIND == 1) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else if constexpr (KIND == 2)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int KIND, int NACC>
__global__ __launch_bounds__(512) void mfma_rate(uint64_t* out, float* sink, int iters) {
  __shared__ uint8_t lds[kLdsBytes];
  using A = typename Acc<KIND>::type;
  const int lane = threadIdx.x & 63;
  // operands that depend on the lane, so nothing folds
  bf16x8_t a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + 0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + e) & 7));
  }
  A acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = A{};
  for (int i = threadIdx.x; i < kLdsBytes; i += blockDim.x) lds[i] = (uint8_t)(i == iters);
  __syncthreads();
  const float l0 = (float)lds[(threadIdx.x * 37) % kLdsBytes];  // keeps the LDS allocation
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[i] = mfma<KIND>(a, b, acc[i]);
  }
  // wait for the last results before reading the clocks again
  float s = l0;
#pragma unroll
  for (int i = 0; i < NACC; ++i) s += acc[i][0];
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime() + (uint64_t)(s == 12345.f);
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (lane == 0) {
    out[2 * wave] = c1 - c0;
    out[2 * wave + 1] = r1 - r0;
  }
  if (s == 12345.f) sink[threadIdx.x] = s;
}

template <int KIND>
hipError_t launch_kind(int nacc, int threads, int blocks, int iters, uint64_t* out, float* sink, hipStream_t st) {
  void* args[] = {&out, &sink, &iters};
  const void* f = nullptr;
  switch (nacc) {
    case 1: f = (const void*)&mfma_rate<KIND, 1>; break;
    case 2: f = (const void*)&mfma_rate<KIND, 2>; break;
    case 4: f = (const void*)&mfma_rate<KIND, 4>; break;
    case 8: f = (const void*)&mfma_rate<KIND, 8>; break;
    default: return hipErrorInvalidValue;
  }
  return hipLaunchKernel(f, dim3(blocks), dim3(threads), args, 0, st);
}

// LDS read rate. Each wave issues `iters` rounds of 8 independent LDS reads
// (MODE 0: ds_read_b128, 16 bytes per lane; MODE 1: ds_read_b64_tr_b16, the
// transposing 8-byte read) at bank-conflict-free addresses, and waits for
// each round before the next (an empty asm statement consumes every
// result, so no vector instruction is spent on them). One workgroup per CU.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int MODE>
__global__ __launch_bounds__(512) void lds_rate(uint64_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16)
    *(u32x4_t*)(lds + i) = u32x4_t{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    const int base = ((it & 7) * 8192 + wave * 1024) & (65536 - 1);
    if constexpr (MODE == 0) {
      u32x4_t r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) r[u] = *(const u32x4_t*)(lds + ((base + u * 1024 + lane * 16) & 65535));
#pragma unroll
      for (int u = 0; u < 8; ++u) asm volatile("" ::"v"(r[u]));
    } else {
      s16x4_t r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        r[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(lds + ((base + u * 512 + lane * 8) & 65535)));
#pragma unroll
      for (int u = 0; u < 8; ++u) asm volatile("" ::"v"(r[u]));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  if (lane == 0) {
    out[2 * gw] = c1 - c0;
    out[2 * gw + 1] = r1 - r0;
  }
}


// MFMA / vector co-issue. Eight waves per CU, two per SIMD: waves 0-3 issue
// 32x32x16 bf16 MFMAs on four accumulators, waves 4-7 run a softmax-like
// vector stream (fma, exp2, add, max3, packing to bf16 over 64 registers,
// four independent chains). ROLE: 1 = matrix waves only, 2 = vector waves
// only, 3 = both. OPND (matrix waves): 0 = operands held in registers,
// 1 = one 16-byte LDS read per MFMA (a K operand), 2 = two transposing
// 8-byte LDS reads per MFMA (a V^T operand), both issued six MFMAs ahead.
typedef float f32x16_t2 __attribute__((ext_vector_type(16)));

template <int OPND>
__device__ inline u32x4_t opnd_read(const uint8_t* lds, int i, int lane) {
  if constexpr (OPND == 1) {
    return *(const u32x4_t*)(lds + ((i & 31) * 1024 + lane * 16));
  } else {
    const int base = (i & 31) * 1024 + (lane & 15) * 8 + (lane >> 4) * 256;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(lds + base));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(lds + base + 128));
    const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{a[0], a[1], b[0], b[1]};
  }
}

template <int OPND>
__global__ __launch_bounds__(512) void coissue(uint64_t* out, float* sink, int iters, int role) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16)
    *(u32x4_t*)(lds + i) = u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool matrix = wave < 4;
  float sres = 0.f;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  if (matrix && (role & 1)) {
    bf16x8_t b;
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + e) & 7));
    f32x16_t2 acc[4] = {};
    if constexpr (OPND == 0) {
      bf16x8_t a;
      for (int e = 0; e < 8; ++e) a[e] = (__bf16)(1.0f + 0.001f * (float)((lane + e) & 7));
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 3], 0, 0, 0);
      }
    } else {
      for (int it = 0; it < iters; ++it) {
        u32x4_t buf[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) buf[i] = opnd_read<OPND>(lds, i, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, buf[i % 6]), b, acc[i & 3], 0, 0, 0);
          if (i + 6 < 32) buf[i % 6] = opnd_read<OPND>(lds, i + 6, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) sres += acc[k][0];
  } else if (!matrix && (role & 2)) {
    float x[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = 0.01f * (float)((lane + i) & 15) - 0.05f;
    float m = 0.f, l = 0.f;
    uint32_t pk = 0;
    for (int it = 0; it < iters; ++it) {
      // one softmax of 64 scores per lane: max, scale and subtract, exp2, sum, pack
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 64; ++i) mx = fmaxf(mx, x[i]);
      const float nm = -mx * 0.125f;
      float ls0 = 0.f, ls1 = 0.f, ls2 = 0.f, ls3 = 0.f;
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], 0.125f, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], 0.125f, nm));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 2], 0.125f, nm));
        const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 3], 0.125f, nm));
        ls0 += p0; ls1 += p1; ls2 += p2; ls3 += p3;
        bf16x2_t h = {(__bf16)p0, (__bf16)p1};
        bf16x2_t g = {(__bf16)p2, (__bf16)p3};
        pk ^= __builtin_bit_cast(uint32_t, h) ^ __builtin_bit_cast(uint32_t, g);
        x[i] = p0 * 0.999f;
      }
      m += mx;
      l += (ls0 + ls1) + (ls2 + ls3);
    }
    sres = m + l + (float)(pk & 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  if (lane == 0) out[gw] = c1 - c0;
  if (sres == 12345.f) sink[threadIdx.x] = sres;
}

// Scores of e4m3 attention inputs on the two matrix paths an e4m3 kernel
// could take: v_mfma_f32_32x32x16_fp8_fp8 on the codes themselves, and
// v_mfma_f32_32x32x16_bf16 on the codes widened exactly to bf16 (every e4m3
// value is a bf16 value). One wave per 32 x 32 block of S = Q K^T (raw
// scores, before any scale), queries [0, rows) against all n keys of one
// head; q8 and k8 are row-major e4m3 [n][128]. out8 / out16 are fp32
// [rows][n].
__global__ __launch_bounds__(64) void fp8_scores(const uint8_t* q8, const uint8_t* k8, int n, float* out8,
                                                float* out16) {
  const int lane = threadIdx.x, lr = lane & 31, hl = lane >> 5;
  const int q0 = blockIdx.y * 32, k0 = blockIdx.x * 32;
  f32x16_t2 s8 = {}, s16 = {};
  for (int ks = 0; ks < 8; ++ks) {
    const int dcol = ks * 16 + hl * 8;
    const uint64_t a = *(const uint64_t*)(k8 + (size_t)(k0 + lr) * 128 + dcol);  // key k0 + lr
    const uint64_t b = *(const uint64_t*)(q8 + (size_t)(q0 + lr) * 128 + dcol);  // query q0 + lr
    s8 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8((long)a, (long)b, s8, 0, 0, 0);
    const uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32), blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
    u32x4_t aw = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(alo, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(alo, 1.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ahi, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ahi, 1.0f, true))};
    u32x4_t bw = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(blo, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(blo, 1.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bhi, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bhi, 1.0f, true))};
    s16 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw), __builtin_bit_cast(bf16x8_t, bw),
                                                 s16, 0, 0, 0);
  }
  // accumulator register i of lane (lr, hl): key k0 + 8 (i / 4) + 4 hl + i % 4, query q0 + lr
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = k0 + 8 * (i / 4) + 4 * hl + (i % 4);
    const size_t at = (size_t)(q0 + lr) * n + key;
    out8[at] = s8[i];
    out16[at] = s16[i];
  }
}

// Global -> LDS copy rate, and how copies share the LDS with operand reads.
// One workgroup of eight waves per CU (96 KiB of LDS). A copying wave moves
// 4 KiB per round from src (offsets cycle through src_bytes, a power of two
// of at least 64 KiB) into a double-buffered LDS area:
//   MODE 0: all eight waves copy straight into LDS (buffer_load_dwordx4 ... lds);
//   MODE 1: all eight waves copy through registers (16-byte buffer loads,
//           then ds_write_b128), two rounds of registers in flight;
//   MODE 2: waves 0-3 copy as in MODE 0 while waves 4-7 read LDS
//           (eight ds_read_b128 per round) until the copies are done;
//   MODE 3: as MODE 2 with MODE 1's copies;
//   MODE 4: waves 4-7 read LDS alone (for as many rounds as in MODE 2);
//   MODE 5: waves 0-3 copy as in MODE 0 while waves 4-7 issue 32x32x16 bf16
//           MFMAs whose A operands are 16-byte LDS reads (six ahead, 32 per
//           round) until the copies are done;
//   MODE 6: those MFMA waves alone (`iters` rounds);
//   MODE 7: as MODE 5 with MODE 1's copies.
// out holds, per wave, its elapsed shader cycles and its rounds.
__device__ inline void probe_dma16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, uint32_t voffset) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voffset), "s"(rsrc), "{m0}"(m0) : "memory");
}

template <int MODE>
__global__ __launch_bounds__(512) void copy_rate(const uint8_t* src, uint32_t src_bytes, uint64_t* out, float* sink,
                                                 int iters) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  __shared__ int done;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, (int)src_bytes, 0x00020000);
  for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16) *(u32x4_t*)(lds + i) = u32x4_t{1u, 2u, 3u, 4u};
  if (threadIdx.x == 0) done = 0;
  __syncthreads();
  const bool copier = MODE <= 1 || ((MODE <= 3 || MODE == 5 || MODE == 7) && wave < 4);
  const bool reader = MODE >= 2 && MODE <= 4 && wave >= 4;
  const bool matrix = MODE >= 5 && wave >= 4;
  constexpr bool kRegCopy = MODE == 1 || MODE == 3 || MODE == 7;
  const int cw = MODE <= 1 ? wave : (wave & 3);        // copier slot
  const int ncw = MODE <= 1 ? 8 : 4;                   // copying waves
  int rounds = 0;
  float acc = 0.f;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  if (copier) {
    auto off = [&](int it, int i) { return (((uint32_t)(it * ncw + cw) * 4096u) & (src_bytes - 1)) + i * 1024 + lane * 16; };
    auto dst = [&](int it, int i) { return lds + (it & 1) * (ncw * 4096) + cw * 4096 + i * 1024; };
    if constexpr (!kRegCopy) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) probe_dma16(rsrc, dst(it, i), off(it, i));
        __builtin_amdgcn_s_waitcnt((4 & 15) | (7 << 4) | (15 << 8));  // vmcnt(4): one round in flight
      }
    } else {
      u32x4_t ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off(0, i), 0, 0));
      for (int it = 0; it + 1 < iters; it += 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          rb[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off(it + 1, i), 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4_t*)(dst(it, i) + lane * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ra[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off(it + 2, i), 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4_t*)(dst(it + 1, i) + lane * 16) = rb[i];
      }
    }
    rounds = iters;
    __builtin_amdgcn_s_waitcnt(0);
    acc = __uint_as_float(*(const uint32_t*)(lds + (threadIdx.x * 4100) % kLdsBytes));  // keeps the copies
    if (MODE >= 2 && lane == 0) __hip_atomic_fetch_add(&done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else if (matrix) {
    bf16x8_t bop;
    for (int e = 0; e < 8; ++e) bop[e] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + e) & 7));
    f32x16_t macc[4] = {};
    const int cap = MODE == 6 ? iters : 64 * iters;
    const uint8_t* abase = lds + 32768 + (wave & 3) * 8192;  // outside the copies' double buffer
    auto rd = [&](int i) { return *(const u32x4_t*)(abase + ((i & 7) * 1024 + lane * 16)); };
    for (int it = 0; it < cap; ++it) {
      u32x4_t buf[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) buf[i] = rd(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        macc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, buf[i % 6]), bop, macc[i & 3], 0, 0, 0);
        if (i + 6 < 32) buf[i % 6] = rd(i + 6);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++rounds;
      if (MODE != 6 && __hip_atomic_load(&done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 4) break;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += macc[k][0];
  } else if (reader) {
    const int cap = MODE == 4 ? iters : 64 * iters;
    u32x4_t x = {};
    for (int it = 0; it < cap; ++it) {
      u32x4_t r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) r[u] = *(const u32x4_t*)(lds + ((it * 8 + u) * 1024 + (wave & 3) * 16384 + lane * 16) % kLdsBytes);
#pragma unroll
      for (int u = 0; u < 8; ++u) x ^= r[u];
      ++rounds;
      if (MODE != 4 && (it & 7) == 7 && __hip_atomic_load(&done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 4) break;
    }
    acc = (float)(x[0] ^ x[1] ^ x[2] ^ x[3]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const int gw = blockIdx.x * 8 + wave;
  if (lane == 0) {
    out[2 * gw] = c1 - c0;
    out[2 * gw + 1] = (uint64_t)rounds;
  }
  if (acc == 12345.f) sink[threadIdx.x] = acc;
}

// Vector ALU rate. Waves 0-3 (one per SIMD) run operation A, waves 4-7 (the
// SIMD partners of waves 0-3) run operation B; 0 = idle, 1 = v_exp_f32,
// 2 = v_fma_f32, 3 = v_add_f32, 4 = v_cvt_pk_bf16_f32, 5 = v_max3_f32,
// 6 = v_exp_f16, 7 = v_mfma_f32_32x32x16_bf16 (four accumulators). Each
// round issues 16 independent instructions (no result feeds a source in the
// same round) and each wave records its elapsed shader cycles.
template <int OP>
__device__ inline float valu_round(float (&x)[16], const float (&y)[16], f32x16_t (&acc)[4], bf16x8_t a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (OP == 1) asm volatile("v_exp_f32 %0, %1" : "=v"(x[i]) : "v"(y[i]));
    else if constexpr (OP == 2) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x[i]) : "v"(y[i]), "v"(y[(i + 1) & 15]));
    else if constexpr (OP == 3) asm volatile("v_add_f32 %0, %1, %2" : "=v"(x[i]) : "v"(y[i]), "v"(y[(i + 1) & 15]));
    else if constexpr (OP == 4) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(x[i]) : "v"(y[i]), "v"(y[(i + 1) & 15]));
    else if constexpr (OP == 5) asm volatile("v_max3_f32 %0, %1, %2, %0" : "+v"(x[i]) : "v"(y[i]), "v"(y[(i + 1) & 15]));
    else if constexpr (OP == 6) asm volatile("v_exp_f16 %0, %1" : "=v"(x[i]) : "v"(y[i]));
    else if constexpr (OP == 7) {
      if ((i & 1) == 0) acc[(i >> 1) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[(i >> 1) & 3], 0, 0, 0);
    }
  }
  float r = 0.f;
  if constexpr (OP >= 1 && OP <= 6) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(x[i]));
  }
  return r;
}

template <int OP>
__device__ inline void valu_run(int iters, float* sink, uint64_t* out, int gw, int lane) {
  float x[16], y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) { y[i] = 0.01f * (float)((lane + i) & 15) - 0.07f; x[i] = y[i]; }
  bf16x8_t a;
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)(1.0f + 0.001f * (float)((lane + e) & 7));
  f32x16_t acc[4] = {};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) valu_round<OP>(x, y, acc, a);
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  float r = x[0] + acc[0][0] + acc[1][0] + acc[2][0] + acc[3][0];
  if (lane == 0) out[gw] = c1 - c0;
  if (r == 12345.f) sink[lane] = r;
}

__global__ __launch_bounds__(512) void valu_rate(uint64_t* out, float* sink, int iters, int op_a, int op_b) {
  // one workgroup per CU: the workgroup asks for more than half of the LDS
  __shared__ uint8_t lds[kLdsBytes];
  for (int i = threadIdx.x; i < kLdsBytes; i += blockDim.x) lds[i] = (uint8_t)(i == iters);
  __syncthreads();
  if (lds[(threadIdx.x * 37) % kLdsBytes] == 7) sink[threadIdx.x] = 1.f;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * 8 + wave;
  const int op = wave < 4 ? op_a : op_b;
  switch (op) {
    case 1: valu_run<1>(iters, sink, out, gw, lane); break;
    case 2: valu_run<2>(iters, sink, out, gw, lane); break;
    case 3: valu_run<3>(iters, sink, out, gw, lane); break;
    case 4: valu_run<4>(iters, sink, out, gw, lane); break;
    case 5: valu_run<5>(iters, sink, out, gw, lane); break;
    case 6: valu_run<6>(iters, sink, out, gw, lane); break;
    case 7: valu_run<7>(iters, sink, out, gw, lane); break;
    default: if (lane == 0) out[gw] = 0; break;
  }
}

// Wave placement: each wave of a 512-thread workgroup records the HW_ID
// hardware register (SIMD, CU, shader array and engine it runs on).
__global__ __launch_bounds__(512) void hwid(uint32_t* out) {
  const uint32_t id = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);  // HW_REG_HW_ID, 32 bits
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if ((threadIdx.x & 63) == 0) out[wave] = id;
}

}  // namespace

extern "C" {

// Launch the probe: `blocks` workgroups of 4 * waves_per_simd waves each.
// out: device array of 2 * blocks * 4 * waves_per_simd uint64 (per wave:
// shader cycles, 100 MHz ticks). sink: device array of 512 floats (never
// written in practice). Returns 0 or a hipError_t code; nothing is
// allocated.
int fa_probe_mfma_rate(int kind, int nacc, int waves_per_simd, int blocks, int iters, uint64_t* out,
                       float* sink, void* stream) {
  if (waves_per_simd < 1 || waves_per_simd > 2 || blocks < 1 || iters < 1 || !out || !sink) return (int)hipErrorInvalidValue;
  const int threads = 256 * waves_per_simd;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case 0: e = launch_kind<0>(nacc, threads, blocks, iters, out, sink, st); break;
    case 1: e = launch_kind<1>(nacc, threads, blocks, iters, out, sink, st); break;
    case 2: e = launch_kind<2>(nacc, threads, blocks, iters, out, sink, st); break;
    case 3: e = launch_kind<3>(nacc, threads, blocks, iters, out, sink, st); break;
    default: e = hipErrorInvalidValue;
  }
  return (int)e;
}

// Launch the LDS read probe: `blocks` workgroups of `waves` waves (1..8);
// mode 0 = ds_read_b128, 1 = ds_read_b64_tr_b16. out as for the MFMA probe
// (2 * blocks * waves uint64).
int fa_probe_lds_rate(int mode, int waves, int blocks, int iters, uint64_t* out, void* stream) {
  if (waves < 1 || waves > 8 || blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  void* args[] = {&out, &iters};
  const void* f = mode == 0 ? (const void*)&lds_rate<0> : mode == 1 ? (const void*)&lds_rate<1> : nullptr;
  if (!f) return (int)hipErrorInvalidValue;
  return (int)hipLaunchKernel(f, dim3(blocks), dim3(64 * waves), args, 0, static_cast<hipStream_t>(stream));
}

// Launch the co-issue probe: `blocks` workgroups of 8 waves; out holds one
// uint64 of shader cycles per wave (8 * blocks).
int fa_probe_coissue(int opnd, int role, int blocks, int iters, uint64_t* out, float* sink, void* stream) {
  if (role < 1 || role > 3 || blocks < 1 || iters < 1 || !out || !sink) return (int)hipErrorInvalidValue;
  void* args[] = {&out, &sink, &iters, &role};
  const void* f = opnd == 0 ? (const void*)&coissue<0> : opnd == 1 ? (const void*)&coissue<1>
                : opnd == 2 ? (const void*)&coissue<2> : nullptr;
  if (!f) return (int)hipErrorInvalidValue;
  return (int)hipLaunchKernel(f, dim3(blocks), dim3(512), args, 0, static_cast<hipStream_t>(stream));
}

// Launch the copy-rate probe: `blocks` workgroups of 8 waves; src holds
// src_bytes (a power of two, at least 65536); out holds 2 uint64 per wave
// (16 * blocks).
int fa_probe_copy_rate(int mode, const void* src, unsigned src_bytes, int blocks, int iters, uint64_t* out,
                       float* sink, void* stream) {
  if (mode < 0 || mode > 7 || !src || src_bytes < 65536 || (src_bytes & (src_bytes - 1)) || blocks < 1 || iters < 2 ||
      iters % 2 || !out || !sink)
    return (int)hipErrorInvalidValue;
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  void* args[] = {&s8, &src_bytes, &out, &sink, &iters};
  const void* fs[8] = {(const void*)&copy_rate<0>, (const void*)&copy_rate<1>, (const void*)&copy_rate<2>,
                       (const void*)&copy_rate<3>, (const void*)&copy_rate<4>, (const void*)&copy_rate<5>,
                       (const void*)&copy_rate<6>, (const void*)&copy_rate<7>};
  const void* f = fs[mode];
  return (int)hipLaunchKernel(f, dim3(blocks), dim3(512), args, 0, static_cast<hipStream_t>(stream));
}

// Launch the vector ALU rate probe: `blocks` workgroups of 8 waves; out
// holds one uint64 of shader cycles per wave (8 * blocks); op codes as in
// valu_rate (0-7).
int fa_probe_valu_rate(int op_a, int op_b, int blocks, int iters, uint64_t* out, float* sink, void* stream) {
  if (op_a < 0 || op_a > 7 || op_b < 0 || op_b > 7 || blocks < 1 || iters < 1 || !out || !sink)
    return (int)hipErrorInvalidValue;
  void* args[] = {&out, &sink, &iters, &op_a, &op_b};
  return (int)hipLaunchKernel((const void*)&valu_rate, dim3(blocks), dim3(512), args, 0,
                              static_cast<hipStream_t>(stream));
}

// Launch the e4m3 score probe: rows and n multiples of 32, d_k 128.
int fa_probe_fp8_scores(const void* q8, const void* k8, int n, int rows, float* out8, float* out16, void* stream) {
  if (!q8 || !k8 || !out8 || !out16 || n < 32 || rows < 32 || n % 32 || rows % 32 || rows > n)
    return (int)hipErrorInvalidValue;
  void* args[] = {&q8, &k8, &n, &out8, &out16};
  return (int)hipLaunchKernel((const void*)&fp8_scores, dim3(n / 32, rows / 32), dim3(64), args, 0,
                              static_cast<hipStream_t>(stream));
}

// Launch the placement probe: out holds one HW_ID word per wave (8 * blocks).
int fa_probe_hwid(int blocks, uint32_t* out, void* stream) {
  if (blocks < 1 || !out) return (int)hipErrorInvalidValue;
  void* args[] = {&out};
  return (int)hipLaunchKernel((const void*)&hwid, dim3(blocks), dim3(512), args, 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"
