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

// Launch the placement probe: out holds one HW_ID word per wave (8 * blocks).
int fa_probe_hwid(int blocks, uint32_t* out, void* stream) {
  if (blocks < 1 || !out) return (int)hipErrorInvalidValue;
  void* args[] = {&out};
  return (int)hipLaunchKernel((const void*)&hwid, dim3(blocks), dim3(512), args, 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"
