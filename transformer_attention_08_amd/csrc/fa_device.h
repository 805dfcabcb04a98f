// Device helpers shared by the forward and backward kernels (gfx950):
// vector types, the MFMA and packing wrappers, lane-pair exchanges, buffer
// resources, the direct-to-LDS copy, the transposing LDS read and the
// workgroup -> tile mapping. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896340736f;

struct TileId {
  int bh;
  int t;
};

// Workgroup id -> (batch*head, tile). With reverse, the tiles of a head are
// visited from the last one (the longest under a causal mask when a tile
// holds query rows). When the number of (batch, head) pairs is a multiple of
// 8, the workgroups of each head go to one XCD (workgroups are dispatched
// round-robin over the 8 XCDs), so a head's tiles share that XCD's L2; XCD x
// holds the pairs x, x + 8, x + 16, ..., so consecutive heads -- the heads of
// one sequence of a ragged batch -- spread over all XCDs. Each XCD takes its
// heads in groups of G, the longest tiles of a group first: a head's
// workgroups then run close together and re-read its K/V tiles from L2
// rather than HBM. The group size depends on the head's length in rows (the
// same rule for every kernel, whatever its tile size): heads of 16384 rows
// or more go one at a time (a head's keys then stream through the XCD in
// fewer rounds of its CUs), heads of 8192 to 16383 rows in groups of 2,
// shorter ones in one group, where the longest tiles of every head going
// first matters more for the tail than the re-reads. tile_rows is the
// calling kernel's rows (or keys) per tile; head_tiles (when not negative)
// is the head's length in such tiles when a workgroup holds more than one.
__device__ inline TileId tile_of_block(int pid, int bh_count, int tiles, bool reverse, int tile_rows,
                                       int head_tiles = -1) {
  int bh, tt;
  if ((bh_count & 7) == 0) {
    const int xcd = pid & 7, slot = pid >> 3, per = bh_count >> 3;
    const int rows = (head_tiles < 0 ? tiles : head_tiles) * tile_rows;
    const int G = rows >= 16384 ? 1 : (rows >= 8192 && (per & 1) == 0) ? 2 : per;
    const int g = slot / (G * tiles), r = slot - g * (G * tiles);
    tt = r / G;
    bh = (g * G + r % G) * 8 + xcd;
  } else {
    tt = pid / bh_count;
    bh = pid % bh_count;
  }
  return {bh, reverse ? tiles - 1 - tt : tt};
}

// Accumulator row m of S^T holds key perm32(m) of the 32-key block.
__device__ inline int perm32(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <Elt E>
__device__ inline uint32_t pack2(float a, float b) {
  if constexpr (E == Elt::F16) {
    f16x2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    bf16x2_t h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
}

// o += a * b on the 32x32x16 MFMA with 16-bit operands (F16 or BF16).
template <Elt E>
__device__ inline f32x16_t mfma16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (E == Elt::F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x of this lane and of lane ^ 32, in an order that is the same on both lanes.
struct PairVals {
  float a, b;
};
__device__ inline PairVals pair_vals(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ inline float pair_max(float x) {
  const PairVals p = pair_vals(x);
  return fmaxf(p.a, p.b);
}
__device__ inline float pair_sum(float x) {
  const PairVals p = pair_vals(x);
  return p.a + p.b;
}

// Buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros, which pads ragged tiles without branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline u32x2_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Bytes a buffer resource must cover for `rows` rows of `row_bytes` at a
// stride of `rs` bytes (0 rows: nothing).
__device__ inline uint32_t span_bytes(int rows, uint32_t rs, int row_bytes) {
  return rows > 0 ? (uint32_t)(rows - 1) * rs + (uint32_t)row_bytes : 0u;
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ inline u32x2_t lds_read_tr16(const uint8_t* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// One 16-byte buffer load per lane straight into LDS: lane i writes
// lds + 16 * i. lds must be the same for the whole wave (it goes to M0).
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, uint32_t voffset) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(m0)
               : "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Enqueue kernel(a) and return the status of this launch itself (never a
// stale error that an earlier, unrelated HIP call left on the thread, which
// hipGetLastError would report -- and clear -- instead).
template <typename A>
inline hipError_t launch_kernel(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t stream, const A& a) {
  A arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
}

}  // namespace
}  // namespace fa
