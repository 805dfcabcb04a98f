// Unfused attention forward (f16 / bf16): the step-by-step computation that
// the fused kernel replaces, kept as a measured contrast. It materialises S
// and P in HBM. Slides "Case study: FlashAttention": done step by step, S and
// P (n x n per head) go out to HBM and back (slide "FlashAttention: the
// idea"), they are 64x larger than Q, K, V, O at the Llama-3-8B shape and
// grow as n^2 (slide "The same computation at real size"), while the fused
// kernel's memory grows as n (slide "Takeaways"):
//   1. unf_scores : S = scale Q K^T (+ causal mask as -inf), fp32 [bh][n][n]
//   2. unf_softmax: per row m = max S, l = sum exp(S - m), P = exp(S - m) / l
//                   in the input type, LSE = m + ln l
//   3. unf_pv     : O = P V
// Each step is a plain kernel of its own; nothing is fused or skipped (the
// causal upper triangle is written as -inf and read back like any entry).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kUnfWaves = 4;
constexpr int kUnfThreads = 64 * kUnfWaves;

// 1. S = scale Q K^T. Each wave owns 32 keys (K rows as B operands in
// registers) and walks every 32-query block: the accumulator C[query][key]
// puts one key on each lane, so every register of the 32 lanes of a half
// stores 128 contiguous bytes of one S row.
template <Elt IN, int D, bool CAUSAL>
__global__ __launch_bounds__(kUnfThreads) void unf_scores(UnfArgs a) {
  constexpr int NKS = D / 16;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int n = a.n;
  const int ktiles = (n + 32 * kUnfWaves - 1) / (32 * kUnfWaves);
  const int bh = blockIdx.x / ktiles;
  const int key = (blockIdx.x % ktiles) * 32 * kUnfWaves + 32 * w + lr;
  const size_t head_off = (size_t)bh * (size_t)n * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint8_t*)a.q + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint8_t*)a.k + head_off * 2, head_bytes);
  u32x4_t kf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) kf[ks] = bload16(rk, ((uint32_t)key * D + ks * 16 + hl * 8) * 2);
  float* S = a.s + (size_t)bh * n * n;
  for (int q0 = 0; q0 < n; q0 += 32) {
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4_t qa = bload16(rq, ((uint32_t)(q0 + lr) * D + ks * 16 + hl * 8) * 2);
      acc = mfma16<IN>(qa, kf[ks], acc);
    }
    if (key < n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + 8 * (i >> 2) + 4 * hl + (i & 3);
        if (q < n) S[(size_t)q * n + key] = (CAUSAL && key > q) ? -INFINITY : acc[i] * a.scale;
      }
    }
  }
}

// 2. Row softmax: one wave per row, two passes over S (max and sum, then P).
template <Elt IN>
__global__ __launch_bounds__(kUnfThreads) void unf_softmax(UnfArgs a) {
  const int row = blockIdx.x * kUnfWaves + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = a.n;
  if (row >= a.rows) return;
  const float* S = a.s + (size_t)row * n;
  float m = -INFINITY, l = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float x = S[j];
    if (x > m) {
      l = l * fast_exp2((m - x) * kLog2e) + 1.f;  // m = -inf: l is 0, the product 0
      m = x;
    } else if (x != -INFINITY) {
      l += fast_exp2((x - m) * kLog2e);
    }
  }
  // combine the 64 lanes' (m, l)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float mo = __shfl_xor(m, off, 64);
    const float lo = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, mo);
    const float ea = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
    const float eb = mo == -INFINITY ? 0.f : fast_exp2((mo - mn) * kLog2e);
    l = l * ea + lo * eb;
    m = mn;
  }
  const float inv = 1.f / l;
  uint16_t* P = a.p + (size_t)row * n;
  for (int j = lane; j < n; j += 64) {
    const float p = fast_exp2((S[j] - m) * kLog2e) * inv;
    const uint32_t h = pack2<IN>(p, 0.f);
    P[j] = (uint16_t)(h & 0xffffu);
  }
  if (lane == 0 && a.lse) a.lse[row] = m + __logf(l);
}

// 3. O = P V. Four waves x 32 query rows; per 64-key tile, V is staged in LDS
// (row-major, swizzled as in the forward) and read with the transposing LDS
// read, P is read from HBM as B operands; O^T = V^T P^T on the MFMA.
template <Elt IN, int D>
__global__ __launch_bounds__(kUnfThreads) void unf_pv(UnfArgs a) {
  constexpr int ROWB = D * 2, BK = 64, NDB = D / 32;
  constexpr int CPR = D / 8;                          // 16-byte chunks per V row
  constexpr int NLD = BK * CPR / kUnfThreads;         // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint8_t vt[BK * ROWB];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int n = a.n;
  const int qtiles = (n + 32 * kUnfWaves - 1) / (32 * kUnfWaves);
  const int bh = blockIdx.x / qtiles;
  const int qrow = (blockIdx.x % qtiles) * 32 * kUnfWaves + 32 * w + lr;
  const size_t head_off = (size_t)bh * (size_t)n * D;
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint8_t*)a.v + head_off * 2, (uint32_t)n * ROWB);
  // one row of P per lane; rows past n read as zeros
  const uint16_t* Prow = a.p + ((size_t)bh * n + min(qrow, n - 1)) * n;
  const bool qok = qrow < n;
  const bool rows16 = (n & 7) == 0;  // P rows start 16-byte aligned
  auto vswz = [](int row) { return CPR == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };
  const int grp = lane >> 4, li = lane & 15;
  const int trow = 8 * hl + (li >> 2);
  const int sw = vswz(trow);
  const int tcol = 16 * (grp & 1) + 4 * (li & 3);
  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
  for (int k0 = 0; k0 < n; k0 += BK) {
    u32x4_t st[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + it * kUnfThreads, row = idx / CPR, c = idx % CPR;
      st[it] = bload16(rv, (uint32_t)(k0 + row) * ROWB + c * 16);
    }
    // P^T fragments: keys k0 + 16*s2 + 8*hl .. +8 of this lane's row (zeros past n)
    u32x4_t pb[BK / 16];
#pragma unroll
    for (int s2 = 0; s2 < BK / 16; ++s2) {
      const int kk = k0 + 16 * s2 + 8 * hl;
      u32x4_t x = u32x4_t{0, 0, 0, 0};
      if (qok) {
        if (rows16 && kk + 8 <= n) {
          x = *(const u32x4_t*)(Prow + kk);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) e[t] = kk + t < n ? Prow[kk + t] : (uint16_t)0;
#pragma unroll
          for (int t = 0; t < 4; ++t) x[t] = (uint32_t)e[2 * t] | ((uint32_t)e[2 * t + 1] << 16);
        }
      }
      pb[s2] = x;
    }
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + it * kUnfThreads, row = idx / CPR, c = idx % CPR;
      *(u32x4_t*)(vt + row * ROWB + ((c ^ vswz(row)) * 16)) = st[it];
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < BK / 16; ++s2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int r = 16 * s2 + trow, col = db * 32 + tcol;
        const uint8_t* p0 = vt + r * ROWB + (((col >> 3) ^ sw) * 16) + ((col & 4) << 1);
        const u32x2_t lo = lds_read_tr16(p0);
        const u32x2_t hi = lds_read_tr16(p0 + 4 * ROWB);
        o[db] = mfma16<IN>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pb[s2], o[db]);
      }
    }
  }
  if (qok) {
    uint16_t* O = (uint16_t*)a.o + head_off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hl;
        *(u32x2_t*)(O + d) = u32x2_t{pack2<IN>(o[db][4 * g], o[db][4 * g + 1]),
                                     pack2<IN>(o[db][4 * g + 2], o[db][4 * g + 3])};
      }
    }
  }
}

template <Elt E, int D>
hipError_t launch_unf_t(const UnfArgs& a, hipStream_t s) {
  const unsigned g13 = (unsigned)a.bh * (unsigned)((a.n + 127) / 128);
  const unsigned g2 = (unsigned)((a.rows + kUnfWaves - 1) / kUnfWaves);
  hipError_t e = a.causal ? launch_kernel(unf_scores<E, D, true>, dim3(g13), dim3(kUnfThreads), s, a)
                          : launch_kernel(unf_scores<E, D, false>, dim3(g13), dim3(kUnfThreads), s, a);
  if (e != hipSuccess) return e;
  e = launch_kernel(unf_softmax<E>, dim3(g2), dim3(kUnfThreads), s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(unf_pv<E, D>, dim3(g13), dim3(kUnfThreads), s, a);
}

}  // namespace

hipError_t launch_unfused(const UnfArgs& a, hipStream_t stream) {
  if (a.elt == Elt::F16)
    return a.d == 64 ? launch_unf_t<Elt::F16, 64>(a, stream) : launch_unf_t<Elt::F16, 128>(a, stream);
  return a.d == 64 ? launch_unf_t<Elt::BF16, 64>(a, stream) : launch_unf_t<Elt::BF16, 128>(a, stream);
}

}  // namespace fa
