// Attention backward pass for gfx950 (CDNA4, MI355X), f16 / bf16.
//
// Gradients of O = softmax(S) V with S = scale Q K^T + mask, given dO:
//   P  = exp(S - LSE)             (recomputed from Q, K and the forward's
//                                  per-row log-sum-exp; never stored)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O)
//   dQ = scale dS K,  dK = scale dS^T Q.
// The backward recomputes the attention matrix on-chip in two passes instead
// of storing it (article "Mastering FlashAttention: The Algebraic
// Foundation", technical deep dive). Here the two passes are:
//   1. bwd_dq, query-major: one workgroup per (batch*head, 256 query rows)
//      streams the K/V tiles like the forward and accumulates dQ in
//      registers. It also computes D for its rows (from dO and O) and
//      -LSE*log2(e), and leaves both in the caller's workspace.
//   2. bwd_dkdv2, key-major: one workgroup per (batch*head, 128 keys)
//      streams the Q / dO tiles (with D and LSE) and accumulates dK and dV;
//      the two products of each key run on two waves that share a SIMD
//      (bwd_dkdv, one wave per key block, is the single-wave form).
// Each pass owns its outputs, so no atomics and no second reduction: the
// result is deterministic. The price is that S and dP are computed in both
// passes (7 matrix products instead of the 5 the gradient needs).
//
// Register layouts follow the forward kernel: the 32x32 MFMA puts the index
// a wave owns (queries in pass 1, keys in pass 2) on the lanes, so the
// per-row or per-key statistics are lane-local; the contraction index of the
// second product in each pass is permuted (perm32) so that accumulator
// registers, packed to 16 bits, are directly the B operand of that product.
//
// LDS. Tiles are copied straight into LDS by the buffer unit (buffer_load
// ... lds) through an NS-stage ring. Each tile is read both row-wise (16-byte
// operand reads, 16 rows per 16 lanes) and transposed (ds_read_b64_tr_b16,
// 4 consecutive rows x 4 chunks per 32 lanes), so its 16-byte chunks are
// XOR-swizzled with a function of the row that keeps both access patterns
// on distinct banks (swz2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

// Ring stages and tile rows (keys in pass 1, queries in pass 2) of the
// backward kernels.
#ifndef FA_BWD_STAGES
#define FA_BWD_STAGES 4
#endif
#ifndef FA_BWD_TILE
#define FA_BWD_TILE 64
#endif
#ifndef FA_BWD_SPLIT
#define FA_BWD_SPLIT 1
#endif
#ifndef FA_BWD_LAG
#define FA_BWD_LAG 1
#endif
#ifndef FA_BWD_SDP_AHEAD
#define FA_BWD_SDP_AHEAD 4
#endif
static_assert(FA_BWD_SDP_AHEAD >= 1, "operand read-ahead");
constexpr int kBwdStages = FA_BWD_STAGES;
static_assert(kBwdStages >= 2 && kBwdStages <= 4, "stages");

// Chunk swizzle for rows of D 16-bit elements: bijective on the 16 rows of
// one row-wise read, and distinct in its upper bits (D = 128: bits 2-3 over
// the 16 chunks of a 256-byte row; D = 64: bit 2 within a row parity) for
// the 4 consecutive rows of one transposing read.
template <int D>
__device__ inline int swz2(int row) {
  if constexpr (D == 128)
    return 4 * (row & 3) + ((row >> 2) & 3);
  else
    return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Sum of the products of 8 16-bit values (fp32). The words are copied out of
// the vectors before the bit cast: a bit cast applied to a vector element
// expression read element 0 whatever the index.
template <Elt E>
__device__ inline float dot8(u32x4_t a, u32x4_t b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ai = a[i], bi = b[i];
    if constexpr (E == Elt::F16) {
      const f16x2_t x = __builtin_bit_cast(f16x2_t, ai);
      const f16x2_t y = __builtin_bit_cast(f16x2_t, bi);
      s = __builtin_fmaf((float)x[0], (float)y[0], s);
      s = __builtin_fmaf((float)x[1], (float)y[1], s);
    } else {
      s = __builtin_fmaf(__uint_as_float(ai << 16), __uint_as_float(bi << 16), s);
      s = __builtin_fmaf(__uint_as_float(ai & 0xffff0000u), __uint_as_float(bi & 0xffff0000u), s);
    }
  }
  return s;
}

// One (batch, head), or one sequence of a ragged batch: row 0 of each
// [rows, d] array, the byte row stride they share, the row count and row 0
// of the per-row statistics (LSE, D, -LSE log2 e). Ragged offsets are clamped
// to [0, total] and lengths to n, so no cu_seqlens content sends an access
// outside the arrays.
struct BwdView {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* o;
  const uint8_t* g;
  uint8_t* dq;
  uint8_t* dk;
  uint8_t* dv;
  uint32_t rs;
  int n;
  const float* lse;
  float* delta;
  float* nlse2;
};
__device__ inline BwdView bwd_view(const BwdArgs& a, int bh) {
  int n = a.n;
  int64_t row0;   // element offset of row 0
  size_t st0;     // index of row 0's statistics
  if (a.cu_seqlens) {
    const int b = bh / a.heads, h = bh - b * a.heads;
    const int s0 = min(max(a.cu_seqlens[b], 0), a.total);
    const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.total);
    n = min(s1 - s0, a.n);
    row0 = ((int64_t)s0 * a.heads + h) * a.d;
    st0 = (size_t)h * a.total + s0;
  } else {
    row0 = (int64_t)bh * a.n * a.d;
    st0 = (size_t)bh * a.n;
  }
  BwdView v;
  v.q = (const uint8_t*)a.q + row0 * 2;
  v.k = (const uint8_t*)a.k + row0 * 2;
  v.v = (const uint8_t*)a.v + row0 * 2;
  v.o = (const uint8_t*)a.o + row0 * 2;
  v.g = (const uint8_t*)a.dout + row0 * 2;
  v.dq = (uint8_t*)a.dq + row0 * 2;
  v.dk = (uint8_t*)a.dk + row0 * 2;
  v.dv = (uint8_t*)a.dv + row0 * 2;
  v.rs = (uint32_t)(a.rs * 2);
  v.n = n;
  v.lse = a.lse + st0;
  v.delta = a.delta + st0;
  v.nlse2 = a.nlse2 + st0;
  return v;
}

// 32 columns (one per lane, rows 4 per register group) of a d-major
// accumulator -> 8-byte stores of 4 consecutive d values: acc[db][4g + r] is
// d-column db*32 + 8g + 4*hl + r of this lane's row.
template <Elt E, int NDB>
__device__ inline void store_rows(uint16_t* row_ptr, int hl, const f32x16_t (&acc)[NDB], float mult) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * hl;
      const uint32_t x0 = pack2<E>(acc[db][4 * g] * mult, acc[db][4 * g + 1] * mult);
      const uint32_t x1 = pack2<E>(acc[db][4 * g + 2] * mult, acc[db][4 * g + 3] * mult);
      *(u32x2_t*)(row_ptr + d) = u32x2_t{x0, x1};
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 1: dQ. Eight waves, 32 query rows each; 64-key tiles of K and V.
// Per tile and 32-key block: S^T = K Q^T and dP^T = V dO^T (row-wise reads
// of K and V), P = exp2(c S - LSE log2 e), dS = P (dP - D), then
// dQ^T += K^T dS^T with K^T from transposing reads of the same K tile.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBq = 32 * kDqWaves;

template <int BYTES>
struct PairSlot {
  __attribute__((aligned(1024))) uint8_t a[BYTES];
  __attribute__((aligned(1024))) uint8_t b[BYTES];
};

template <Elt IN, int D, bool CAUSAL>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq(BwdArgs a) {
  constexpr int ROWB = D * 2, BK = FA_BWD_TILE, TILE_B = BK * ROWB;
  constexpr int LPW = TILE_B / 1024 / kDqWaves;  // 1 KiB loads per wave per tile (K and V each)
  constexpr int NS = kBwdStages;
  constexpr int KB = BK / 32, NKS = D / 16, NDB = D / 32;
  static_assert(LPW >= 1, "tile too small for the wave count");

  __shared__ PairSlot<TILE_B> ring0, ring1, ring2, ring3;  // a: K, b: V

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int tiles = (a.n + kDqBq - 1) / kDqBq;
  // Paired query tiles, as in the forward: tile T-1-p, then tile p of the
  // same head, with the K/V ring running on between them. The launcher pairs
  // only when every first tile's key-tile count is a multiple of NS, so the
  // second tile starts on slot 0.
  const bool pair = a.pair;
  const TileId tl = pair ? tile_of_block(blockIdx.x, a.bh, tiles / 2, false, kDqBq, tiles)
                         : tile_of_block(blockIdx.x, a.bh, tiles, CAUSAL, kDqBq);
  const BwdView hv = bwd_view(a, tl.bh);
  const int n = hv.n;
  int q0 = (pair ? tiles - 1 - tl.t : tl.t) * kDqBq;
  if (q0 >= n) return;  // a tile past a short sequence (uniform)
  int qw0 = q0 + 32 * w;
  int qrow = qw0 + lr;
  const uint32_t span = span_bytes(n, hv.rs, ROWB);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(hv.q, span);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(hv.k, span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(hv.v, span);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(hv.o, span);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(hv.g, span);

  // ring positions 0 .. nt-1: key tiles 0 .. nt0-1, then (paired) those of the second query tile
  const int nt0 = ((CAUSAL ? min(q0 + kDqBq, n) : n) + BK - 1) / BK;
  const int nt = pair ? nt0 + ((CAUSAL ? min(tl.t * kDqBq + kDqBq, n) : n) + BK - 1) / BK : nt0;

  uint32_t off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (w * LPW + i) * 1024 + lane * 16;
    const int row = byte / ROWB, p = (byte % ROWB) / 16;
    off[i] = (uint32_t)row * hv.rs + (uint32_t)((p ^ swz2<D>(row)) * 16);
  }
  auto issue = [&](PairSlot<TILE_B>& slot, int J) __attribute__((always_inline)) {
    const int t = pair && J >= nt0 ? J - nt0 : J;
    const uint32_t base = J < nt ? (uint32_t)(t * BK) * hv.rs : 0x80000000u;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(rk, slot.a + (w * LPW + i) * 1024, base + off[i]);
      lds_dma16(rv, slot.b + (w * LPW + i) * 1024, base + off[i]);
    }
  };

  // Q and dO fragments (B operands), O only for D = rowsum(dO * O); D and
  // -LSE log2(e) of this lane's row also go to the workspace.
  u32x4_t qf[NKS], gf[NKS];
  float dsum, nl2;
  auto start_rows = [&]() __attribute__((always_inline)) {
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t o_ = (uint32_t)qrow * hv.rs + (ks * 16 + hl * 8) * 2;
      qf[ks] = bload16(rq, o_);
      gf[ks] = bload16(rg, o_);
      dpart += dot8<IN>(gf[ks], bload16(ro, o_));
    }
    dsum = pair_sum(dpart);
    nl2 = qrow < n ? -hv.lse[qrow] * kLog2e : 0.f;
    if (hl == 0 && qrow < n) {
      hv.delta[qrow] = dsum;
      hv.nlse2[qrow] = nl2;
    }
  };
  start_rows();
  wait_vmcnt<0>();

  const int krow = perm32(lr);
  const int sw_k = swz2<D>(krow);
  const int grp = lane >> 4, li = lane & 15;
  const int trow = 8 * hl + (li >> 2);  // + kb*32 + 16*s2 (+4 for the second read)
  const int sw_lo = swz2<D>(trow), sw_hi = swz2<D>(trow + 4);
  const int tcol = 16 * (grp & 1) + 4 * (li & 3);  // + db*32

  const float c = a.c;
  // a masked score must give c * s = -inf whatever the sign of c
  const float s_masked = c > 0.f ? -INFINITY : INFINITY;
  f32x16_t dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16_t{};
  auto live = [&](int j) __attribute__((always_inline)) { return qw0 < n && !(CAUSAL && j * BK > qw0 + 31); };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    return (j * BK + BK > n) || (CAUSAL && j * BK + BK - 1 > qw0);
  };

  auto compute = [&](const PairSlot<TILE_B>& slot, int j) __attribute__((always_inline)) {
    const bool mask = needs_mask(j);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      const int row = kb * 32 + krow;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int at = row * ROWB + (((2 * ks + hl) ^ sw_k) * 16);
        s = mfma16<IN>(*(const u32x4_t*)(slot.a + at), qf[ks], s);
        dp = mfma16<IN>(*(const u32x4_t*)(slot.b + at), gf[ks], dp);
      }
      if (mask) {
        // register i holds key j*BK + kb*32 + 8*hl + off, off = 16*(i >> 3) +
        // (i & 7): visible (key < n and, causal, key <= qrow) iff off <= lim
        const int lim = (CAUSAL ? min(n - 1, qrow) : n - 1) - (j * BK + kb * 32 + 8 * hl);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 16 * (i >> 3) + (i & 7) <= lim ? s[i] : s_masked;
      }
      u32x4_t dsb[2];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[i], c, nl2));
        const float p1 = fast_exp2(__builtin_fmaf(s[i + 1], c, nl2));
        dsb[i >> 3][(i & 7) >> 1] = pack2<IN>(p0 * (dp[i] - dsum), p1 * (dp[i + 1] - dsum));
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int r = kb * 32 + 16 * s2 + trow;
          const int col = db * 32 + tcol;
          const int half = (col & 4) << 1;
          const u32x2_t lo = lds_read_tr16(slot.a + r * ROWB + (((col >> 3) ^ sw_lo) * 16) + half);
          const u32x2_t hi = lds_read_tr16(slot.a + (r + 4) * ROWB + (((col >> 3) ^ sw_hi) * 16) + half);
          dq[db] = mfma16<IN>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, dsb[s2], dq[db]);
        }
      }
    }
  };

  auto slot_ref = [&](auto S) __attribute__((always_inline)) -> PairSlot<TILE_B>& {
    if constexpr (decltype(S)::value == 0) return ring0;
    else if constexpr (decltype(S)::value == 1) return ring1;
    else if constexpr (decltype(S)::value == 2) return ring2;
    else return ring3;
  };
  auto step = [&](auto S, int J, int base) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, (decltype(S)::value + NS - 1) % NS>;
    wait_vmcnt<(NS - 2) * 2 * LPW>();
    __syncthreads();
    issue(slot_ref(SN{}), J + NS - 1);
    if (live(J - base)) compute(slot_ref(S), J - base);
  };
  // positions J0 .. J1-1 (J0 a multiple of NS: slot J mod NS)
  auto run = [&](int J0, int J1, int base) __attribute__((always_inline)) {
    for (int J = J0; J < J1; J += NS) {
      step(std::integral_constant<int, 0>{}, J, base);
      if (J + 1 < J1) step(std::integral_constant<int, 1>{}, J + 1, base);
      if constexpr (NS > 2) if (J + 2 < J1) step(std::integral_constant<int, 2>{}, J + 2, base);
      if constexpr (NS > 3) if (J + 3 < J1) step(std::integral_constant<int, 3>{}, J + 3, base);
    }
  };

  {
    PairSlot<TILE_B>* slots[4] = {&ring0, &ring1, &ring2, &ring3};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4_t* p = (u32x4_t*)slots[s];
      for (int i = tid; i < (int)(sizeof(PairSlot<TILE_B>) / 16); i += kDqThreads) p[i] = u32x4_t{0, 0, 0, 0};
    }
  }
  __syncthreads();

  issue(ring0, 0);
  if constexpr (NS > 2) issue(ring1, 1);
  if constexpr (NS > 3) issue(ring2, 2);
  run(0, nt0, 0);
  if (pair) {
    if (qrow < n) store_rows<IN, NDB>((uint16_t*)hv.dq + (size_t)qrow * (hv.rs / 2), hl, dq, a.scale);
    q0 = tl.t * kDqBq;
    qw0 = q0 + 32 * w;
    qrow = qw0 + lr;
    start_rows();
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16_t{};
    run(nt0, nt, nt0);
  }
  wait_vmcnt<0>();

  if (qrow < n) store_rows<IN, NDB>((uint16_t*)hv.dq + (size_t)qrow * (hv.rs / 2), hl, dq, a.scale);
}

// ---------------------------------------------------------------------------
// Pass 2: dK and dV. Four waves (one per SIMD, so each has the full register
// file), 32 keys each; 64-query tiles of Q and dO plus their D and
// -LSE*log2(e). Per tile and 32-query block: S = Q K^T and dP = dO V^T
// (row-wise reads of Q and dO; K and V of the wave's keys are B operands held
// in registers), P and dS as in pass 1, then dV^T += dO^T P and
// dK^T += Q^T dS with dO^T and Q^T from transposing reads.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvBk = 32 * kKvWaves;  // keys per workgroup
constexpr int kKvBq = FA_BWD_TILE;    // queries per tile

template <int BYTES>
struct QSlot {
  __attribute__((aligned(1024))) uint8_t q[BYTES];
  __attribute__((aligned(1024))) uint8_t g[BYTES];
  // [0, 256): -LSE*log2(e) of the tile's 64 rows; [256, 512): D. Each copy
  // writes 1 KiB, the rest of each half is padding.
  __attribute__((aligned(1024))) float st[512];
};

// The ring of the two-wave dK/dV kernel as three arrays of four slots.
template <int BYTES>
struct KvRing {
  __attribute__((aligned(1024))) uint8_t q[4][BYTES];
  __attribute__((aligned(1024))) uint8_t g[4][BYTES];
  __attribute__((aligned(1024))) float st[4][512];
};
struct QView {
  uint8_t* q;
  uint8_t* g;
  float* st;
  int off;  // the slot's byte offset within the q (and the g) array
};

template <Elt IN, int D, bool CAUSAL>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv(BwdArgs a) {
  constexpr int ROWB = D * 2, TILE_B = kKvBq * ROWB;
  constexpr int LPW = TILE_B / 1024 / kKvWaves;
  constexpr int NS = kBwdStages;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int LOADS = 2 * LPW + 2;  // per wave per tile
  static_assert(LPW >= 1, "tile too small for the wave count");

  __shared__ QSlot<TILE_B> ring0, ring1, ring2, ring3;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int ktiles = (a.n + kKvBk - 1) / kKvBk;
  // ascending key tiles: under a causal mask the first ones see the most queries
  const TileId tl = tile_of_block(blockIdx.x, a.bh, ktiles, false, kKvBk);
  const BwdView hv = bwd_view(a, tl.bh);
  const int n = hv.n;
  const int k0 = tl.t * kKvBk;
  if (k0 >= n) return;  // a tile past a short sequence (uniform)
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + lr;
  const uint32_t span = span_bytes(n, hv.rs, ROWB);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(hv.q, span);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(hv.k, span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(hv.v, span);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(hv.g, span);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(hv.nlse2, (uint32_t)n * 4);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(hv.delta, (uint32_t)n * 4);

  const int i_lo = CAUSAL ? k0 / kKvBq : 0;  // query tiles i_lo .. nt-1
  const int nt = (n + kKvBq - 1) / kKvBq;

  uint32_t off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (w * LPW + i) * 1024 + lane * 16;
    const int row = byte / ROWB, p = (byte % ROWB) / 16;
    off[i] = (uint32_t)row * hv.rs + (uint32_t)((p ^ swz2<D>(row)) * 16);
  }
  // Every wave copies the statistics too (the same bytes), so that all waves
  // issue the same number of loads per tile.
  auto issue = [&](QSlot<TILE_B>& slot, int t) __attribute__((always_inline)) {
    const bool in = t < nt;
    const uint32_t base = in ? (uint32_t)(t * kKvBq) * hv.rs : 0x80000000u;
    const uint32_t sbase = in ? (uint32_t)t * (kKvBq * 4) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(rq, slot.q + (w * LPW + i) * 1024, base + off[i]);
      lds_dma16(rg, slot.g + (w * LPW + i) * 1024, base + off[i]);
    }
    lds_dma16(rl, (uint8_t*)slot.st, sbase + lane * 16);
    lds_dma16(rd, (uint8_t*)(slot.st + 256), sbase + lane * 16);
  };

  // K and V of this lane's key as B operands (d-columns ks*16 + hl*8 .. +8).
  u32x4_t kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint32_t o_ = (uint32_t)key * hv.rs + (ks * 16 + hl * 8) * 2;
    kf[ks] = bload16(rk, o_);
    vf[ks] = bload16(rv, o_);
  }
  wait_vmcnt<0>();

  const int qr = perm32(lr);
  const int sw_r = swz2<D>(qr);
  const int grp = lane >> 4, li = lane & 15;
  const int trow = 8 * hl + (li >> 2);
  const int sw_lo = swz2<D>(trow), sw_hi = swz2<D>(trow + 4);
  const int tcol = 16 * (grp & 1) + 4 * (li & 3);

  const float c = a.c;
  const float s_masked = c > 0.f ? -INFINITY : INFINITY;  // c * s_masked = -inf
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x16_t{};
  const bool wave_live = kw0 < n;
  auto live = [&](int i) __attribute__((always_inline)) {
    return wave_live && !(CAUSAL && i * kKvBq + kKvBq - 1 < kw0);
  };
  auto needs_mask = [&](int i) __attribute__((always_inline)) {
    return (kw0 + 31 >= n) || (CAUSAL && i * kKvBq < kw0 + 31);
  };

  // S = Q K^T and dP = dO V^T of the 32-query block qb
  // The row-wise operand reads run FA_BWD_SDP_AHEAD MFMAs ahead in a pinned
  // order (operand i is Q (even i) or dO (odd i) at k-step i / 2): the wave
  // is alone on its SIMD, so nothing else hides an LDS read that an MFMA
  // waits on.
  auto sdp = [&](const QSlot<TILE_B>& slot, int qb, f32x16_t& s, f32x16_t& dp) __attribute__((always_inline)) {
    s = f32x16_t{};
    dp = f32x16_t{};
    const int row = qb * 32 + qr;
    constexpr int NOP = 2 * NKS, PA = FA_BWD_SDP_AHEAD < NOP ? FA_BWD_SDP_AHEAD : NOP;
    auto rd = [&](int i) __attribute__((always_inline)) {
      const int at = row * ROWB + (((2 * (i >> 1) + hl) ^ sw_r) * 16);
      return *(const u32x4_t*)(((i & 1) ? slot.g : slot.q) + at);
    };
    u32x4_t buf[PA];
#pragma unroll
    for (int i = 0; i < PA; ++i) buf[i] = rd(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      if (i & 1) dp = mfma16<IN>(buf[i % PA], vf[i >> 1], dp);
      else s = mfma16<IN>(buf[i % PA], kf[i >> 1], s);
      if (i + PA < NOP) buf[i % PA] = rd(i + PA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Per tile, the products of block qb + 1 are issued before the softmax of
  // block qb, so that a wave (alone on its SIMD) has them on the matrix pipe
  // while it works on the exponentials.
  auto compute = [&](const QSlot<TILE_B>& slot, int it) __attribute__((always_inline)) {
    constexpr int QB = kKvBq / 32;
    const bool mask = needs_mask(it);
    f32x16_t s[2], dp[2];
    sdp(slot, 0, s[0], dp[0]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (qb + 1 < QB) sdp(slot, qb + 1, s[(qb + 1) & 1], dp[(qb + 1) & 1]);
      f32x16_t& sc = s[qb & 1];
      const f32x16_t& dc = dp[qb & 1];
      // register i holds query qb*32 + 8*hl + i (i < 8) or qb*32 + 16 + 8*hl + i - 8
      float nl[16], dd[16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int q_ = qb * 32 + 16 * h + 8 * hl + 4 * e;
          const u32x4_t x = *(const u32x4_t*)(slot.st + q_);
          const u32x4_t y = *(const u32x4_t*)(slot.st + 256 + q_);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            nl[8 * h + 4 * e + r] = __uint_as_float(x[r]);
            dd[8 * h + 4 * e + r] = __uint_as_float(y[r]);
          }
        }
      }
      if (mask) {
        // register r holds query it*Bq + qb*32 + 8*hl + off, off = 16*(r >> 3)
        // + (r & 7): visible (key < n and, causal, key <= query) iff off >= lo
        const int lo = key < n ? (CAUSAL ? key - (it * kKvBq + qb * 32 + 8 * hl) : INT_MIN) : INT_MAX;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 16 * (r >> 3) + (r & 7) >= lo ? sc[r] : s_masked;
      }
      u32x4_t pb[2], dsb[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(sc[r], c, nl[r]));
        const float p1 = fast_exp2(__builtin_fmaf(sc[r + 1], c, nl[r + 1]));
        pb[r >> 3][(r & 7) >> 1] = pack2<IN>(p0, p1);
        dsb[r >> 3][(r & 7) >> 1] = pack2<IN>(p0 * (dc[r] - dd[r]), p1 * (dc[r + 1] - dd[r + 1]));
      }
      // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int r = qb * 32 + 16 * s2 + trow;
          const int col = db * 32 + tcol;
          const int half = (col & 4) << 1;
          const int at_lo = r * ROWB + (((col >> 3) ^ sw_lo) * 16) + half;
          const int at_hi = (r + 4) * ROWB + (((col >> 3) ^ sw_hi) * 16) + half;
          const u32x2_t glo = lds_read_tr16(slot.g + at_lo);
          const u32x2_t ghi = lds_read_tr16(slot.g + at_hi);
          dv[db] = mfma16<IN>(u32x4_t{glo[0], glo[1], ghi[0], ghi[1]}, pb[s2], dv[db]);
          const u32x2_t qlo = lds_read_tr16(slot.q + at_lo);
          const u32x2_t qhi = lds_read_tr16(slot.q + at_hi);
          dk[db] = mfma16<IN>(u32x4_t{qlo[0], qlo[1], qhi[0], qhi[1]}, dsb[s2], dk[db]);
        }
      }
    }
  };

  auto slot_ref = [&](auto S) __attribute__((always_inline)) -> QSlot<TILE_B>& {
    if constexpr (decltype(S)::value == 0) return ring0;
    else if constexpr (decltype(S)::value == 1) return ring1;
    else if constexpr (decltype(S)::value == 2) return ring2;
    else return ring3;
  };
  auto step = [&](auto S, int i) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, (decltype(S)::value + NS - 1) % NS>;
    wait_vmcnt<(NS - 2) * LOADS>();
    __syncthreads();
    issue(slot_ref(SN{}), i + NS - 1);
    if (live(i)) compute(slot_ref(S), i);
  };

  {
    QSlot<TILE_B>* slots[4] = {&ring0, &ring1, &ring2, &ring3};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4_t* p = (u32x4_t*)slots[s];
      for (int i = tid; i < (int)(sizeof(QSlot<TILE_B>) / 16); i += kKvThreads) p[i] = u32x4_t{0, 0, 0, 0};
    }
  }
  __syncthreads();

  issue(ring0, i_lo);
  if constexpr (NS > 2) issue(ring1, i_lo + 1);
  if constexpr (NS > 3) issue(ring2, i_lo + 2);
  for (int i0 = i_lo; i0 < nt; i0 += NS) {
    step(std::integral_constant<int, 0>{}, i0);
    if (i0 + 1 < nt) step(std::integral_constant<int, 1>{}, i0 + 1);
    if constexpr (NS > 2) if (i0 + 2 < nt) step(std::integral_constant<int, 2>{}, i0 + 2);
    if constexpr (NS > 3) if (i0 + 3 < nt) step(std::integral_constant<int, 3>{}, i0 + 3);
  }
  wait_vmcnt<0>();

  if (key < n) {
    store_rows<IN, NDB>((uint16_t*)hv.dv + (size_t)key * (hv.rs / 2), hl, dv, 1.0f);
    store_rows<IN, NDB>((uint16_t*)hv.dk + (size_t)key * (hv.rs / 2), hl, dk, a.scale);
  }
}

// ---------------------------------------------------------------------------
// Pass 2 with the two products of each key split over two waves, so that two
// waves share every SIMD (the single-wave pass above holds K, V, dK and dV in
// one wave, ~400 registers, alone on its SIMD). Eight waves, 128 keys: waves
// w and w + 4 (one SIMD) own keys 32 (w mod 4) .. + 31 of the workgroup.
//   wave w     (K in registers): S = Q K^T, P = exp2(c S - LSE log2 e), P to
//              LDS, then dV^T += dO^T P;
//   wave w + 4 (V in registers): dP = dO V^T, then, with P from LDS,
//              dS = P (dP - D) and dK^T += Q^T dS.
// Two barriers per tile: the tile has landed; P is in LDS. Each phase puts
// 16 MFMAs of each wave of a SIMD on its matrix pipe, beside the vector work
// of one of them (the exponentials in the first, dS in the second). dS is
// formed from P as rounded to the input type, the P that dV uses too.
// ---------------------------------------------------------------------------
constexpr int kKv2Waves = 8;
constexpr int kKv2Threads = 64 * kKv2Waves;

template <Elt E>
__device__ inline void unpack2(uint32_t x, float& a, float& b) {
  if constexpr (E == Elt::F16) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, x);
    a = (float)h[0];
    b = (float)h[1];
  } else {
    a = __uint_as_float(x << 16);
    b = __uint_as_float(x & 0xffff0000u);
  }
}

template <Elt IN, int D, bool CAUSAL>
__global__ __launch_bounds__(kKv2Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv2(BwdArgs a) {
  constexpr int ROWB = D * 2, TILE_B = kKvBq * ROWB;
  constexpr int LPW = TILE_B / 1024 / kKv2Waves;
  constexpr int NS = kBwdStages;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int QB = kKvBq / 32;
  constexpr int LOADS = 2 * LPW + 2;  // per wave per tile
  static_assert(LPW >= 1, "tile too small for the wave count");
  static_assert(kKvBk == 4 * 32, "four key blocks of 32 per workgroup");

  // Q tiles, dO tiles and their row statistics in three arrays, so that
  // every read of a slot is a lane base register plus an immediate below
  // 64 KiB (with one QSlot per slot the compiler held address registers per
  // slot)
  __shared__ KvRing<TILE_B> kr;
  // P of the current tile: [register half][key block][query block][lane]
  __shared__ u32x4_t pbuf[2][4][QB][64];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kblk = w & 3;
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int ktiles = (a.n + kKvBk - 1) / kKvBk;
  const TileId tl = tile_of_block(blockIdx.x, a.bh, ktiles, false, kKvBk);
  const BwdView hv = bwd_view(a, tl.bh);
  const int n = hv.n;
  const int k0 = tl.t * kKvBk;
  if (k0 >= n) return;  // a tile past a short sequence (uniform)
  const int kw0 = k0 + 32 * kblk;
  const int key = kw0 + lr;
  const uint32_t span = span_bytes(n, hv.rs, ROWB);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(hv.q, span);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(hv.g, span);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(hv.nlse2, (uint32_t)n * 4);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(hv.delta, (uint32_t)n * 4);

  const int i_lo = CAUSAL ? k0 / kKvBq : 0;  // query tiles i_lo .. nt-1
  const int nt = (n + kKvBq - 1) / kKvBq;

  uint32_t off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (w * LPW + i) * 1024 + lane * 16;
    const int row = byte / ROWB, p = (byte % ROWB) / 16;
    off[i] = (uint32_t)row * hv.rs + (uint32_t)((p ^ swz2<D>(row)) * 16);
  }
  auto issue = [&](const QView& slot, int t) __attribute__((always_inline)) {
    const bool in = t < nt;
    const uint32_t base = in ? (uint32_t)(t * kKvBq) * hv.rs : 0x80000000u;
    const uint32_t sbase = in ? (uint32_t)t * (kKvBq * 4) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(rq, slot.q + (w * LPW + i) * 1024, base + off[i]);
      lds_dma16(rg, slot.g + (w * LPW + i) * 1024, base + off[i]);
    }
    lds_dma16(rl, (uint8_t*)slot.st, sbase + lane * 16);
    lds_dma16(rd, (uint8_t*)(slot.st + 256), sbase + lane * 16);
  };

  const int qr = perm32(lr);
  const int sw_r = swz2<D>(qr);
  const int grp = lane >> 4, li = lane & 15;
  const int trow = 8 * hl + (li >> 2);
  const int sw_lo = swz2<D>(trow), sw_hi = swz2<D>(trow + 4);
  const int tcol = 16 * (grp & 1) + 4 * (li & 3);

  const float c = a.c;
  const float s_masked = c > 0.f ? -INFINITY : INFINITY;  // c * s_masked = -inf
  const bool wave_live = kw0 < n;
  auto live = [&](int i) __attribute__((always_inline)) {
    return wave_live && !(CAUSAL && i * kKvBq + kKvBq - 1 < kw0);
  };
  auto needs_mask = [&](int i) __attribute__((always_inline)) {
    return (kw0 + 31 >= n) || (CAUSAL && i * kKvBq < kw0 + 31);
  };

  // acc[qb] = X F^T for the 32-row query blocks qb of X (Q or dO) and this
  // lane's key fragments F (K or V). The MFMAs alternate between the blocks
  // (two independent accumulators); operand i (block i % QB, k-step i / QB)
  // is read FA_BWD_SDP_AHEAD MFMAs ahead in a pinned order.
  // lb[ks]: this lane's read address for k-step ks in slot 0 of the array
  auto prod = [&](const uint32_t (&lb)[NKS], int off, const u32x4_t (&f)[NKS], f32x16_t (&acc)[QB])
                  __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[qb] = f32x16_t{};
    constexpr int NOP = QB * NKS, PA = FA_BWD_SDP_AHEAD < NOP ? FA_BWD_SDP_AHEAD : NOP;
    auto rd_ = [&](int i) __attribute__((always_inline)) {
      const int ks = i / QB;
      return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(lb[ks] + off +
                                                                          (i % QB) * 32 * ROWB);
    };
    u32x4_t buf[PA];
#pragma unroll
    for (int i = 0; i < PA; ++i) buf[i] = rd_(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      acc[i % QB] = mfma16<IN>(buf[i % PA], f[i / QB], acc[i % QB]);
      if (i + PA < NOP) buf[i % PA] = rd_(i + PA);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc[db] += X^T B over the 32 queries of block qb: X^T (dO^T or Q^T) from
  // transposing reads, B (P or dS, 16 queries per half) from registers.
  // tb[db][0 / 1]: this lane's addresses of the two transposing reads of
  // d-block db in slot 0 of the array
  auto prod_t = [&](const uint32_t (&tb)[NDB][2], int off, int qb, const u32x4_t (&b)[2], f32x16_t (&acc)[NDB])
                    __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int rr = off + (qb * 32 + 16 * s2) * ROWB;
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(tb[db][0] + rr)));
        const u32x2_t hi = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(tb[db][1] + rr)));
        acc[db] = mfma16<IN>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, b[s2], acc[db]);
      }
    }
  };

  auto slot_ref = [&](auto S) __attribute__((always_inline)) -> QView {
    constexpr int sv = decltype(S)::value;
    return QView{kr.q[sv], kr.g[sv], kr.st[sv], sv * TILE_B};
  };

  // The two roles run separate copies of the tile loop with the same
  // sequence of barriers, so each keeps only its own registers.
  auto run = [&](auto ROLE) __attribute__((always_inline)) {
    constexpr bool kS = decltype(ROLE)::value;  // the S / P / dV wave
    u32x4_t f[NKS];  // K (kS) or V of this lane's key, d-columns ks*16 + hl*8 .. +8
    {
      const __amdgpu_buffer_rsrc_t rf = make_rsrc(kS ? hv.k : hv.v, span);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f[ks] = bload16(rf, (uint32_t)key * hv.rs + (ks * 16 + hl * 8) * 2);
    }
    wait_vmcnt<0>();
    // lane base addresses: lbx for the row-wise reads (Q for the S waves,
    // dO for the dP waves), tby for the transposing reads (dO, resp. Q); the
    // empty asm hides their origin and the mask tells the compiler the sign
    // bit is clear, so that slot and block offsets fold into immediates
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    uint32_t lbx[NKS], tby[NDB][2];
    {
      const uint32_t xa = (uint32_t)(uintptr_t)(lds_u8*)(kS ? &kr.q[0][0] : &kr.g[0][0]);
      const uint32_t ya = (uint32_t)(uintptr_t)(lds_u8*)(kS ? &kr.g[0][0] : &kr.q[0][0]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        lbx[ks] = xa + qr * ROWB + (((2 * ks + hl) ^ sw_r) * 16);
        asm volatile("" : "+v"(lbx[ks]));
        lbx[ks] &= 0x3ffffu;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + tcol;
        const int half = (col & 4) << 1;
        tby[db][0] = ya + trow * ROWB + (((col >> 3) ^ sw_lo) * 16) + half;
        tby[db][1] = ya + (trow + 4) * ROWB + (((col >> 3) ^ sw_hi) * 16) + half;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          asm volatile("" : "+v"(tby[db][e]));
          tby[db][e] &= 0x3ffffu;
        }
      }
    }
    f32x16_t acc[NDB];  // dV (kS) or dK
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

    {
      u32x4_t* p = (u32x4_t*)&kr;
      for (int i = tid; i < (int)(sizeof(kr) / 16); i += kKv2Threads) p[i] = u32x4_t{0, 0, 0, 0};
    }
    __syncthreads();
    issue(slot_ref(std::integral_constant<int, 0>{}), i_lo);
    if constexpr (NS > 2) issue(slot_ref(std::integral_constant<int, 1>{}), i_lo + 1);
    if constexpr (NS > 3) issue(slot_ref(std::integral_constant<int, 2>{}), i_lo + 2);

    // dS of the previous tile and whether that tile was live (dS waves): its
    // dK product runs in the next step, beside the S waves' exponentials.
    u32x4_t dsp[QB][2];
    bool pl = false;
    auto step = [&](auto S, int it) __attribute__((always_inline)) {
      using SN = std::integral_constant<int, (decltype(S)::value + NS - 1) % NS>;
      wait_vmcnt<(NS - 2) * LOADS>();
      __syncthreads();  // tile it has landed; every wave is past tile it - 1
#if !FA_BWD_LAG
      issue(slot_ref(SN{}), it + NS - 1);
#endif
      const QView slot = slot_ref(S);
      const bool lv = live(it);
      if constexpr (kS) {
        u32x4_t pb[QB][2];
        if (lv) {
          f32x16_t sv[QB];
          prod(lbx, slot.off, f, sv);
          const bool mask = needs_mask(it);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            // register r holds query qb*32 + 16*(r >> 3) + 8*hl + (r & 7)
            float nl[16];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const u32x4_t x = *(const u32x4_t*)(slot.st + qb * 32 + 16 * h + 8 * hl + 4 * e);
#pragma unroll
                for (int r = 0; r < 4; ++r) nl[8 * h + 4 * e + r] = __uint_as_float(x[r]);
              }
            }
            if (mask) {
              // register r holds query it*Bq + qb*32 + 8*hl + off, off =
              // 16*(r >> 3) + (r & 7): visible iff off >= lo
              const int lo = key < n ? (CAUSAL ? key - (it * kKvBq + qb * 32 + 8 * hl) : INT_MIN) : INT_MAX;
#pragma unroll
              for (int r = 0; r < 16; ++r) sv[qb][r] = 16 * (r >> 3) + (r & 7) >= lo ? sv[qb][r] : s_masked;
            }
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float p0 = fast_exp2(__builtin_fmaf(sv[qb][r], c, nl[r]));
              const float p1 = fast_exp2(__builtin_fmaf(sv[qb][r + 1], c, nl[r + 1]));
              pb[qb][r >> 3][(r & 7) >> 1] = pack2<IN>(p0, p1);
            }
            pbuf[0][kblk][qb][lane] = pb[qb][0];
            pbuf[1][kblk][qb][lane] = pb[qb][1];
          }
        }
        __syncthreads();  // P is in LDS
#if FA_BWD_LAG
        issue(slot_ref(SN{}), it + NS - 1);
#endif
        if (lv) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) prod_t(tby, slot.off, qb, pb[qb], acc);  // dV^T += dO^T P
        }
      } else {
        f32x16_t dp[QB];
#if FA_BWD_LAG
        // dK^T += Q^T dS of the previous tile, whose slot is refilled only
        // after the next barrier
        if (pl) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) prod_t(tby, slot_ref(SN{}).off, qb, dsp[qb], acc);
        }
#endif
        if (lv) prod(lbx, slot.off, f, dp);
        __syncthreads();  // P is in LDS
#if FA_BWD_LAG
        issue(slot_ref(SN{}), it + NS - 1);
#endif
        if (lv) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const u32x4_t pw[2] = {pbuf[0][kblk][qb][lane], pbuf[1][kblk][qb][lane]};
            float dd[16];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const u32x4_t y = *(const u32x4_t*)(slot.st + 256 + qb * 32 + 16 * h + 8 * hl + 4 * e);
#pragma unroll
                for (int r = 0; r < 4; ++r) dd[8 * h + 4 * e + r] = __uint_as_float(y[r]);
              }
            }
            u32x4_t dsb[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              float p0, p1;
              unpack2<IN>(pw[r >> 3][(r & 7) >> 1], p0, p1);
              dsb[r >> 3][(r & 7) >> 1] = pack2<IN>(p0 * (dp[qb][r] - dd[r]), p1 * (dp[qb][r + 1] - dd[r + 1]));
            }
#if FA_BWD_LAG
            dsp[qb][0] = dsb[0];
            dsp[qb][1] = dsb[1];
#else
            prod_t(tby, slot.off, qb, dsb, acc);  // dK^T += Q^T dS
#endif
          }
        }
        pl = lv;
      }
    };

    for (int i0 = i_lo; i0 < nt; i0 += NS) {
      step(std::integral_constant<int, 0>{}, i0);
      if (i0 + 1 < nt) step(std::integral_constant<int, 1>{}, i0 + 1);
      if constexpr (NS > 2) if (i0 + 2 < nt) step(std::integral_constant<int, 2>{}, i0 + 2);
      if constexpr (NS > 3) if (i0 + 3 < nt) step(std::integral_constant<int, 3>{}, i0 + 3);
    }
#if FA_BWD_LAG
    if constexpr (!kS) {
      if (pl) {  // the last tile's dK product (no copy targets its slot any more)
        const int ls = (nt - 1 - i_lo) % NS;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) prod_t(tby, ls * TILE_B, qb, dsp[qb], acc);
      }
    }
#endif
    wait_vmcnt<0>();
    if (key < n) {
      if constexpr (kS) store_rows<IN, NDB>((uint16_t*)hv.dv + (size_t)key * (hv.rs / 2), hl, acc, 1.0f);
      else store_rows<IN, NDB>((uint16_t*)hv.dk + (size_t)key * (hv.rs / 2), hl, acc, a.scale);
    }
  };
  if (w < 4) run(std::true_type{});
  else run(std::false_type{});
}

#ifndef FA_BWD_PAIR
#define FA_BWD_PAIR 1
#endif

// Compute units of the current device, read once per device.

template <Elt E, int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int tiles = (a.n + kDqBq - 1) / kDqBq;
  // Paired dQ tiles when every first tile ends on a full ring round (n a
  // multiple of the tile, NS dividing the key tiles per query tile) and, without
  // a mask, while the paired grid still covers every CU.
  BwdArgs b = a;
  b.pair = !a.cu_seqlens && tiles % 2 == 0 && a.n % kDqBq == 0 && (kDqBq / FA_BWD_TILE) % kBwdStages == 0 &&
           FA_BWD_PAIR && (a.causal || (long)a.bh * (tiles / 2) >= device_cus());
  const unsigned g1 = (unsigned)a.bh * (unsigned)(b.pair ? tiles / 2 : tiles);
  const unsigned g2 = (unsigned)a.bh * (unsigned)((a.n + kKvBk - 1) / kKvBk);
  if (a.causal) {
    hipError_t e = launch_kernel(bwd_dq<E, D, true>, dim3(g1), dim3(kDqThreads), s, b);
    if (e != hipSuccess) return e;
    if (FA_BWD_SPLIT) return launch_kernel(bwd_dkdv2<E, D, true>, dim3(g2), dim3(kKv2Threads), s, a);
    return launch_kernel(bwd_dkdv<E, D, true>, dim3(g2), dim3(kKvThreads), s, a);
  } else {
    hipError_t e = launch_kernel(bwd_dq<E, D, false>, dim3(g1), dim3(kDqThreads), s, b);
    if (e != hipSuccess) return e;
    if (FA_BWD_SPLIT) return launch_kernel(bwd_dkdv2<E, D, false>, dim3(g2), dim3(kKv2Threads), s, a);
    return launch_kernel(bwd_dkdv<E, D, false>, dim3(g2), dim3(kKvThreads), s, a);
  }
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  if (a.elt == Elt::F16)
    return a.d == 64 ? launch_bwd_t<Elt::F16, 64>(a, stream) : launch_bwd_t<Elt::F16, 128>(a, stream);
  return a.d == 64 ? launch_bwd_t<Elt::BF16, 64>(a, stream) : launch_bwd_t<Elt::BF16, 128>(a, stream);
}

}  // namespace fa
