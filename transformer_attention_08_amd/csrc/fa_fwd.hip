// Fused attention forward pass for gfx950 (CDNA4, MI355X).
//
// One workgroup owns one tile of query rows of one (batch, head) and streams
// every key/value tile it needs through LDS, merging tiles with the online
// softmax of the slides "Case study: FlashAttention" (slide "Online softmax:
// divide once, at the end"): running max m, running sum l, unnormalised
// output o, rescale alpha = e^(m_old - m_new), and one division by l per row
// at the end. Neither the score tile S nor the probability tile P leaves the
// registers (slide "FlashAttention: the idea": tiling plus fusion, S and P
// never stored).
//
// Register layout (the central design choice). Each wave owns 32 query rows.
// It computes the transposed score tile S^T = K Q^T with the 32x32 MFMA, so
// the MFMA accumulator puts one query on each lane (lane % 32) and 16 keys
// in that lane's registers; the other 16 keys of the 32-key block sit in the
// partner lane (lane ^ 32). Consequences:
//   * the row max and row sum are reductions over a lane's own registers
//     plus one exchange with lane ^ 32;
//   * the accumulator registers, packed to 16 bits, are directly the B
//     operand of the second MFMA O^T = V^T P^T, which again has the query on
//     the lane, so the per-row rescale alpha is a lane-local multiply;
//   * keys are assigned to accumulator rows by a fixed permutation (bits 2
//     and 3 of the row index swapped) so that the 8 keys a lane feeds into
//     one P.V MFMA step are 8 consecutive keys. A sum over keys does not
//     depend on their order, so only the K and V tile reads need to agree.
// V rows keep their memory order in LDS; the A operand of O^T = V^T P^T
// (eight consecutive keys at one d-column per lane) comes from two
// transposing LDS reads (ds_read_b64_tr_b16) of four keys each.
//
// Scale. The exponentials are exp2 with c = scale * log2(e) folded into the
// score ("Mastering FlashAttention: The Algebraic Foundation", key points:
// the qk_scale constant log2(e)/sqrt(D)). The running max is kept in those
// base-2 units; LSE is converted back to natural-log units at the end.
//
// Work decomposition. The grid has one workgroup per (batch*head, query
// tile), or, for the f16 / bf16 kernel with an even tile count, one per pair
// of query tiles T-1-p and p of a head (equal work under a causal mask; the
// K/V ring runs on from one tile into the other). Unpaired causal launches
// visit the longest query tiles first. When the number of (batch, head)
// pairs is a multiple of 8, the workgroups of each head are mapped onto one
// XCD (workgroups are dispatched round-robin over the 8 XCDs), so the K/V
// tiles of a head are re-read from that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBq = 32 * kWaves;  // query rows per workgroup

// Key tiles [lo, hi) of this workgroup: its block of keys (grid dimension y),
// cut at the last query row of the tile under a causal mask.
struct KeyTiles {
  int lo, hi;
};
template <int BK>
__device__ inline KeyTiles key_tiles(const FwdArgs& a, int n, int q_end, bool causal) {
  const int kbeg = blockIdx.y * a.split_keys;
  int kend = min(n, kbeg + a.split_keys);
  if (causal) kend = min(kend, q_end);
  const int lo = kbeg / BK;
  return {lo, kend > kbeg ? (kend + BK - 1) / BK : lo};
}

// The reference max used for the exponentials: a row that has seen no
// visible key yet (possible in a later key block) keeps -inf as its max but
// exponentiates against 0, so its weights are exactly 0 rather than NaN.
__device__ inline float exp_ref(float m) { return m == -INFINITY ? 0.f : m; }

// One (batch, head) -- or one sequence of a ragged batch -- of the layout
// described by FwdArgs: row 0 of q, k, v, o, the row strides in bytes (O's
// in elements), the row count and the LSE of row 0. Ragged-batch offsets are
// clamped to [0, total] and the length to n, so that no access leaves the
// packed arrays whatever cu_seqlens holds.
struct HeadView {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint8_t* o;
  uint32_t qrs, krs, vrs;
  size_t ors;
  int n;
  float* lse;
};
template <int IN_B, int OUT_B>
__device__ inline HeadView head_view(const FwdArgs& a, int bh) {
  const int b = bh / a.heads, h = bh - b * a.heads;
  int64_t start = 0;
  int n = a.n;
  int64_t bq = b, bk = b, bv = b, bo = b;
  if (a.cu_seqlens) {
    const int s0 = min(max(a.cu_seqlens[b], 0), a.total);
    const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.total);
    start = s0;
    n = min(s1 - s0, a.n);
    bq = bk = bv = bo = 0;
  }
  HeadView v;
  v.q = (const uint8_t*)a.q + (bq * a.q_sb + h * a.q_sh + start * a.q_sr) * IN_B;
  v.k = (const uint8_t*)a.k + (bk * a.k_sb + h * a.k_sh + start * a.k_sr) * IN_B;
  v.v = (const uint8_t*)a.v + (bv * a.v_sb + h * a.v_sh + start * a.v_sr) * IN_B;
  v.o = (uint8_t*)a.o + (bo * a.o_sb + h * a.o_sh + start * a.o_sr) * OUT_B;
  v.qrs = (uint32_t)(a.q_sr * IN_B);
  v.krs = (uint32_t)(a.k_sr * IN_B);
  v.vrs = (uint32_t)(a.v_sr * IN_B);
  v.ors = (size_t)a.o_sr;
  v.n = n;
  v.lse = !a.lse ? nullptr : a.cu_seqlens ? a.lse + (size_t)h * a.total + start : a.lse + (size_t)bh * a.n;
  return v;
}

// Split-KV partial result of one row (lane halves hold d-columns as in the
// O^T accumulator): O_g = o / l (times o_mult), LSE_g; zeros and -inf when
// the block held no visible key.
template <int NDB>
__device__ inline void store_partial(const FwdArgs& a, int bh, int qrow, int hl, const f32x16_t (&o)[NDB],
                                     float m2, float lt) {
  constexpr int D = NDB * 32;
  const size_t row = ((size_t)blockIdx.y * a.bh + bh) * a.n + qrow;
  float* po = a.part_o + row * D;
  const float inv = lt > 0.f ? a.o_mult / lt : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * hl;
      u32x4_t x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = __float_as_uint(o[db][4 * g + r] * inv);
      *(u32x4_t*)(po + d) = x;
    }
  }
  if (hl == 0) a.part_lse[row] = lt > 0.f ? (m2 + __log2f(lt)) * kLn2 : -INFINITY;
}

// Two OCP e4m3 codes (bytes 0,1 or, with HI, bytes 2,3 of w) -> two bf16,
// exactly (every e4m3 value is a bf16 value).
template <bool HI>
__device__ inline uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Lazy rescale (all kernels). The reference max m of a row only moves when a
// tile's max exceeds it by more than kLazy (log2 units), so p <= 2^kLazy and
// o and l are rescaled rarely. The result is unchanged: m cancels in o / l,
// and the log-sum-exp is m + log2(l) for whatever m was used.
constexpr float kLazy = 8.0f;

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel for f16 / bf16 inputs. Eight waves (256 query rows)
// per workgroup, 128-key tiles, and an NS-stage ring (2 stages: 128 KiB of
// LDS at d_k 128) of K/V tiles in LDS that the buffer unit fills directly
// (buffer_load ... lds): no staging registers, no VALU work to move tiles,
// and NS - 1 tiles of prefetch to hide memory latency. Loads past the end of
// a head return zeros.
//
// LDS layouts. K rows are stored as they are in memory but with their
// 16-byte chunks XOR-swizzled by row, so that the 16 rows one MFMA operand
// read touches fall in distinct bank groups. V rows are stored the same way
// (another swizzle) and read with the transposing LDS read
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes i / 4, 4 + i / 4, 8 + i / 4
// and 12 + i / 4. When those four lanes address four consecutive key rows at
// one group of four d-columns, every lane receives four consecutive keys at
// its own d-column -- the A operand of O^T = V^T P^T -- without a transpose
// on the write side.
//
// Each ring slot is its own __shared__ array and the key loop is unrolled
// over the slots, so the compiler can tell the slot being filled from the
// slot being read and does not wait for the newest loads.
// ---------------------------------------------------------------------------
#ifndef FA_DIRECT_WAVES
#define FA_DIRECT_WAVES 8
#endif
#ifndef FA_DIRECT_KEYS
#define FA_DIRECT_KEYS 128
#endif
constexpr int kDirectWaves = FA_DIRECT_WAVES;
constexpr int kDirectThreads = 64 * kDirectWaves;
constexpr int kDirectBq = 32 * kDirectWaves;
#ifndef FA_STAGES
#define FA_STAGES 2
#endif
#ifndef FA_PAIR_TILES
#define FA_PAIR_TILES 1
#endif
#ifndef FA_QK_AHEAD
#define FA_QK_AHEAD 6
#endif
#ifndef FA_PV_AHEAD
#define FA_PV_AHEAD 4
#endif
#ifndef FA_PAIR_TILES_NOMASK
#define FA_PAIR_TILES_NOMASK 1
#endif

// S^T = K Q^T for one key tile: KB accumulators of 32 keys, NKS k-steps.
// K is read from its swizzled LDS tile (row kb * 32 + krow, 16-byte chunk
// 2 ks + hl of the row, XOR kswz); Q is the register-held B operand. The
// reads take lane base registers, kbase[ks] = this lane's address of k-step
// ks in slot 0 of the K array, plus the slot's offset and kb * 32 rows as
// immediates. The K operands are read FA_QK_AHEAD MFMAs ahead in a fixed
// order (operand i, i.e. k-step i / KB of key block i % KB, feeds MFMA i, and
// the read of operand i + FA_QK_AHEAD goes out right after MFMA i), so that
// LDS latency hides behind the MFMAs already issued.
template <Elt IN, int KB, int NKS, int ROWB>
__device__ inline void qk_tile(f32x16_t (&s)[KB], const uint32_t (&kbase)[NKS], int off,
                               const u32x4_t (&qf)[NKS]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16_t{};
  auto kread = [&](int i) __attribute__((always_inline)) {
    const int ks = i / KB, kb = i % KB;
    return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(kbase[ks] + off + kb * 32 * ROWB);
  };
  constexpr int NQ = NKS * KB, PA = FA_QK_AHEAD > 0 ? (FA_QK_AHEAD < NQ ? FA_QK_AHEAD : NQ) : 1;
  u32x4_t kf[PA];
#pragma unroll
  for (int i = 0; i < PA; ++i) kf[i] = kread(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    s[i % KB] = mfma16<IN>(kf[i % PA], qf[i / KB], s[i % KB]);
    if (i + PA < NQ) kf[i % PA] = kread(i + PA);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T P^T for one key tile: for each 32-key block kb, 16-key half s2
// and 32-column block db, the V^T operand (eight consecutive keys at one
// d-column per lane) comes from two transposing LDS reads of the swizzled V
// tile, and P^T (packed 16-bit p) is the register-held B operand. The reads
// take lane base registers, vbase[db] = this lane's address of the first
// read of d-block db in slot 0 of the V array, plus the slot's offset and
// the row offsets as immediates. The V^T operands are read FA_PV_AHEAD MFMAs
// ahead in a fixed order, the read of operand i + FA_PV_AHEAD issued right
// after MFMA i, so that the latency of the transposing reads hides behind the
// MFMAs already issued.
template <Elt IN, int KB, int NDB, int ROWB>
__device__ inline void pv_tile(f32x16_t (&o)[NDB], const uint32_t (&vbase)[NDB], int off,
                               const u32x4_t (&pb)[KB][2]) {
  auto vread = [&](int i) __attribute__((always_inline)) -> u32x4_t {
    const int kb = i / (2 * NDB), s2 = (i / NDB) % 2, db = i % NDB;
    const uint32_t a0 = vbase[db] + off + (kb * 32 + 16 * s2) * ROWB;
    const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)a0));
    const u32x2_t hi = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(a0 + 4 * ROWB)));
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };
  constexpr int NPV = KB * 2 * NDB;
  constexpr int PA = FA_PV_AHEAD > 0 ? (FA_PV_AHEAD < NPV ? FA_PV_AHEAD : NPV) : 1;
  u32x4_t vf[PA];
#pragma unroll
  for (int i = 0; i < PA; ++i) vf[i] = vread(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    const int kb = i / (2 * NDB), s2 = (i / NDB) % 2, db = i % NDB;
    o[db] = mfma16<IN>(vf[i % PA], pb[kb][s2], o[db]);
    if (i + PA < NPV) vf[i % PA] = vread(i + PA);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue store of one wave's 32 rows of O through LDS. The O^T
// accumulator holds one query row per lane, so storing it directly writes 32
// rows, 16 bytes each, per store instruction; at the end of a query tile the
// eight waves of every workgroup then queue 4096 such partial-line writes.
// Here each lane first writes its row's packed values into the wave's
// 32-row block of `stage` (16-byte chunks XOR-swizzled by row, conflict-free
// in both directions), then reads the block back as 16-byte chunks of whole
// rows, so that each store instruction writes four complete rows. Rows at or
// past nrows are not stored.
template <Elt IN, int NDB>
__device__ inline void store_o_staged(uint8_t* stage, int lr, int hl, int lane, const f32x16_t (&o)[NDB],
                                      float inv, uint16_t* orow0, size_t ors, int nrows) {
  constexpr int ROWB = NDB * 32 * 2, CPR = ROWB / 16;  // bytes and 16-byte chunks per row
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ch = db * 4 + g;  // the chunk of d-columns db*32 + 8g .. +7; this lane's half is hl
      const uint32_t x0 = pack2<IN>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
      const uint32_t x1 = pack2<IN>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *(u32x2_t*)(stage + lr * ROWB + ((ch ^ (lr % CPR)) * 16) + hl * 8) = u32x2_t{x0, x1};
    }
  }
#pragma unroll
  for (int k = 0; k < 32 * CPR / 64; ++k) {
    const int c = k * 64 + lane, row = c / CPR, ch = c % CPR;
    const u32x4_t x = *(const u32x4_t*)(stage + row * ROWB + ((ch ^ (row % CPR)) * 16));
    if (row < nrows) *(u32x4_t*)(orow0 + (size_t)row * ors + ch * 8) = x;
  }
}

// Direct store of one lane's row of O (8-byte stores of 4 consecutive
// d-columns: o[db][4g + r] is d-column db*32 + 8g + 4*hl + r), for ring
// layouts whose slot cannot hold the staged rows of every wave.
template <Elt IN, int NDB>
__device__ inline void store_o_row(uint16_t* row_ptr, int hl, const f32x16_t (&o)[NDB], float inv) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t x0 = pack2<IN>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
      const uint32_t x1 = pack2<IN>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *(u32x2_t*)(row_ptr + db * 32 + 8 * g + 4 * hl) = u32x2_t{x0, x1};
    }
  }
}

template <int D, int KEYS = FA_DIRECT_KEYS>
struct DirectLayout {
  // keys per tile (64 when a smaller tile would leave a wave without a load)
  static constexpr int BK = KEYS * D * 2 >= 1024 * kDirectWaves ? KEYS : 64;
  static constexpr int ROWB = D * 2;            // bytes per K or V row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int TILE_B = BK * ROWB;      // bytes per K (or V) tile
  static constexpr int LPW = TILE_B / 1024 / kDirectWaves;  // 1 KiB loads per wave per tile
  static_assert(LPW >= 1, "tile too small for the wave count");
  // chunk swizzles (see the comment above)
  __device__ static int kswz(int row) { return CPR == 16 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static int vswz(int row) { return CPR == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

template <int BYTES>
struct LdsSlot {
  __attribute__((aligned(1024))) uint8_t k[BYTES];
  __attribute__((aligned(1024))) uint8_t v[BYTES];
};

// The K/V ring of fwd_direct as two arrays of NSL slots, so that each array
// (64 KiB at most) is reached from one set of lane base registers with the
// slot and block offsets as immediates.
template <int BYTES, int NSL>
struct DirectRing {
  __attribute__((aligned(1024))) uint8_t k[NSL][BYTES];
  __attribute__((aligned(1024))) uint8_t v[NSL][BYTES];
};
struct RingView {
  uint8_t* k;
  uint8_t* v;
  int off;  // the slot's byte offset within each array
};

template <Elt IN, int D, bool CAUSAL>
__global__ __launch_bounds__(kDirectThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_direct(FwdArgs a) {
  using L = DirectLayout<D>;
  constexpr int BK = L::BK, ROWB = L::ROWB, TILE_B = L::TILE_B, LPW = L::LPW;
  constexpr int NS = FA_STAGES;
  constexpr int KB = BK / 32;          // 32-key blocks per tile
  constexpr int NKS = D / 16;          // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;          // 32-column blocks of O

  __shared__ DirectRing<TILE_B, NS> dr;
  static_assert(NS >= 2 && NS <= 4, "stages");

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int tiles = (a.n + kDirectBq - 1) / kDirectBq;
  // Paired causal tiles: the workgroup takes query tile T-1-p, then tile p of
  // the same head -- 2T + 2 key tiles in all, the same for every pair -- and
  // its K/V ring runs on from the first tile's keys into the second's, so
  // the second tile starts with its first keys already in LDS.
  const bool pair = a.pair;
  const TileId tl = pair ? tile_of_block(blockIdx.x, a.bh, tiles / 2, false, kDirectBq, tiles)
                         : tile_of_block(blockIdx.x, a.bh, tiles, CAUSAL, kDirectBq);
  const HeadView hv = head_view<2, 2>(a, tl.bh);
  const int n = hv.n;
  int q0 = (pair ? tiles - 1 - tl.t : tl.t) * kDirectBq;
  if (q0 >= n) return;  // a tile past a short sequence (uniform)
  int qw0 = q0 + 32 * w;
  int qrow = qw0 + lr;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(hv.q, span_bytes(n, hv.qrs, ROWB));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(hv.k, span_bytes(n, hv.krs, ROWB));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(hv.v, span_bytes(n, hv.vrs, ROWB));

  const KeyTiles kt = key_tiles<BK>(a, n, min(q0 + kDirectBq, n), CAUSAL);
  // Ring positions J run over j_lo .. nt-1: the key tiles of the (first) query
  // tile, then, paired, those of the second (key tile J - nt0).
  const int j_lo = kt.lo, nt0 = kt.hi;
  const int nt = pair ? nt0 + key_tiles<BK>(a, n, min(tl.t * kDirectBq + kDirectBq, n), CAUSAL).hi : nt0;

  // Per-lane source offsets of this wave's share of a tile (tile 0).
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (w * LPW + i) * 1024 + lane * 16;
    const int row = byte / ROWB, p = (byte % ROWB) / 16;
    koff[i] = (uint32_t)row * hv.krs + (uint32_t)((p ^ L::kswz(row)) * 16);
    voff[i] = (uint32_t)row * hv.vrs + (uint32_t)((p ^ L::vswz(row)) * 16);
  }
  // Issue the loads of tile t into a slot; tiles past the loop load nothing
  // (an offset past the buffer end returns zeros without a memory access),
  // so every step issues the same number of loads. The copies are issued
  // through inline assembly: the compiler does not track them, and the
  // explicit vmcnt wait plus barrier in each step orders them.
  auto issue = [&](const RingView& slot, int J) __attribute__((always_inline)) {
    const int t = pair && J >= nt0 ? J - nt0 : J;
    const uint32_t kb = J < nt ? (uint32_t)(t * BK) * hv.krs : 0x80000000u;
    const uint32_t vb = J < nt ? (uint32_t)(t * BK) * hv.vrs : 0x80000000u;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(rk, slot.k + (w * LPW + i) * 1024, kb + koff[i]);
      lds_dma16(rv, slot.v + (w * LPW + i) * 1024, vb + voff[i]);
    }
  };

  // Q fragments (B operand of S^T = K Q^T). They land while the ring is
  // zeroed; loads complete in issue order, so the first step's wait for its
  // tile covers them too.
  u32x4_t qf[NKS];
  auto load_q = [&](int row) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = bload16(rq, (uint32_t)row * hv.qrs + (ks * 16 + hl * 8) * 2);
    // a negative scale: q -> -q (the sign bits; uniform branch, so the loads
    // are waited for here only in that case)
    if (a.qneg) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] ^= 0x80008000u;
    }
  };
  load_q(qrow);

  // Per-lane LDS read offsets.
  const int krow = perm32(lr);
  const int kswz = L::kswz(krow);
  const int grp = lane >> 4, li = lane & 15;
  const int vrow0 = 8 * hl + (li >> 2);                 // + kb*32 + 16*s2 + 4*r
  const int vswz = L::vswz(vrow0);
  const int vcol = 16 * (grp & 1) + 4 * (li & 3);       // + db*32 (d-column of the 8-byte chunk)
  // the read addresses of slot 0 (K: per k-step; V: per d-block), hidden
  // from the compiler behind an empty asm, the mask telling it the sign bit
  // is clear, so that slot and block offsets fold into immediates
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  uint32_t kbase[NKS], vbase[NDB];
  {
    const uint32_t ka = (uint32_t)(uintptr_t)(lds_u8*)&dr.k[0][0];
    const uint32_t va = (uint32_t)(uintptr_t)(lds_u8*)&dr.v[0][0];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kbase[ks] = ka + krow * ROWB + (((2 * ks + hl) ^ kswz) * 16);
      asm volatile("" : "+v"(kbase[ks]));
      kbase[ks] &= 0x3ffffu;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = db * 32 + vcol;
      vbase[db] = va + vrow0 * ROWB + (((col >> 3) ^ vswz) * 16) + ((col & 4) << 1);
      asm volatile("" : "+v"(vbase[db]));
      vbase[db] &= 0x3ffffu;
    }
  }

  const float c = a.c;
  float m2 = -INFINITY, lp = 0.f;
  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
  auto live = [&](int j) __attribute__((always_inline)) { return qw0 < n && !(CAUSAL && j * BK > qw0 + 31); };
  auto needs_mask = [&](int j) __attribute__((always_inline)) { return (j * BK + BK > n) || (CAUSAL && j * BK + BK - 1 > qw0); };

  auto compute = [&](const RingView& slot, int j, auto&& mid) __attribute__((always_inline)) {
    // S^T = K Q^T
    f32x16_t s[KB];
    qk_tile<IN, KB, NKS, ROWB>(s, kbase, slot.off, qf);
    if (needs_mask(j)) {
      // register i of key block kb holds key j*BK + 8*hl + off with
      // off = kb*32 + 16*(i >> 3) + (i & 7), a constant: the key is visible
      // (key < n and, causal, key <= qrow) iff off <= lim
      const int kofs = j * BK + 8 * hl;
      const int lim = (CAUSAL ? min(n - 1, qrow) : n - 1) - kofs;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 16 * (i >> 3) + (i & 7);
          s[kb][i] = off <= lim ? s[kb][i] : -INFINITY;
        }
      }
    }
    // online softmax with the lazy rescale
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int kb = 1; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float mc = mx * c;
    const bool up = mc > m2 + kLazy;
    const float m_use = up ? mc : m2;
    const float alpha = fast_exp2(m2 - exp_ref(m_use));
    const float nm = -exp_ref(m_use);
    // l sums the fp32 p: a sum of 16-bit rounded p would carry their 2^-9
    // relative rounding into l and so into the log-sum-exp
    float ls = 0.f;
    u32x4_t pb[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][i], c, nm));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][i + 1], c, nm));
        ls += p0 + p1;
        pb[kb][i >> 3][(i & 7) >> 1] = pack2<IN>(p0, p1);
      }
    }
    lp = __builtin_fmaf(alpha, lp, ls);
    m2 = m_use;
    if (__any(up)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    // the next tile's copies go out here, between the softmax and P.V (see step)
    mid();
    // O^T += V^T P^T; consecutive MFMAs go to different accumulators
    pv_tile<IN, KB, NDB, ROWB>(o, vbase, slot.off, pb);
  };

  auto slot_ref = [&](auto S) __attribute__((always_inline)) -> RingView {
    constexpr int sv = decltype(S)::value;
    return RingView{dr.k[sv], dr.v[sv], sv * TILE_B};
  };
  // Epilogue of a query tile: O = o / l once per row; LSE = ln 2 * (m2 + log2 l).
  // O goes out through `stage`, a ring slot no wave reads any more once every
  // wave has passed the barrier here (the copies in flight fill the other
  // slot).
  auto finish = [&](const RingView& slot) __attribute__((always_inline)) {
    const float lt = pair_sum(lp);
    if (a.part_o) {
      if (qrow < n) store_partial<NDB>(a, tl.bh, qrow, hl, o, m2, lt);
    } else {
      const float inv = a.o_mult / lt;
      // the staged rows of all waves must fit in one ring slot (64-key tiles
      // at d_k 128 leave a 32 KiB slot for 64 KiB of rows: store directly)
      if constexpr (2 * TILE_B >= kDirectWaves * 32 * ROWB) {
        __syncthreads();
        // the slot's K tile, then its V tile, as one staging area of
        // 32-row blocks (a tile holds a whole number of blocks)
        const int sb = w * 32 * ROWB;
        uint8_t* stage = sb < TILE_B ? slot.k + sb : slot.v + (sb - TILE_B);
        store_o_staged<IN, NDB>(stage, lr, hl, lane, o, inv,
                                (uint16_t*)hv.o + (size_t)qw0 * hv.ors, hv.ors, n - qw0);
      } else {
        if (qrow < n) store_o_row<IN, NDB>((uint16_t*)hv.o + (size_t)qrow * hv.ors, hl, o, inv);
      }
      if (qrow < n && hl == 0 && hv.lse) hv.lse[qrow] = (m2 + __log2f(lt)) * kLn2;
    }
  };

  // One step: ring position J (key tile J - base) lives in slot S; the slot
  // of J - 1 is refilled with position J + NS - 1 once every wave is past
  // J - 1.
  auto step = [&](auto S, int J, int base) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, (decltype(S)::value + NS - 1) % NS>;
    wait_vmcnt<(NS - 2) * 2 * LPW>();  // this wave's share of position J has landed
    __syncthreads();                   // ... and every other wave's
    // The copies of position J + NS - 1 are issued inside the compute, after
    // the softmax and before P.V: their LDS writes then overlap the P.V
    // phase rather than Q K^T (measured +1.5% over issuing them first).
    auto refill = [&]() __attribute__((always_inline)) { issue(slot_ref(SN{}), J + NS - 1); };
    if (live(J - base)) compute(slot_ref(S), J - base, refill);
    else refill();
  };
  // Positions J0 .. J1-1 of one query tile; slots are (J - j_lo) mod NS, so a
  // second tile (paired, NS = 2) may start on slot 1.
  auto run = [&](int J0, int J1, int base) __attribute__((always_inline)) {
    int J = J0;
    if constexpr (NS == 2) {
      if (((J - j_lo) & 1) && J < J1) {
        step(std::integral_constant<int, 1>{}, J, base);
        ++J;
      }
    }
    for (; J < J1; J += NS) {
      step(std::integral_constant<int, 0>{}, J, base);
      if (J + 1 < J1) step(std::integral_constant<int, 1>{}, J + 1, base);
      if constexpr (NS > 2) if (J + 2 < J1) step(std::integral_constant<int, 2>{}, J + 2, base);
      if constexpr (NS > 3) if (J + 3 < J1) step(std::integral_constant<int, 3>{}, J + 3, base);
    }
  };

  // Zero the ring once, so that rows a load leaves unwritten can never hold
  // NaN patterns (P is 0 there, but 0 * NaN is NaN).
  {
    u32x4_t* p = (u32x4_t*)&dr;
    for (int i = tid; i < (int)(sizeof(dr) / 16); i += kDirectThreads) p[i] = u32x4_t{0, 0, 0, 0};
  }
  __syncthreads();

  // prologue: tiles j_lo .. j_lo + NS - 2
  issue(slot_ref(std::integral_constant<int, 0>{}), j_lo);
  if constexpr (NS > 2) issue(slot_ref(std::integral_constant<int, 1>{}), j_lo + 1);
  if constexpr (NS > 3) issue(slot_ref(std::integral_constant<int, 2>{}), j_lo + 2);

  run(j_lo, nt0, 0);
  if (pair) {
    // the second query tile: its first keys are already in the ring (the
    // slot of position nt0). Its Q loads go out before the first tile's
    // epilogue (the first tile no longer needs its Q fragments), so that
    // their latency overlaps it; the next step waits for them and the keys.
    // The slot of the first tile's last position is free for O.
    load_q(tl.t * kDirectBq + 32 * w + lr);
    {
      const int fs = (nt0 - 1 - j_lo) & 1;
      finish(RingView{dr.k[fs], dr.v[fs], fs * TILE_B});
    }
    q0 = tl.t * kDirectBq;
    qw0 = q0 + 32 * w;
    qrow = qw0 + lr;
    m2 = -INFINITY;
    lp = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
    run(nt0, nt, nt0);
  }
  wait_vmcnt<0>();  // no load may still be writing LDS (nor may when the workgroup ends)
  finish(slot_ref(std::integral_constant<int, 0>{}));
}

// ---------------------------------------------------------------------------
// e4m3 variant of fwd_direct. The buffer unit copies each K/V tile as e4m3
// bytes into an LDS staging area (half the bytes of a bf16 tile). One step
// before a tile is used, the waves widen it -- exactly, every e4m3 value is a
// bf16 value -- into the swizzled ring layout of fwd_direct, whose compute
// then runs on the bf16 MFMA (the fp8 MFMA accumulates with about 3e-5
// relative error, too much for the LSE bar at scores near 100). Two barriers
// per step: before the widening (the staged tile has landed; the target slot
// is free) and after it (the slot is ready; the staging area is free for the
// next copy). LDS: two bf16 slots plus the staging area, 160 KiB at d_k 128.
// ---------------------------------------------------------------------------
template <int D>
struct Stage8 {
  __attribute__((aligned(1024))) uint8_t k[DirectLayout<D, 128>::BK * D];
  __attribute__((aligned(1024))) uint8_t v[DirectLayout<D, 128>::BK * D];
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDirectThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_direct8(FwdArgs a) {
  using L = DirectLayout<D, 128>;  // e4m3 staging copies need 128-key tiles
  constexpr int BK = L::BK, ROWB = L::ROWB, TILE_B = L::TILE_B;
  constexpr int KB = BK / 32, NKS = D / 16, NDB = D / 32;
  constexpr int STILE = BK * D;                         // bytes per staged e4m3 tile (K or V)
  constexpr int SLPW = STILE / 1024 / kDirectWaves;     // 1 KiB copies per wave per tile
  constexpr int SCPR = D / 16;                          // 16-byte e4m3 chunks per row
  constexpr int CPT = STILE / 16 / kDirectThreads;      // staged chunks per thread
  static_assert(SLPW >= 1 && CPT >= 1, "tile mapping");

  __shared__ DirectRing<TILE_B, 2> dr;
  __shared__ Stage8<D> stage;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int tiles = (a.n + kDirectBq - 1) / kDirectBq;
  const TileId tl = tile_of_block(blockIdx.x, a.bh, tiles, CAUSAL, kDirectBq);
  const HeadView hv = head_view<1, 2>(a, tl.bh);
  const int n = hv.n;
  const int q0 = tl.t * kDirectBq;
  if (q0 >= n) return;  // a tile past a short sequence (uniform)
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + lr;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(hv.q, span_bytes(n, hv.qrs, D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(hv.k, span_bytes(n, hv.krs, D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(hv.v, span_bytes(n, hv.vrs, D));

  const KeyTiles kt = key_tiles<BK>(a, n, min(q0 + kDirectBq, n), CAUSAL);
  const int j_lo = kt.lo, nt = kt.hi;

  // staging copies: plain row-major e4m3 rows
  uint32_t koff[SLPW], voff[SLPW];
#pragma unroll
  for (int i = 0; i < SLPW; ++i) {
    const int byte = (w * SLPW + i) * 1024 + lane * 16;
    const int row = byte / D, c = (byte % D) / 16;
    koff[i] = (uint32_t)row * hv.krs + (uint32_t)(c * 16);
    voff[i] = (uint32_t)row * hv.vrs + (uint32_t)(c * 16);
  }
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t kb = t < nt ? (uint32_t)(t * BK) * hv.krs : 0x80000000u;
    const uint32_t vb = t < nt ? (uint32_t)(t * BK) * hv.vrs : 0x80000000u;
#pragma unroll
    for (int i = 0; i < SLPW; ++i) {
      lds_dma16(rk, stage.k + (w * SLPW + i) * 1024, kb + koff[i]);
      lds_dma16(rv, stage.v + (w * SLPW + i) * 1024, vb + voff[i]);
    }
  };
  // widen the staged tile into a ring slot: 16 e4m3 values -> two 16-byte
  // bf16 chunks at their swizzled places
  auto widen = [&](const RingView& slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * kDirectThreads;
      const int row = ch / SCPR, c = ch % SCPR;
      const u32x4_t xk = *(const u32x4_t*)(stage.k + ch * 16);
      const u32x4_t xv = *(const u32x4_t*)(stage.v + ch * 16);
      const int ks = L::kswz(row), vs = L::vswz(row);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const u32x4_t bk = u32x4_t{e4m3x2_to_bf16x2<false>(xk[2 * e]), e4m3x2_to_bf16x2<true>(xk[2 * e]),
                                   e4m3x2_to_bf16x2<false>(xk[2 * e + 1]), e4m3x2_to_bf16x2<true>(xk[2 * e + 1])};
        const u32x4_t bv = u32x4_t{e4m3x2_to_bf16x2<false>(xv[2 * e]), e4m3x2_to_bf16x2<true>(xv[2 * e]),
                                   e4m3x2_to_bf16x2<false>(xv[2 * e + 1]), e4m3x2_to_bf16x2<true>(xv[2 * e + 1])};
        *(u32x4_t*)(slot.k + row * ROWB + (((2 * c + e) ^ ks) * 16)) = bk;
        *(u32x4_t*)(slot.v + row * ROWB + (((2 * c + e) ^ vs) * 16)) = bv;
      }
    }
  };

  // Q fragments as e4m3; they land during the prologue and are widened once
  // after its first wait
  u32x2_t q8[NKS];
  u32x4_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) q8[ks] = bload8(rq, (uint32_t)qrow * hv.qrs + (ks * 16 + hl * 8));

  const int krow = perm32(lr);
  const int kswz = L::kswz(krow);
  const int grp = lane >> 4, li = lane & 15;
  const int vrow0 = 8 * hl + (li >> 2);
  const int vswz = L::vswz(vrow0);
  const int vcol = 16 * (grp & 1) + 4 * (li & 3);
  // the read addresses of slot 0 (as in fwd_direct)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  uint32_t kbase[NKS], vbase[NDB];
  {
    const uint32_t ka = (uint32_t)(uintptr_t)(lds_u8*)&dr.k[0][0];
    const uint32_t va = (uint32_t)(uintptr_t)(lds_u8*)&dr.v[0][0];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kbase[ks] = ka + krow * ROWB + (((2 * ks + hl) ^ kswz) * 16);
      asm volatile("" : "+v"(kbase[ks]));
      kbase[ks] &= 0x3ffffu;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = db * 32 + vcol;
      vbase[db] = va + vrow0 * ROWB + (((col >> 3) ^ vswz) * 16) + ((col & 4) << 1);
      asm volatile("" : "+v"(vbase[db]));
      vbase[db] &= 0x3ffffu;
    }
  }

  const float c = a.c;
  float m2 = -INFINITY, lp = 0.f;
  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
  const bool wave_live = qw0 < n;
  auto live = [&](int j) __attribute__((always_inline)) { return wave_live && !(CAUSAL && j * BK > qw0 + 31); };
  auto needs_mask = [&](int j) __attribute__((always_inline)) { return (j * BK + BK > n) || (CAUSAL && j * BK + BK - 1 > qw0); };

  // the compute of fwd_direct on the widened tile
  auto compute = [&](const RingView& slot, int j) __attribute__((always_inline)) {
    f32x16_t s[KB];
    qk_tile<Elt::BF16, KB, NKS, ROWB>(s, kbase, slot.off, qf);
    if (needs_mask(j)) {
      // register i of key block kb holds key j*BK + 8*hl + off with
      // off = kb*32 + 16*(i >> 3) + (i & 7), a constant: the key is visible
      // (key < n and, causal, key <= qrow) iff off <= lim
      const int kofs = j * BK + 8 * hl;
      const int lim = (CAUSAL ? min(n - 1, qrow) : n - 1) - kofs;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 16 * (i >> 3) + (i & 7);
          s[kb][i] = off <= lim ? s[kb][i] : -INFINITY;
        }
      }
    }
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int kb = 1; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float mc = mx * c;
    const bool up = mc > m2 + kLazy;
    const float m_use = up ? mc : m2;
    const float alpha = fast_exp2(m2 - exp_ref(m_use));
    const float nm = -exp_ref(m_use);
    float ls = 0.f;
    u32x4_t pb[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][i], c, nm));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][i + 1], c, nm));
        ls += p0 + p1;
        pb[kb][i >> 3][(i & 7) >> 1] = pack2<Elt::BF16>(p0, p1);
      }
    }
    lp = __builtin_fmaf(alpha, lp, ls);
    m2 = m_use;
    if (__any(up)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    pv_tile<Elt::BF16, KB, NDB, ROWB>(o, vbase, slot.off, pb);
  };

  // Step j: tile j is in `cur`; tile j + 1 is staged; tile j + 2 is copied next.
  auto step = [&](const RingView& cur, const RingView& nxt, int j) __attribute__((always_inline)) {
    wait_vmcnt<0>();   // this wave's share of tile j + 1 is staged
    __syncthreads();   // ... every wave's; nobody reads tile j - 1 from nxt any more
    if (j + 1 < nt) widen(nxt);
    __syncthreads();   // nxt holds tile j + 1; the staging area is free
    issue(j + 2);
    if (live(j)) compute(cur, j);
  };

  const RingView r0{dr.k[0], dr.v[0], 0}, r1{dr.k[1], dr.v[1], TILE_B};
  {
    u32x4_t* p = (u32x4_t*)&dr;
    for (int i = tid; i < (int)(sizeof(dr) / 16); i += kDirectThreads) p[i] = u32x4_t{0, 0, 0, 0};
  }
  issue(j_lo);
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = u32x4_t{e4m3x2_to_bf16x2<false>(q8[ks][0]), e4m3x2_to_bf16x2<true>(q8[ks][0]),
                     e4m3x2_to_bf16x2<false>(q8[ks][1]), e4m3x2_to_bf16x2<true>(q8[ks][1])};
    if (a.qneg) qf[ks] ^= 0x80008000u;  // a negative scale: q -> -q
  }
  __syncthreads();
  widen(r0);
  __syncthreads();
  issue(j_lo + 1);
  for (int j0 = j_lo; j0 < nt; j0 += 2) {
    step(r0, r1, j0);
    if (j0 + 1 < nt) step(r1, r0, j0 + 1);
  }
  wait_vmcnt<0>();

  const float lt = pair_sum(lp);
  if (qrow < n && a.part_o) {
    store_partial<NDB>(a, tl.bh, qrow, hl, o, m2, lt);
  } else if (qrow < n) {
    const float inv = a.o_mult / lt;
    uint16_t* Og = (uint16_t*)hv.o + (size_t)qrow * hv.ors;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hl;
        const uint32_t x0 = pack2<Elt::BF16>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        const uint32_t x1 = pack2<Elt::BF16>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *(u32x2_t*)(Og + d) = u32x2_t{x0, x1};
      }
    }
    if (hl == 0 && hv.lse) hv.lse[qrow] = (m2 + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (32x32x2 fp32 MFMA, 32-key tiles). Same structure and register
// layout as above; with one element per operand lane the P.V step reads V
// rows straight from a row-major LDS tile, so no transpose is needed.
// The k index of the Q K^T MFMA maps lane half hl, step ks to column
// hl * D/2 + ks, so both operands are read as contiguous 16-byte runs.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_mfma32(FwdArgs a) {
  constexpr int BK = 32;
  constexpr int KS = D + 4;   // K row stride (floats): 16-byte reads of 16 rows hit distinct banks
  constexpr int VS = D + 8;   // V row stride (floats): rows r and r+4 fall in opposite bank halves
  constexpr int K_FL = BK * KS, V_FL = BK * VS, STAGE = K_FL + V_FL;
  constexpr int CPR = D / 4;                 // 16-byte chunks per row
  constexpr int NLD = BK * CPR / kThreads;   // chunks per thread per tile (2 or 4)
  constexpr int HALF = D / 2;
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
  const int lane = tid & 63, lr = lane & 31, hl = lane >> 5;
  const int tiles = (a.n + kBq - 1) / kBq;
  const TileId tl = tile_of_block(blockIdx.x, a.bh, tiles, CAUSAL, kBq);
  const HeadView hv = head_view<4, 4>(a, tl.bh);
  const int n = hv.n;
  const int q0 = tl.t * kBq;
  if (q0 >= n) return;  // a tile past a short sequence (uniform)
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + lr;
  // row r of q, k, v (16-byte chunks of a row are contiguous)
  auto qrow_ptr = [&](int r) { return (const u32x4_t*)(hv.q + (size_t)r * hv.qrs); };
  auto krow_ptr = [&](int r) { return (const u32x4_t*)(hv.k + (size_t)r * hv.krs); };
  auto vrow_ptr = [&](int r) { return (const u32x4_t*)(hv.v + (size_t)r * hv.vrs); };

  float qf[HALF];
  {
    const bool ok = qrow < n;
    const u32x4_t* qp = qrow_ptr(ok ? qrow : 0) + hl * HALF / 4;
#pragma unroll
    for (int i = 0; i < HALF / 4; ++i) {
      u32x4_t x = qp[i];
#pragma unroll
      for (int e = 0; e < 4; ++e)  // a negative scale: q -> -q
        qf[4 * i + e] = ok ? __uint_as_float(x[e] ^ (a.qneg ? 0x80000000u : 0u)) : 0.f;
    }
  }

  const KeyTiles kt = key_tiles<BK>(a, n, min(q0 + kBq, n), CAUSAL);
  const int j_lo = kt.lo, nt = kt.hi;  // key tiles j_lo .. nt-1

  u32x4_t kreg[NLD], vreg[NLD];
  auto gload = [&](int j) {
    const int key0 = j * BK;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + it * kThreads;
      const int row = idx / CPR, ch = idx % CPR;
      const int key = key0 + row;
      const bool ok = key < n;
      kreg[it] = ok ? krow_ptr(key)[ch] : u32x4_t{0, 0, 0, 0};
      vreg[it] = ok ? vrow_ptr(key)[ch] : u32x4_t{0, 0, 0, 0};
    }
  };
  auto swrite = [&](int buf) {
    float* kl = smem + buf * STAGE;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
      const int idx = tid + it * kThreads;
      const int row = idx / CPR, ch = idx % CPR;
      *(u32x4_t*)(kl + row * KS + ch * 4) = kreg[it];
      *(u32x4_t*)(kl + K_FL + row * VS + ch * 4) = vreg[it];
    }
  };

  float m2 = -INFINITY, lp = 0.f;
  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
  const float c = a.c;
  const bool wave_live = qw0 < n;

  gload(j_lo);
  swrite(0);
  __syncthreads();

  for (int j = j_lo; j < nt; ++j) {
    const int r = j - j_lo;  // double-buffer slots are relative to j_lo
    if (j + 1 < nt) gload(j + 1);
    const int kbase = j * BK;
    const bool skip = !wave_live || (CAUSAL && kbase > qw0 + 31);
    if (!skip) {
      const float* kl = smem + (r & 1) * STAGE;
      const float* vl = kl + K_FL;
      f32x16_t s = f32x16_t{};
      const float* kr = kl + lr * KS + hl * HALF;
#pragma unroll
      for (int i = 0; i < HALF / 4; ++i) {
        const u32x4_t kv = *(const u32x4_t*)(kr + 4 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(kv[e]), qf[4 * i + e], s, 0, 0, 0);
      }
      // accumulator register i of lane half hl holds key 8(i/4) + 4 hl + i%4
      const bool need_mask = (kbase + BK > n) || (CAUSAL && kbase + BK - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 8 * (i >> 2) + 4 * hl + (i & 3);
          const bool ok = key < n && (!CAUSAL || key <= qrow);
          s[i] = ok ? s[i] : -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m2, mx * c);
      const float alpha = fast_exp2(m2 - exp_ref(m_new));
      const float nm = -exp_ref(m_new);
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = fast_exp2(__builtin_fmaf(s[i], c, nm));
        ls += s[i];
      }
      lp = __builtin_fmaf(alpha, lp, ls);
      m2 = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * hl + (i & 3);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[key * VS + db * 32 + lr], s[i], o[db], 0, 0, 0);
        }
      }
    }
    if (j + 1 < nt) swrite((r + 1) & 1);
    __syncthreads();
  }

  const float lt = lp + __shfl_xor(lp, 32);
  if (qrow < n && a.part_o) {
    store_partial<NDB>(a, tl.bh, qrow, hl, o, m2, lt);
  } else if (qrow < n) {
    const float inv = a.o_mult / lt;
    float* Og = (float*)hv.o + (size_t)qrow * hv.ors;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hl;
        u32x4_t x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = __float_as_uint(o[db][4 * g + r] * inv);
        *(u32x4_t*)(Og + d) = x;
      }
    }
    if (hl == 0 && hv.lse) hv.lse[qrow] = (m2 + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fwd_w48: eight waves of 48 query rows (384 per workgroup) on the 16x16x32
// MFMA, d_k 128, f16 / bf16; the kernel for long heads. Every K operand (16
// keys x 32 d-columns) and every V^T operand (16 d-columns x 32 keys) read
// from LDS feeds the MFMAs of the wave's three 16-row query blocks, and every
// key tile copied into LDS serves 384 query rows (fwd_direct: one MFMA per
// operand read, 256 rows per tile), so both the LDS operand reads and the
// L2 -> LDS copies per FLOP are a third lower. 32-key tiles in a 9-slot ring
// (144 KiB), one workgroup barrier per three tiles.
//
// 16x16x32 operand layouts: A, lane l: row l % 16, k-elements 8(l/16)..+7;
// B, lane l: column l % 16, k-elements 8(l/16)..+7; accumulator, lane l:
// rows 4(l/16)..+3 of column l % 16. Per 16-key sub-tile t of a 32-key chunk
// and query block qb, S^T = K Q^T puts query 16 qb + l % 16 on lane l and
// keys kt(t, 4(l/16) + i), i < 4, in its registers, with the sub-tile's rows
// permuted, kt(t, m) = 8 (m >> 2) + 4 t + (m & 3): the 8 keys 8 (l/16) .. + 7
// that lane l feeds into the chunk's P.V MFMA (B operand, 32 keys) are then
// its own registers of sub-tiles 0 and 1. A query's 32 keys lie in lanes l,
// l ^ 16, l ^ 32 and l ^ 48.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#ifndef FA_W48
#define FA_W48 1
#endif
#ifndef FA_W48_STAGES
#define FA_W48_STAGES 9
#endif
#ifndef FA_W48_AHEAD
#define FA_W48_AHEAD 3  // K operands read ahead, one workgroup per tile
#endif
#ifndef FA_W48_PACK_AHEAD
#define FA_W48_PACK_AHEAD 4  // the same, packed causal tiles
#endif
#ifndef FA_W48_PACK_MIN_N
#define FA_W48_PACK_MIN_N 6144
#endif
#ifndef FA_W48_MIN_N
#define FA_W48_MIN_N 16384
#endif
#ifndef FA_W48_GROUP
#define FA_W48_GROUP 3  // key tiles per workgroup barrier (1, 2 or 3; the ring has 3x as many slots)
#endif
#ifndef FA_W48_PRIO
#define FA_W48_PRIO 1
#endif
constexpr int kW48Waves = 8;
constexpr int kW48Threads = 64 * kW48Waves;
constexpr int kW48Rows = 48;
constexpr int kW48Bq = kW48Rows * kW48Waves;
#ifndef FA_W48_KEYS
#define FA_W48_KEYS 32
#endif
constexpr int kW48Bk = FA_W48_KEYS;  // keys per tile: 32 or 64
#ifndef FA_W48_PACK
#define FA_W48_PACK 1
#endif
// Query tiles per head that a packed causal launch can take (n <= 97920).
constexpr int kW48PlanTiles = 255;
struct W48Plan {
  int bins;                            // groups of tiles per head
  int heads_seq;                       // heads each workgroup takes one after another
  uint8_t bin_of_tile[kW48PlanTiles];  // the group (0 .. bins-1) of each query tile
};
struct W48Args {
  FwdArgs a;
  W48Plan plan;
};

template <Elt E>
__device__ inline f32x4_t mfma16x16(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (E == Elt::F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Chunk swizzles of the K and V tiles (16-byte chunks of 256-byte rows).
// K: bijective on the 16 rows of one A-operand read (rows 8m' + (m & 3) + a
// sub-tile offset), so its 16 lanes per phase hit distinct bank groups. V:
// even values, distinct over the 8 rows that the 32 lanes of one
// transposing-read phase address (4 rows each of two lane groups), so the
// two 16-byte chunks of each row land on distinct bank groups too.
// max / sum of x over lanes l and l ^ 16 (v_permlane16_swap exchanges the
// odd and even 16-lane rows of its two operands; with both operands x each
// lane gets its own value and its partner's)
__device__ inline float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Largest lane sum of p the 48-row kernel accepts without moving the
// reference max: each p is then below it, within the 16-bit P operand's
// range (f16: 65504) and far from fp32 overflow in o and l.
template <Elt E>
constexpr float kW48Bound = E == Elt::F16 ? 32768.f : 1.8446744e19f;  // 2^15, 2^64

template <int NSL, int BYTES>
struct W48Ring {
  __attribute__((aligned(1024))) uint8_t k[NSL][BYTES];
  __attribute__((aligned(1024))) uint8_t v[NSL][BYTES];
};
struct SlotView {
  uint8_t* k;
  uint8_t* v;
  int off;  // the slot's byte offset within the K (and the V) array
};

__device__ inline int w48_kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
__device__ inline int w48_vswz(int row) { return ((row & 3) | (((row >> 3) & 1) << 2)) << 1; }

// K tiles and V tiles in two arrays, so that every slot's reads are one lane
// register plus an immediate offset below 64 KiB
using W48RingT = W48Ring<FA_W48_STAGES, kW48Bk * 256>;

// One 384-row query tile (head tl.bh, tile tl.t), from its Q loads to its
// O and LSE stores, with the workgroup's LDS ring.
template <Elt IN, bool CAUSAL, int KA>
__device__ __attribute__((always_inline)) inline void w48_tile(const FwdArgs& a, W48RingT& ring,
                                                               const TileId tl) {
  constexpr int ROWB = 256, BK = kW48Bk, QB = 3, KT = 2, NKS = 4, NDT = 8, NH = BK / 32;
  static_assert(BK == 32 || BK == 64, "32- or 64-key tiles");
  constexpr int TILE_B = BK * ROWB;
  constexpr int LPW = TILE_B / 1024 / kW48Waves;
  constexpr int NS = FA_W48_STAGES;
  static_assert(FA_W48_GROUP > 1 ? NS == 3 * FA_W48_GROUP : (NS >= 3 && NS <= 4), "ring stages");
  static_assert(FA_W48_GROUP >= 1 && FA_W48_GROUP <= 3, "tiles per barrier");
  static_assert(LPW >= 1, "tile too small for the wave count");

  // The lane index comes from the execution mask (mbcnt) and passes through
  // an empty asm, so that in a loop over tiles neither the work-item id
  // register nor anything derived from the lane stays live across a tile.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(lane));
  const int tid = w * 64 + lane, lm = lane & 15, g = lane >> 4;
  const HeadView hv = head_view<2, 2>(a, tl.bh);
  const int n = hv.n;
  // n is rarely a multiple of 384: the tiles are laid out from the last row
  // back, so the partial tile is the first one -- under a causal mask the
  // one with the fewest keys -- and rows before 0 are masked and not stored.
  const int tiles_n = (n + kW48Bq - 1) / kW48Bq;
  if (tl.t >= tiles_n) return;  // a tile past a short sequence (uniform)
  const int q0 = tl.t * kW48Bq - (tiles_n * kW48Bq - n);
  const int qw0 = q0 + kW48Rows * w;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(hv.q, span_bytes(n, hv.qrs, ROWB));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(hv.k, span_bytes(n, hv.krs, ROWB));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(hv.v, span_bytes(n, hv.vrs, ROWB));
  const KeyTiles kt = key_tiles<BK>(a, n, q0 + kW48Bq, CAUSAL);
  const int j_lo = kt.lo, nt = kt.hi;

  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (w * LPW + i) * 1024 + lane * 16;
    const int row = byte / ROWB, p = (byte % ROWB) / 16;
    koff[i] = (uint32_t)row * hv.krs + (uint32_t)((p ^ w48_kswz(row)) * 16);
    voff[i] = (uint32_t)row * hv.vrs + (uint32_t)((p ^ w48_vswz(row)) * 16);
  }
  auto issue = [&](SlotView slot, int J) __attribute__((always_inline)) {
    const uint32_t kb = J < nt ? (uint32_t)(J * BK) * hv.krs : 0x80000000u;
    const uint32_t vb = J < nt ? (uint32_t)(J * BK) * hv.vrs : 0x80000000u;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(rk, slot.k + (w * LPW + i) * 1024, kb + koff[i]);
      lds_dma16(rv, slot.v + (w * LPW + i) * 1024, vb + voff[i]);
    }
  };

#if FA_W48_PRIO
  // waves 0-3 issue ahead of their SIMD partners 4-7, so that one wave's
  // softmax runs beside the other's MFMAs rather than at the same time
  if (w < 4) __builtin_amdgcn_s_setprio(FA_W48_PRIO);
#endif
  // Q fragments: B operand of S^T = K Q^T, query 16 qb + lm, d-columns
  // 32 ks + 8 g .. + 7.
  u32x4_t qf[QB][NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int row = qw0 + 16 * qb + lm;  // rows before 0: an offset past the end (zeros)
      qf[qb][ks] = bload16(rq, row >= 0 ? (uint32_t)row * hv.qrs + (32 * ks + 8 * g) * 2 : 0x80000000u);
    }
  }
  if (a.qneg) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[qb][ks] ^= 0x80008000u;
    }
  }

  // LDS read offsets. K: sub-tile t's row for lane l is krow + 32 (t >> 1) +
  // 4 (t & 1) with krow = 8 (lm >> 2) + (lm & 3); its swizzle is lm for
  // every t. V: the transposing reads of key block kb, half r, d-tile dt
  // address row 32 kb + 8 g + 4 r + (lm >> 2), bytes 32 dt + 8 (lm & 3) of
  // the unswizzled row; the row's swizzle is the same for every kb, r.
  const int krow = 8 * (lm >> 2) + (lm & 3);
  const int vrow = 8 * g + (lm >> 2);
  const int vsw = 2 * ((lm >> 2) | ((g & 1) << 2));
  const int vch = (lm & 3) >> 1, vhalf = (lm & 1) * 8;
  // LDS read addresses per K k-step and per V d-tile, relative to the start
  // of each array and formed once: a slot's and a sub-tile's offsets then
  // fit the reads' 16-bit immediates (each array spans 48 KiB), instead of
  // one set of address registers per slot. The empty asm hides their
  // origin; the mask after it tells the compiler the sign bit is clear,
  // which lets it fold the immediates.
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  uint32_t kad[NKS], vad[NDT];
  {
    const uint32_t kb = (uint32_t)(uintptr_t)(lds_u8*)&ring.k[0][0];
    const uint32_t vb = (uint32_t)(uintptr_t)(lds_u8*)&ring.v[0][0];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kad[ks] = kb + krow * ROWB + (((4 * ks + g) ^ lm) * 16);
      asm volatile("" : "+v"(kad[ks]));
      kad[ks] &= 0x3ffffu;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      vad[dt] = vb + vrow * ROWB + (((2 * dt + vch) ^ vsw) * 16) + vhalf;
      asm volatile("" : "+v"(vad[dt]));
      vad[dt] &= 0x3ffffu;
    }
  }

  const float c = a.c;
  float m2[QB], lp[QB];
  f32x4_t o[NDT][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m2[qb] = -INFINITY;  // the reference max (base-2 units); see the softmax below
    lp[qb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt][qb] = f32x4_t{};
  }
  auto live = [&](int j) __attribute__((always_inline)) {
    return qw0 < n && qw0 + kW48Rows > 0 && !(CAUSAL && j * BK > qw0 + kW48Rows - 1);
  };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    return (j * BK + BK > n) || (CAUSAL && j * BK + BK - 1 > qw0);
  };

  // One tile: NH chunks of 32 keys, each Q K^T (two 16-key sub-tiles), the
  // softmax and P.V (one 32-key block); the next tile's copies go out after
  // the first chunk's softmax.
  auto compute = [&](const SlotView slot, int j, auto&& mid) __attribute__((always_inline)) {
    const bool mask = needs_mask(j);
#pragma unroll 1
    for (int h = 0; h < NH; ++h) {
      f32x4_t s[KT][QB];
#pragma unroll
      for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[t][qb] = f32x4_t{};
      }
      // operand i = (k-step i / KT, sub-tile i % KT), read KA
      // ahead in a pinned order
      constexpr int NKO = NKS * KT;
      auto kread = [&](int i) __attribute__((always_inline)) {
        const int ks = i / KT, t = i % KT;
        const int row = 32 * h + krow + 4 * t;
        return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)(kad[ks] + slot.off +
                                                                             (row - krow) * ROWB);
      };
      u32x4_t kf[KA];
#pragma unroll
      for (int i = 0; i < KA; ++i) kf[i] = kread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NKO; ++i) {
        const int ks = i / KT, t = i % KT;
        const u32x4_t cur = kf[i % KA];
        if (i + KA < NKO) kf[i % KA] = kread(i + KA);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[t][qb] = mfma16x16<IN>(cur, qf[qb][ks], s[t][qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (mask) {
        // register i of sub-tile t holds key j*BK + 8g + off, off = 32h +
        // 4t + i: visible iff off <= lim
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lim = (CAUSAL ? min(n - 1, qw0 + 16 * qb + lm) : n - 1) - (j * BK + 8 * g);
#pragma unroll
          for (int t = 0; t < KT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int off = 32 * h + 4 * t + i;
              s[t][qb][i] = off <= lim ? s[t][qb][i] : -INFINITY;
            }
          }
        }
      }
      // online softmax without a chunk max on the common path: p against the
      // row's current reference m. Since p >= 0, a lane's sum of p bounds
      // each of its p; only when some lane's sum passes kW48Bound (or is not
      // finite), or a row has no reference yet, does the chunk take the true
      // max, move the reference, rescale o and l and redo its exponentials.
      // The result is the same for any reference: m cancels in o / l and the
      // LSE is m + log2 l for whatever m was used; the first reference is a
      // true max, so a row's largest weight so far is exactly 1.
      u32x4_t pb[QB];
      float ls[QB];
      auto expo = [&](int qb, float nm) __attribute__((always_inline)) {
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float p0 = fast_exp2(__builtin_fmaf(s[t][qb][i], c, nm));
            const float p1 = fast_exp2(__builtin_fmaf(s[t][qb][i + 1], c, nm));
            acc += p0 + p1;
            pb[qb][2 * t + (i >> 1)] = pack2<IN>(p0, p1);
          }
        }
        ls[qb] = acc;
      };
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) expo(qb, -exp_ref(m2[qb]));
      const float lmax = fmaxf(fmaxf(ls[0], ls[1]), ls[2]);
      const float mmin = fminf(fminf(m2[0], m2[1]), m2[2]);
      if (__any(!(lmax <= kW48Bound<IN>) || mmin == -INFINITY)) {
        float alpha[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx = s[0][qb][0];
#pragma unroll
          for (int t = 0; t < KT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][qb][i]);
          }
          mx = pair_max(pair16_max(mx));
          const float mn = fmaxf(m2[qb], mx * c);  // -inf while the row has seen no visible key
          alpha[qb] = fast_exp2(m2[qb] - exp_ref(mn));
          m2[qb] = mn;
          lp[qb] *= alpha[qb];
          expo(qb, -exp_ref(mn));
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[dt][qb] *= alpha[qb];
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lp[qb] += ls[qb];
      if (h == 0) mid();
      // O^T += V^T P^T: per d-tile one V^T operand (two transposing reads of
      // four keys each), three MFMAs
      auto vread = [&](int dt) __attribute__((always_inline)) {
        const uint32_t a0 = vad[dt] + slot.off + 32 * h * ROWB;
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)a0));
        const u32x2_t hi = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(a0 + 4 * ROWB)));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4_t vf[KA];
#pragma unroll
      for (int i = 0; i < KA; ++i) vf[i] = vread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const u32x4_t cur = vf[dt % KA];
        if (dt + KA < NDT) vf[dt % KA] = vread(dt + KA);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[dt][qb] = mfma16x16<IN>(cur, pb[qb], o[dt][qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto slot_ref = [&](auto S) __attribute__((always_inline)) -> SlotView {
    return SlotView{ring.k[decltype(S)::value], ring.v[decltype(S)::value], decltype(S)::value * TILE_B};
  };
#if FA_W48_GROUP > 1
  // One barrier per group of GB tiles (NS = 3 GB slots): at a group's first
  // step every wave is past the previous group, whose slots take the group
  // after next; the other steps neither wait nor copy.
  constexpr int GB = FA_W48_GROUP;
  auto step = [&](auto S, int J) __attribute__((always_inline)) {
    constexpr int sv = decltype(S)::value;
    if constexpr (sv % GB == 0) {
      wait_vmcnt<GB * 2 * LPW>();  // this group's tiles have landed (the next group's may not)
      __syncthreads();
      auto refill = [&]() __attribute__((always_inline)) {
        issue(slot_ref(std::integral_constant<int, (sv + 2 * GB) % NS>{}), J + 2 * GB);
        issue(slot_ref(std::integral_constant<int, (sv + 2 * GB + 1) % NS>{}), J + 2 * GB + 1);
        if constexpr (GB > 2) issue(slot_ref(std::integral_constant<int, (sv + 2 * GB + 2) % NS>{}), J + 2 * GB + 2);
      };
      if (live(J)) compute(slot_ref(S), J, refill);
      else refill();
    } else {
      __builtin_amdgcn_sched_barrier(0);  // no motion across the step boundary
      if (live(J)) compute(slot_ref(S), J, []() {});
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#else
  auto step = [&](auto S, int J) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, (decltype(S)::value + NS - 1) % NS>;
    wait_vmcnt<(NS - 2) * 2 * LPW>();  // this wave's share of tile J has landed
    __syncthreads();                   // ... and every other wave's
    auto refill = [&]() __attribute__((always_inline)) { issue(slot_ref(SN{}), J + NS - 1); };
    if (live(J)) compute(slot_ref(S), J, refill);
    else refill();
  };
#endif

  {
    u32x4_t* p = (u32x4_t*)&ring;
    for (int i = tid; i < (int)(sizeof(ring) / 16); i += kW48Threads) p[i] = u32x4_t{0, 0, 0, 0};
  }
  __syncthreads();
  issue(slot_ref(std::integral_constant<int, 0>{}), j_lo);
  issue(slot_ref(std::integral_constant<int, 1>{}), j_lo + 1);
  if constexpr (NS > 3) issue(slot_ref(std::integral_constant<int, 2>{}), j_lo + 2);
  if constexpr (FA_W48_GROUP > 1) issue(slot_ref(std::integral_constant<int, 3>{}), j_lo + 3);
  if constexpr (FA_W48_GROUP > 2) {
    issue(slot_ref(std::integral_constant<int, 4>{}), j_lo + 4);
    issue(slot_ref(std::integral_constant<int, 5>{}), j_lo + 5);
  }
  // Q and the first tiles have landed: the compiler counts only the Q loads
  // (the tile copies are inline assembly), and without this full wait it
  // would wait for the newest loads -- the next tiles' copies -- before
  // every use of Q inside the loop.
  wait_vmcnt<0>();
  for (int J = j_lo; J < nt; J += NS) {
    step(std::integral_constant<int, 0>{}, J);
    if (J + 1 < nt) step(std::integral_constant<int, 1>{}, J + 1);
    if (J + 2 < nt) step(std::integral_constant<int, 2>{}, J + 2);
    if constexpr (NS > 3) if (J + 3 < nt) step(std::integral_constant<int, 3>{}, J + 3);
    if constexpr (NS > 4) if (J + 4 < nt) step(std::integral_constant<int, 4>{}, J + 4);
    if constexpr (NS > 5) if (J + 5 < nt) step(std::integral_constant<int, 5>{}, J + 5);
    if constexpr (NS > 6) if (J + 6 < nt) step(std::integral_constant<int, 6>{}, J + 6);
    if constexpr (NS > 7) if (J + 7 < nt) step(std::integral_constant<int, 7>{}, J + 7);
    if constexpr (NS > 8) if (J + 8 < nt) step(std::integral_constant<int, 8>{}, J + 8);
  }
  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends

  // epilogue: O = o / l per query (the four lanes of a query hold partial l),
  // LSE = ln 2 (m + log2 l). The lane index is formed afresh (opaque), so
  // that the store addresses are not computed before the tile loop and held
  // across it.
  int elane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(elane));
  const int elm = elane & 15, eg = elane >> 4;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(pair16_sum(lp[qb]));
    const int row = qw0 + 16 * qb + elm;
    const float inv = a.o_mult / lt;
    if (row >= 0 && row < n) {
      uint16_t* orow = (uint16_t*)hv.o + (size_t)row * hv.ors;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t x0 = pack2<IN>(o[dt][qb][0] * inv, o[dt][qb][1] * inv);
        const uint32_t x1 = pack2<IN>(o[dt][qb][2] * inv, o[dt][qb][3] * inv);
        *(u32x2_t*)(orow + 16 * dt + 4 * eg) = u32x2_t{x0, x1};
      }
      if (eg == 0 && hv.lse) hv.lse[row] = (m2[qb] + __log2f(lt)) * kLn2;
    }
  }
}

// One workgroup per query tile, in the grid order of tile_of_block.
template <Elt IN, bool CAUSAL>
__global__ __launch_bounds__(kW48Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_w48(FwdArgs a) {
  __shared__ W48RingT ring;
  const int tiles = (a.n + kW48Bq - 1) / kW48Bq;
  w48_tile<IN, CAUSAL, FA_W48_AHEAD>(a, ring, tile_of_block(blockIdx.x, a.bh, tiles, CAUSAL, kW48Bq));
}

// Causal tiles packed: plan.bins groups of tiles per head, each workgroup
// taking group `bin` of plan.heads_seq heads one after another (longest tile
// first within a head). Under a causal mask tile t reads 384 (t + 1) keys, so
// one workgroup per tile leaves the last CUs of a launch with the longest
// tiles; groups of near-equal total length (chosen on the host) finish
// together. With bh a multiple of 8, the workgroups of an XCD (workgroup i
// runs on XCD i mod 8) take the same heads: bh / (8 heads_seq) of them at a
// time, so that few heads' K and V compete for the XCD's L2.
template <Elt IN>
__global__ __launch_bounds__(kW48Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_w48_packed(W48Args wa) {
  __shared__ W48RingT ring;
  const FwdArgs& a = wa.a;
  const int nb = wa.plan.bins, hs = wa.plan.heads_seq, pid = blockIdx.x;
  const int tiles = (a.n + kW48Bq - 1) / kW48Bq;
  for (int i = 0; i < hs; ++i) {
    int bh, bin;
    if ((a.bh & 7) == 0) {
      const int s = pid >> 3;
      bh = ((s / nb) * hs + i) * 8 + (pid & 7);
      bin = s % nb;
    } else {
      bh = pid / nb;
      bin = pid % nb;
    }
    for (int t = tiles - 1; t >= 0; --t) {
      if (wa.plan.bin_of_tile[t] != bin) continue;
      // the arguments are read through the kernel-argument pointer after an
      // empty asm, per tile: loaded where the tile uses them rather than
      // held in scalar registers across the loop
      uint64_t ka = (uint64_t)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(ka));
      const __attribute__((address_space(4))) W48Args* kp = (const __attribute__((address_space(4))) W48Args*)ka;
      w48_tile<IN, true, FA_W48_PACK_AHEAD>(*(const FwdArgs*)&kp->a, ring, TileId{bh, t});
      __syncthreads();  // every wave is past the ring before the next tile clears it
    }
  }
}

hipError_t launch(void (*kernel)(FwdArgs), const FwdArgs& a, hipStream_t stream, int rows = kBq,
                  int threads = kThreads) {
  const int tiles = (a.n + rows - 1) / rows;
  const unsigned grid = (unsigned)a.bh * (unsigned)tiles;
  return launch_kernel(kernel, dim3(grid, (unsigned)a.splits), dim3(threads), stream, a);
}

// ---------------------------------------------------------------------------
// Split-KV combine: for each row, LSE = ln sum_g e^{LSE_g} and
// O = sum_g e^{LSE_g - LSE} O_g (the associative merge of per-block softmax
// states, "Mastering FlashAttention: The Algebraic Foundation"). Memory-bound:
// each lane owns 4 consecutive d-columns of one row (16-byte loads), so a
// wave covers 64 / (D / 4) rows and a 256-thread workgroup kCombineRows(D).
// ---------------------------------------------------------------------------
template <int D>
constexpr int kCombineRows = 256 / (D / 4);

template <Elt OUT, int D>
__global__ __launch_bounds__(256) void combine_splits(CombineArgs a) {
  constexpr int kLanesPerRow = D / 4;
  const int64_t row = (int64_t)blockIdx.x * kCombineRows<D> + (int)threadIdx.x / kLanesPerRow;
  const int col = ((int)threadIdx.x % kLanesPerRow) * 4;
  if (row >= a.rows) return;
  const int64_t plane = a.rows;  // rows per split
  float mx = -INFINITY;
  for (int g = 0; g < a.splits; ++g) mx = fmaxf(mx, a.part_lse[g * plane + row]);
  // every row has a visible key in some block, so mx is finite
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int g = 0; g < a.splits; ++g) {
    const float lg = a.part_lse[g * plane + row];
    const float wg = lg == -INFINITY ? 0.f : fast_exp2((lg - mx) * kLog2e);
    const float4 po = *(const float4*)(a.part_o + (g * plane + row) * D + col);
    wsum += wg;
    acc.x = __builtin_fmaf(wg, po.x, acc.x);
    acc.y = __builtin_fmaf(wg, po.y, acc.y);
    acc.z = __builtin_fmaf(wg, po.z, acc.z);
    acc.w = __builtin_fmaf(wg, po.w, acc.w);
  }
  const float inv = 1.f / wsum;
  const size_t at = (size_t)row * D + col;
  if constexpr (OUT == Elt::F32) {
    *(float4*)((float*)a.o + at) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    using T = typename std::conditional<OUT == Elt::F16, _Float16, __bf16>::type;
    struct alignas(8) T4 { T v[4]; };
    T4 r;
    r.v[0] = (T)(acc.x * inv);
    r.v[1] = (T)(acc.y * inv);
    r.v[2] = (T)(acc.z * inv);
    r.v[3] = (T)(acc.w * inv);
    *(T4*)((T*)a.o + at) = r;
  }
  if (col == 0 && a.lse) a.lse[row] = mx + __logf(wsum);
}

template <Elt OUT>
hipError_t launch_combine_t(const CombineArgs& a, hipStream_t s) {
  if (a.d == 64) {
    const unsigned grid = (unsigned)((a.rows + kCombineRows<64> - 1) / kCombineRows<64>);
    return launch_kernel(combine_splits<OUT, 64>, dim3(grid), dim3(256), s, a);
  }
  const unsigned grid = (unsigned)((a.rows + kCombineRows<128> - 1) / kCombineRows<128>);
  return launch_kernel(combine_splits<OUT, 128>, dim3(grid), dim3(256), s, a);
}


// Groups of causal query tiles for fwd_w48_packed. Tile t of a head costs its
// 32-key steps, ceil(min(n, 384 (t + 1) - shift) / 32), plus two steps' worth
// for its Q loads, ring set-up and stores. The groups are the first-fit-
// decreasing packing at the smallest capacity it fits (binary search), or
// longest-first onto the least-loaded group where that gives the lower
// maximum; the same tiles every call for one (n, bins). Returns the largest
// group's cost (and the total in *total_out).
long w48_plan(int n, int tiles, int bins, W48Plan& p, long* total_out) {
  int cost[kW48PlanTiles];
  long load[256];
  uint8_t ffd[kW48PlanTiles], lpt[kW48PlanTiles];
  const int shift = tiles * kW48Bq - n;
  long total = 0, biggest = 0;
  for (int t = 0; t < tiles; ++t) {
    const int keys = std::min(n, kW48Bq * (t + 1) - shift);
    cost[t] = (keys + kW48Bk - 1) / kW48Bk + 2;
    total += cost[t];
    biggest = std::max<long>(biggest, cost[t]);
  }
  // cost grows with t: t = tiles - 1 .. 0 is decreasing order
  auto fits = [&](long cap) {
    std::fill(load, load + bins, 0L);
    for (int t = tiles - 1; t >= 0; --t) {
      int b = 0;
      while (b < bins && load[b] + cost[t] > cap) ++b;
      if (b == bins) return false;
      load[b] += cost[t];
      ffd[t] = (uint8_t)b;
    }
    return true;
  };
  long lo = std::max(biggest, (total + bins - 1) / bins), hi = total;
  while (lo < hi) {
    const long mid = (lo + hi) / 2;
    if (fits(mid)) hi = mid;
    else lo = mid + 1;
  }
  fits(lo);
  std::fill(load, load + bins, 0L);
  long lpt_max = 0;
  for (int t = tiles - 1; t >= 0; --t) {
    const int b = (int)(std::min_element(load, load + bins) - load);
    load[b] += cost[t];
    lpt[t] = (uint8_t)b;
    lpt_max = std::max(lpt_max, load[b]);
  }
  const uint8_t* best = lpt_max < lo ? lpt : ffd;
  p.bins = bins;
  p.heads_seq = 1;
  std::copy(best, best + tiles, p.bin_of_tile);
  *total_out = total;
  return std::min(lpt_max, lo);
}

template <Elt E, int D>
hipError_t dispatch_causal(const FwdArgs& a, hipStream_t s) {
  if constexpr (E == Elt::F32) {
    return a.causal ? launch(fwd_mfma32<D, true>, a, s) : launch(fwd_mfma32<D, false>, a, s);
  } else if constexpr (E == Elt::FP8) {
    return a.causal ? launch(fwd_direct8<D, true>, a, s, kDirectBq, kDirectThreads)
                    : launch(fwd_direct8<D, false>, a, s, kDirectBq, kDirectThreads);
  } else {
    if constexpr (D == 128 && FA_W48 != 0) {
      const int wt = (a.n + kW48Bq - 1) / kW48Bq;
      // 384-row tiles only while they give every CU two or more workgroups;
      // ragged batches, split keys and partial outputs stay on the 256-row
      // kernel
      const bool dense = !a.cu_seqlens && a.splits == 1 && !a.part_o && (long)a.bh * wt >= 2L * device_cus();
      // causal heads of FA_W48_PACK_MIN_N <= n < FA_W48_MIN_N: the tiles
      // packed into groups of near-equal length, one workgroup per group and
      // at most one per CU, when every head gets two or more groups (longer
      // heads measured faster with one workgroup per tile, in the order of
      // tile_of_block: one head at a time per XCD, longest tiles first)
      const int cus = device_cus(), nb = cus / a.bh;
      if (FA_W48_PACK && dense && a.causal && a.n >= FA_W48_PACK_MIN_N && a.n < FA_W48_MIN_N &&
          wt <= kW48PlanTiles && nb >= 2 && nb <= 255) {
        W48Args wa{};
        wa.a = a;
        long total = 0;
        w48_plan(a.n, wt, nb, wa.plan, &total);
        // fewer heads at a time per XCD (each workgroup taking 2, 4, ... heads
        // in turn, with proportionally more groups per head) while the groups
        // stay within 3% of equal
        if ((a.bh & 7) == 0) {
          for (int hs = 2; (a.bh / 8) % hs == 0 && cus * hs / a.bh <= std::min(wt, 255); hs *= 2) {
            W48Plan p2;
            const int nb2 = cus * hs / a.bh;
            const long mx = w48_plan(a.n, wt, nb2, p2, &total);
            if (mx * nb2 > total + total * 3 / 100) break;
            p2.heads_seq = hs;
            wa.plan = p2;
          }
        }
        const unsigned grid = (unsigned)(a.bh / wa.plan.heads_seq * wa.plan.bins);
        return launch_kernel(fwd_w48_packed<E>, dim3(grid), dim3(kW48Threads), s, wa);
      }
      // otherwise one workgroup per tile: for long heads (n >= FA_W48_MIN_N),
      // and, without the mask, from FA_W48_PACK_MIN_N rows where its grid
      // fills its rounds of workgroups at least 91% as well as the 256-row
      // kernel's does (its rounds run ~12% faster; measured +3% to +24% at
      // 6144 <= n <= 12288, -6% at 48 heads of 8192 (fill ratio 0.83) and
      // -3% at 32 heads of 7000 (0.905))
      bool w48_fill = false;
      if (dense && !a.causal && a.n >= FA_W48_PACK_MIN_N && a.n < FA_W48_MIN_N) {
        const long c = cus, w48 = (long)a.bh * wt;
        const int dt = (a.n + kDirectBq - 1) / kDirectBq;
        const bool dpair = dt % 2 == 0 && FA_PAIR_TILES_NOMASK && FA_STAGES == 2 && (long)a.bh * (dt / 2) >= c;
        const long wd = (long)a.bh * (dpair ? dt / 2 : dt);
        const long r48 = (w48 + c - 1) / c, rd = (wd + c - 1) / c;  // rounds
        // fill(w48) >= 0.91 fill(direct), fill = workgroups / (rounds * CUs)
        w48_fill = 100 * w48 * rd >= 91 * wd * r48;
      }
      if (dense && (a.n >= FA_W48_MIN_N || w48_fill)) {
        const dim3 grid((unsigned)a.bh * (unsigned)wt, 1u);
        return a.causal ? launch_kernel(fwd_w48<E, true>, grid, dim3(kW48Threads), s, a)
                        : launch_kernel(fwd_w48<E, false>, grid, dim3(kW48Threads), s, a);
      }
    }
    const int tiles = (a.n + kDirectBq - 1) / kDirectBq;
    // Pairs of equal tiles (no mask) only when the paired grid still fills
    // every CU; causal pairs are never longer than the longest unpaired tile.
    const bool pair_ok = a.causal ? FA_PAIR_TILES
                                  : FA_PAIR_TILES_NOMASK && (long)a.bh * (tiles / 2) >= device_cus();
    if (!a.cu_seqlens && a.splits == 1 && tiles % 2 == 0 && pair_ok && FA_STAGES == 2) {
      FwdArgs b = a;
      b.pair = 1;
      const dim3 grid((unsigned)a.bh * (unsigned)(tiles / 2), 1u);
      return a.causal ? launch_kernel(fwd_direct<E, D, true>, grid, dim3(kDirectThreads), s, b)
                      : launch_kernel(fwd_direct<E, D, false>, grid, dim3(kDirectThreads), s, b);
    }
    return a.causal ? launch(fwd_direct<E, D, true>, a, s, kDirectBq, kDirectThreads)
                    : launch(fwd_direct<E, D, false>, a, s, kDirectBq, kDirectThreads);
  }
}

template <Elt E>
hipError_t dispatch_d(const FwdArgs& a, hipStream_t s) {
  return a.d == 64 ? dispatch_causal<E, 64>(a, s) : dispatch_causal<E, 128>(a, s);
}

}  // namespace

// Compute units of the current device (256 on MI355X), read once per device.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  switch (a.out) {
    case Elt::F32: return launch_combine_t<Elt::F32>(a, stream);
    case Elt::F16: return launch_combine_t<Elt::F16>(a, stream);
    default: return launch_combine_t<Elt::BF16>(a, stream);
  }
}

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
  switch (a.elt) {
    case Elt::F32: return dispatch_d<Elt::F32>(a, stream);
    case Elt::F16: return dispatch_d<Elt::F16>(a, stream);
    case Elt::BF16: return dispatch_d<Elt::BF16>(a, stream);
    case Elt::FP8: return dispatch_d<Elt::FP8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
