// Launch entry points shared between the host front end (fa_api.cpp) and the
// HIP kernels (fa_fwd.hip). Internal to the library; the public interface is
// include/fa.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace fa {

enum class Elt { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  int bh;          // batch * heads
  int n;           // queries = keys per (batch, head); the longest sequence with cu_seqlens
  int d;           // 64 or 128
  // Layout, in elements: element (b, h, i, c) of q is q[b*q_sb + h*q_sh + i*q_sr + c];
  // likewise k, v, o. The dense [batch, heads, n, d] layout has
  // (sb, sh, sr) = (heads*n*d, n*d, d). LSE is [bh][n] (dense rows).
  int heads;
  int64_t q_sb, q_sh, q_sr, k_sb, k_sh, k_sr, v_sb, v_sh, v_sr, o_sb, o_sh, o_sr;
  // Ragged batches: when set, sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]
  // of a packed row axis of `total` rows (the batch strides are then unused)
  // and LSE is [heads][total].
  const int* cu_seqlens;
  int total;
  bool causal;
  // c = |scale| (times both fp8 descales) times log2(e), > 0. A negative
  // scale is applied as q -> -q (exact in every element type): then
  // scale (q . k) = |scale| ((-q) . k), and the kernels' row max of c s is
  // the max of the scaled scores.
  float c;
  bool qneg = false;
  float o_mult;    // multiplier applied to O in the epilogue (v descale; 1 otherwise)
  Elt elt;
  // Split-KV: the keys are cut into blocks of split_keys (a multiple of 128;
  // n when the keys are not split) and grid dimension y runs over the blocks.
  // When part_o is set, each block writes its partial result there instead of
  // o / lse: O_g normalised by its own row sum, fp32 [splits][bh][n][d], and
  // LSE_g, fp32 [splits][bh][n] (-inf where the block holds no visible key).
  int split_keys;
  int splits;
  float* part_o;
  // Causal f16 / bf16 launches with an even number of 256-row query tiles and
  // no split or ragged batch: each workgroup takes tiles T-1-p and p of one
  // head (set by the launcher).
  int pair = 0;
  float* part_lse;
};

// Merge of split-KV partials into O and LSE (the log-sum-exp combine).
struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;      // may be null
  int64_t rows;    // batch * heads * n
  int d;
  int splits;
  Elt out;         // F32, F16 or BF16
};

// Backward pass (f16 / bf16): gradients of O = softmax(scale Q K^T + mask) V
// given dO, recomputing P from Q, K and the forward's LSE.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // natural-log LSE of the forward, fp32 [bh][n]
  float* delta;       // workspace: D = rowsum(dO * O), fp32 [bh][n]
  float* nlse2;       // workspace: -LSE * log2(e), fp32 [bh][n]
  void* dq;
  void* dk;
  void* dv;
  int bh;
  int n;           // rows per (batch, head); the longest sequence with cu_seqlens
  int d;
  // Row stride (elements) shared by q, k, v, o, dout, dq, dk, dv: d for the
  // dense [bh][n][d] layout, heads * d for packed [total][heads][d] rows.
  int heads;
  int64_t rs;
  // Ragged batches (as FwdArgs): sequence b is rows cu_seqlens[b] ..
  // cu_seqlens[b+1] of `total` packed rows; lse and the workspace rows are
  // then [heads][total].
  const int* cu_seqlens;
  int total;
  bool causal;
  float c;            // scale * log2(e); either sign (never 0: a zero scale is run as FLT_MIN)
  float scale;
  Elt elt;            // F16 or BF16
  // Paired query tiles in the dQ pass (as FwdArgs::pair; set by the launcher).
  int pair = 0;
};

// Unfused forward (f16 / bf16): S and P materialised in the caller's
// workspace.
struct UnfArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  float* s;        // fp32 S [bh][n][n]
  uint16_t* p;     // P in the input type [bh][n][n]
  int bh;
  int n;
  int d;
  int rows;        // bh * n
  bool causal;
  float scale;
  Elt elt;
};

// Enqueue the forward kernel for validated arguments. Returns the HIP status
// of the launch.
hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
// Enqueue the two backward kernels (the query-major dQ pass, which also
// writes delta and nlse2, then the key-major dK / dV pass).
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);
// Enqueue the three unfused kernels (scores, row softmax, P V).
hipError_t launch_unfused(const UnfArgs& a, hipStream_t stream);
// Compute units of the current device (256 on MI355X), read once per device.
int device_cus();

// Size of the fixed per-GPU scratch array of fa_forward_splitkv_noalloc, and
// its device address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = (size_t)128 << 20;
hipError_t noalloc_scratch(void** out);

}  // namespace fa
