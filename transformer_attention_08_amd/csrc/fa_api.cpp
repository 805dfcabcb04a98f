// Host front end of the C ABI declared in include/fa.h: argument validation
// (pure host code, before any HIP call), then the kernel launches.
#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cfloat>

#include <hip/hip_runtime_api.h>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kAbiVersion = 10000;  // 1.0.0

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// The grid has one workgroup per (batch*head, 128-row query tile); its size
// must fit gridDim.x. Element offsets inside the kernels are 64-bit.
constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr double kLog2e = 1.4426950408889634;

// Any finite scale whose product with log2(e) is a finite float.
bool scale_ok(float scale) { return std::isfinite(scale) && std::isfinite((float)(scale * kLog2e)); }

int validate(const void* q, const void* k, const void* v, void* o, const float* lse, int batch,
             int heads, int n, int d_k, float scale, int causal, int dtype) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (batch < 1 || heads < 1 || n < 1) return FA_ERR_SHAPE;
  if (dtype < FA_F32 || dtype > FA_FP8_E4M3) return FA_ERR_DTYPE;
  if ((d_k != 64 && d_k != 128) || (causal != 0 && causal != 1)) return FA_ERR_UNSUPPORTED;
  const uintptr_t ptrs[5] = {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)o, (uintptr_t)lse};
  for (uintptr_t p : ptrs)
    if (p % 16) return FA_ERR_ALIGN;
  if (!scale_ok(scale)) return FA_ERR_SCALE;

  const int64_t bh = (int64_t)batch * heads;
  const int64_t rows = bh * n;
  const int64_t tiles = ((int64_t)n + 127) / 128;
  if (bh > kMaxGrid || bh * tiles > kMaxGrid) return FA_ERR_OVERFLOW;
  const int in_bytes = dtype == FA_F32 ? 4 : dtype == FA_FP8_E4M3 ? 1 : 2;
  const int out_bytes = dtype == FA_F32 ? 4 : 2;
  // byte sizes must fit comfortably in 63 bits, and one head's bytes in the
  // kernels' 32-bit buffer ranges
  if (rows > (INT64_C(1) << 62) / ((int64_t)d_k * 4)) return FA_ERR_OVERFLOW;
  if ((int64_t)n * d_k * std::max(in_bytes, out_bytes) > INT32_MAX) return FA_ERR_OVERFLOW;
  const int64_t in_sz = rows * d_k * in_bytes, out_sz = rows * d_k * out_bytes, lse_sz = rows * 4;

  const Range rq{(uintptr_t)q, (uintptr_t)q + (uintptr_t)in_sz};
  const Range rk{(uintptr_t)k, (uintptr_t)k + (uintptr_t)in_sz};
  const Range rv{(uintptr_t)v, (uintptr_t)v + (uintptr_t)in_sz};
  const Range ro{(uintptr_t)o, (uintptr_t)o + (uintptr_t)out_sz};
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv)) return FA_ERR_ALIAS;
  if (lse) {
    const Range rl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)lse_sz};
    if (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, ro)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// Keys per split-KV block for a requested number of blocks (a multiple of
// 128, the coarsest key tile of the kernels, so that every block starts on a
// tile boundary), and the number of blocks that results.
constexpr int kMaxSplits = 256;
int split_keys_for(int n, int splits) {
  const int64_t per = ((int64_t)n + splits - 1) / splits;
  return (int)(((per + 127) / 128) * 128);
}
int splits_used(int n, int splits) {
  const int sk = split_keys_for(n, splits);
  return (n + sk - 1) / sk;
}
struct SplitLayout {
  size_t o_bytes, lse_off, total;
};
SplitLayout split_layout(int batch, int heads, int n, int d_k, int used) {
  const size_t rows = (size_t)batch * heads * n * (size_t)used;
  SplitLayout s;
  s.o_bytes = rows * d_k * 4;
  s.lse_off = (s.o_bytes + 255) / 256 * 256;
  s.total = s.lse_off + rows * 4;
  return s;
}

// Backward workspace: D = rowsum(dO * O) at byte 0, -LSE*log2(e) from the
// next multiple of 256 bytes; fp32 [batch][heads][n] each.
struct BwdLayout {
  size_t nl_off, total;
};
BwdLayout bwd_layout(int batch, int heads, int n) {
  const size_t rows = (size_t)batch * heads * n;
  BwdLayout l;
  l.nl_off = (rows * 4 + 255) / 256 * 256;
  l.total = l.nl_off + rows * 4;
  return l;
}

int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int n,
                 int d_k, float scale, int causal, int dtype, void* workspace,
                 size_t workspace_bytes) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  if (batch < 1 || heads < 1 || n < 1) return FA_ERR_SHAPE;
  if (dtype < FA_F32 || dtype > FA_FP8_E4M3) return FA_ERR_DTYPE;
  if ((dtype != FA_F16 && dtype != FA_BF16) || (d_k != 64 && d_k != 128) ||
      (causal != 0 && causal != 1))
    return FA_ERR_UNSUPPORTED;
  const uintptr_t ptrs[10] = {(uintptr_t)q,  (uintptr_t)k,  (uintptr_t)v,  (uintptr_t)o,
                              (uintptr_t)dout, (uintptr_t)lse, (uintptr_t)dq, (uintptr_t)dk,
                              (uintptr_t)dv, (uintptr_t)workspace};
  for (uintptr_t p : ptrs)
    if (p % 16) return FA_ERR_ALIGN;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  const int64_t bh = (int64_t)batch * heads;
  const int64_t rows = bh * n;
  if (bh > kMaxGrid || bh * (((int64_t)n + 127) / 128) > kMaxGrid) return FA_ERR_OVERFLOW;
  if (rows > (INT64_C(1) << 62) / ((int64_t)d_k * 4)) return FA_ERR_OVERFLOW;
  if (((int64_t)n + 256) * d_k * 2 > INT32_MAX) return FA_ERR_OVERFLOW;
  const BwdLayout wl = bwd_layout(batch, heads, n);
  if (workspace_bytes < wl.total) return FA_ERR_SHAPE;
  const uintptr_t t_sz = (uintptr_t)(rows * d_k * 2);
  const Range ins[6] = {{(uintptr_t)q, (uintptr_t)q + t_sz},       {(uintptr_t)k, (uintptr_t)k + t_sz},
                        {(uintptr_t)v, (uintptr_t)v + t_sz},       {(uintptr_t)o, (uintptr_t)o + t_sz},
                        {(uintptr_t)dout, (uintptr_t)dout + t_sz}, {(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(rows * 4)}};
  const Range outs[4] = {{(uintptr_t)dq, (uintptr_t)dq + t_sz},
                         {(uintptr_t)dk, (uintptr_t)dk + t_sz},
                         {(uintptr_t)dv, (uintptr_t)dv + t_sz},
                         {(uintptr_t)workspace, (uintptr_t)workspace + wl.total}};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// Unfused workspace: fp32 S [bh][n][n] at byte 0, P in the input type from
// the next multiple of 256 bytes.
struct UnfLayout {
  size_t p_off, total;
};
UnfLayout unf_layout(int batch, int heads, int n) {
  const size_t cells = (size_t)batch * heads * (size_t)n * (size_t)n;
  UnfLayout l;
  l.p_off = (cells * 4 + 255) / 256 * 256;
  l.total = l.p_off + cells * 2;
  return l;
}

// Element strides (batch, head, row) of q, k, v, o, and the ragged-batch
// description; null in run() means the dense [batch, heads, n, d_k] layout.
struct Layout {
  int64_t s[12];
  const int* cu_seqlens;
  int total;
};

int elt_bytes_in(int dtype) { return dtype == FA_F32 ? 4 : dtype == FA_FP8_E4M3 ? 1 : 2; }
int elt_bytes_out(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Byte range [lo, hi) a strided tensor touches.
Range strided_span(const void* p, const int64_t* s, int batch, int heads, int n, int d_k, int esize) {
  const int64_t last = (int64_t)(batch - 1) * s[0] + (int64_t)(heads - 1) * s[1] + (int64_t)(n - 1) * s[2] + d_k;
  return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)(last * esize)};
}

// Do the (batch, head, row) positions of a strided tensor address disjoint
// d_k-element rows? Sufficient test: sorted by stride, every dimension of
// extent > 1 steps over the whole extent of the ones below it.
bool rows_disjoint(const int64_t* s, int batch, int heads, int n, int d_k) {
  int64_t st[3] = {s[0], s[1], s[2]};
  int64_t ex[3] = {batch, heads, n};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i]) {
        std::swap(st[i], st[j]);
        std::swap(ex[i], ex[j]);
      }
  int64_t covered = d_k;  // elements spanned by the dimensions below
  for (int i = 0; i < 3; ++i) {
    if (ex[i] == 1) continue;
    if (st[i] < covered) return false;
    covered = st[i] * (ex[i] - 1) + covered;
  }
  return true;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int heads,
        int n, int d_k, float qk_scale, int causal, int dtype, float o_mult, void* stream,
        int splits = 1, void* workspace = nullptr, const Layout* lay = nullptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.bh = batch * heads;
    a.n = n;
    a.d = d_k;
    a.heads = heads;
    const int64_t dense[3] = {(int64_t)heads * n * d_k, (int64_t)n * d_k, d_k};
    const int64_t* s = lay ? lay->s : nullptr;
    int64_t* dst[12] = {&a.q_sb, &a.q_sh, &a.q_sr, &a.k_sb, &a.k_sh, &a.k_sr,
                        &a.v_sb, &a.v_sh, &a.v_sr, &a.o_sb, &a.o_sh, &a.o_sr};
    for (int i = 0; i < 12; ++i) *dst[i] = s ? s[i] : dense[i % 3];
    a.cu_seqlens = lay ? lay->cu_seqlens : nullptr;
    a.total = lay ? lay->total : 0;
    a.causal = causal != 0;
    // The kernels need c > 0. A negative scale is applied as q -> -q, which
    // is exact: scale (q . k) = |scale| ((-q) . k). A zero scale is replaced
    // by the smallest normal float, for which every exp2 argument rounds to 0
    // exactly as with c = 0 (uniform weights), while masked scores (-inf)
    // still give weight 0.
    float c = (float)(std::fabs((double)qk_scale) * kLog2e);
    if (!(c > 0.f)) c = FLT_MIN;
    a.c = c;
    a.qneg = qk_scale < 0.f;
    a.o_mult = o_mult;
    a.elt = static_cast<fa::Elt>(dtype);
    a.split_keys = n;
    a.splits = 1;
    a.part_o = nullptr;
    a.part_lse = nullptr;
    const int used = splits > 1 ? splits_used(n, splits) : 1;
    if (used > 1) {
      const SplitLayout sl = split_layout(batch, heads, n, d_k, used);
      a.split_keys = split_keys_for(n, splits);
      a.splits = used;
      a.part_o = (float*)workspace;
      a.part_lse = (float*)((char*)workspace + sl.lse_off);
    }
    e = fa::launch_forward(a, static_cast<hipStream_t>(stream));
    if (e == hipSuccess && used > 1) {
      fa::CombineArgs cb;
      cb.part_o = a.part_o;
      cb.part_lse = a.part_lse;
      cb.o = o;
      cb.lse = lse;
      cb.rows = (int64_t)batch * heads * n;
      cb.d = d_k;
      cb.splits = used;
      cb.out = dtype == FA_F32 ? fa::Elt::F32 : dtype == FA_F16 ? fa::Elt::F16 : fa::Elt::BF16;
      e = fa::launch_combine(cb, static_cast<hipStream_t>(stream));
    }
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// Launch the two backward kernels for validated arguments. Dense layout when
// cu_seqlens is null; otherwise packed [total, heads, d_k] rows.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int n, int d_k,
            float scale, int causal, int dtype, void* workspace, const int* cu_seqlens, int total,
            void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    const BwdLayout wl = cu_seqlens ? bwd_layout(1, heads, total) : bwd_layout(batch, heads, n);
    fa::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.delta = (float*)workspace;
    a.nlse2 = (float*)((char*)workspace + wl.nl_off);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.bh = batch * heads;
    a.n = n;
    a.d = d_k;
    a.heads = heads;
    a.rs = cu_seqlens ? (int64_t)heads * d_k : d_k;
    a.cu_seqlens = cu_seqlens;
    a.total = total;
    a.causal = causal != 0;
    // either sign (the kernels mask scores so that c * s = -inf); a zero
    // scale is run as the smallest normal float, as in the forward: uniform
    // weights while masked scores still give weight 0
    float c = (float)(scale * kLog2e);
    if (c == 0.f) c = FLT_MIN;
    a.c = c;
    a.scale = scale;
    a.elt = static_cast<fa::Elt>(dtype);
    e = fa::launch_backward(a, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
               int heads, int n, int d_k, float scale, int causal, int dtype, void* stream) {
  const int st = validate(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype);
  if (st != FA_OK) return st;
  return run(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype, 1.0f, stream);
}

int fa_forward_strided(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                       int heads, int n, int d_k, const int64_t* strides, float scale, int causal,
                       int dtype, void* stream) {
  if (!q || !k || !v || !o || !strides) return FA_ERR_NULL;
  if (batch < 1 || heads < 1 || n < 1) return FA_ERR_SHAPE;
  if (dtype < FA_F32 || dtype > FA_FP8_E4M3) return FA_ERR_DTYPE;
  if ((d_k != 64 && d_k != 128) || (causal != 0 && causal != 1)) return FA_ERR_UNSUPPORTED;
  for (uintptr_t p : {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)o, (uintptr_t)lse})
    if (p % 16) return FA_ERR_ALIGN;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  const int ib = elt_bytes_in(dtype), ob = elt_bytes_out(dtype);
  for (int i = 0; i < 12; ++i) {
    const int eb = i < 9 ? ib : ob;
    if (strides[i] < 0) return FA_ERR_UNSUPPORTED;
    if ((strides[i] * eb) % 16) return FA_ERR_ALIGN;
    if (strides[i] > (INT64_C(1) << 40)) return FA_ERR_OVERFLOW;
  }
  for (int t = 0; t < 4; ++t) {
    const int64_t sr = strides[3 * t + 2];
    const int eb = t < 3 ? ib : ob;
    if (sr < d_k) return FA_ERR_UNSUPPORTED;  // rows of one head must not overlap
    // one head's rows (plus the padding rows of the last tile) within the
    // kernels' 32-bit buffer offsets
    if (((int64_t)n + 256) * sr * eb > INT32_MAX) return FA_ERR_OVERFLOW;
  }
  const int64_t bh = (int64_t)batch * heads;
  if (bh > kMaxGrid || bh * (((int64_t)n + 127) / 128) > kMaxGrid) return FA_ERR_OVERFLOW;
  if (!rows_disjoint(strides + 9, batch, heads, n, d_k)) return FA_ERR_ALIAS;
  const Range rq = strided_span(q, strides, batch, heads, n, d_k, ib);
  const Range rk = strided_span(k, strides + 3, batch, heads, n, d_k, ib);
  const Range rv = strided_span(v, strides + 6, batch, heads, n, d_k, ib);
  const Range ro = strided_span(o, strides + 9, batch, heads, n, d_k, ob);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv)) return FA_ERR_ALIAS;
  if (lse) {
    const Range rl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(bh * n * 4)};
    if (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, ro)) return FA_ERR_ALIAS;
  }
  Layout lay;
  for (int i = 0; i < 12; ++i) lay.s[i] = strides[i];
  lay.cu_seqlens = nullptr;
  lay.total = 0;
  return run(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype, 1.0f, stream, 1, nullptr,
             &lay);
}

int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens, int batch, int total, int max_seqlen, int heads,
                      int d_k, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens) return FA_ERR_NULL;
  if (batch < 1 || heads < 1 || max_seqlen < 1 || total < 0) return FA_ERR_SHAPE;
  if (dtype < FA_F32 || dtype > FA_FP8_E4M3) return FA_ERR_DTYPE;
  if ((d_k != 64 && d_k != 128) || (causal != 0 && causal != 1)) return FA_ERR_UNSUPPORTED;
  for (uintptr_t p : {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)o, (uintptr_t)lse})
    if (p % 16) return FA_ERR_ALIGN;
  if ((uintptr_t)cu_seqlens % 4) return FA_ERR_ALIGN;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  const int ib = elt_bytes_in(dtype), ob = elt_bytes_out(dtype);
  const int64_t rs = (int64_t)heads * d_k;  // row stride, elements
  if (((int64_t)max_seqlen + 256) * rs * std::max(ib, ob) > INT32_MAX) return FA_ERR_OVERFLOW;
  const int64_t bh = (int64_t)batch * heads;
  if (bh > kMaxGrid || bh * (((int64_t)max_seqlen + 127) / 128) > kMaxGrid) return FA_ERR_OVERFLOW;
  if ((int64_t)total * rs > (INT64_C(1) << 50)) return FA_ERR_OVERFLOW;
  const Range rq{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(total * rs * ib)};
  const Range rk{(uintptr_t)k, (uintptr_t)k + (uintptr_t)(total * rs * ib)};
  const Range rv{(uintptr_t)v, (uintptr_t)v + (uintptr_t)(total * rs * ib)};
  const Range ro{(uintptr_t)o, (uintptr_t)o + (uintptr_t)(total * rs * ob)};
  const Range rc{(uintptr_t)cu_seqlens, (uintptr_t)cu_seqlens + (uintptr_t)(batch + 1) * 4};
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(ro, rc)) return FA_ERR_ALIAS;
  if (lse) {
    const Range rl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)((int64_t)heads * total * 4)};
    if (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv) || overlap(rl, ro) || overlap(rl, rc))
      return FA_ERR_ALIAS;
  }
  if (total == 0) return FA_OK;  // no rows: nothing to compute
  Layout lay;
  const int64_t s[3] = {0, d_k, rs};
  for (int i = 0; i < 12; ++i) lay.s[i] = s[i % 3];
  lay.cu_seqlens = cu_seqlens;
  lay.total = total;
  return run(q, k, v, o, lse, batch, heads, max_seqlen, d_k, scale, causal, dtype, 1.0f, stream, 1,
             nullptr, &lay);
}

int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                   int heads, int n, int d_k, float scale, int causal, float q_descale,
                   float k_descale, float v_descale, void* stream) {
  const int st = validate(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, FA_FP8_E4M3);
  if (st != FA_OK) return st;
  for (float s : {q_descale, k_descale, v_descale})
    if (!std::isfinite(s) || !(s > 0.f)) return FA_ERR_SCALE;
  const float qk = (float)((double)scale * q_descale * k_descale);
  if (!std::isfinite((float)(qk * kLog2e))) return FA_ERR_SCALE;
  return run(q, k, v, o, lse, batch, heads, n, d_k, qk, causal, FA_FP8_E4M3, v_descale, stream);
}

size_t fa_splitkv_workspace_size(int batch, int heads, int n, int d_k, int splits) {
  if (batch < 1 || heads < 1 || n < 1 || (d_k != 64 && d_k != 128) || splits < 1 ||
      splits > kMaxSplits)
    return 0;
  const int used = splits_used(n, splits);
  if (used <= 1) return 0;
  return split_layout(batch, heads, n, d_k, used).total;
}

int fa_splitkv_splits(int batch, int heads, int n, int causal, int compute_units) {
  if (batch < 1 || heads < 1 || n < 1 || (causal != 0 && causal != 1)) return 0;
  int cus = compute_units;
  if (cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();  // leave no error behind for a later launch check
      cus = 256;
    }
  }
  const int64_t units = (int64_t)batch * heads * ((n + 255) / 256);
  const int64_t want = (int64_t)cus * (causal ? 2 : 1);
  int splits = 1;
  while (units * splits < want && 2 * splits <= kMaxSplits && (int64_t)512 * splits <= n) splits *= 2;
  return splits;
}

int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                       int heads, int n, int d_k, float scale, int causal, int dtype, int splits,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const int st = validate(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_UNSUPPORTED;
  const int used = splits_used(n, splits);
  if (used > 1) {
    if (!workspace) return FA_ERR_NULL;
    if ((uintptr_t)workspace % 16) return FA_ERR_ALIGN;
    const size_t need = split_layout(batch, heads, n, d_k, used).total;
    if (workspace_bytes < need) return FA_ERR_SHAPE;
    const int64_t rows = (int64_t)batch * heads * n;
    if (rows > INT32_MAX) return FA_ERR_OVERFLOW;  // the merge kernel's grid
    const int in_bytes = dtype == FA_F32 ? 4 : dtype == FA_FP8_E4M3 ? 1 : 2;
    const int out_bytes = dtype == FA_F32 ? 4 : 2;
    const Range rw{(uintptr_t)workspace, (uintptr_t)workspace + need};
    const Range rq{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(rows * d_k * in_bytes)};
    const Range rk{(uintptr_t)k, (uintptr_t)k + (uintptr_t)(rows * d_k * in_bytes)};
    const Range rv{(uintptr_t)v, (uintptr_t)v + (uintptr_t)(rows * d_k * in_bytes)};
    const Range ro{(uintptr_t)o, (uintptr_t)o + (uintptr_t)(rows * d_k * out_bytes)};
    if (overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv) || overlap(rw, ro)) return FA_ERR_ALIAS;
    if (lse && overlap(rw, Range{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(rows * 4)}))
      return FA_ERR_ALIAS;
  }
  return run(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype, 1.0f, stream, splits,
             workspace);
}

size_t fa_noalloc_scratch_bytes(void) { return fa::kNoallocScratchBytes; }

int fa_forward_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int batch, int heads, int n, int d_k, float scale, int causal,
                               int dtype, int splits, void* stream) {
  const int st = validate(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_UNSUPPORTED;
  const int used = splits_used(n, splits);
  const size_t need = used > 1 ? split_layout(batch, heads, n, d_k, used).total : 0;
  if (need > fa::kNoallocScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = fa::noalloc_scratch(&ws);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return FA_ERR_HIP;
    }
  }
  return fa_forward_splitkv(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype, splits, ws, need,
                            stream);
}

size_t fa_unfused_workspace_size(int batch, int heads, int n) {
  if (batch < 1 || heads < 1 || n < 1) return 0;
  if ((double)batch * heads * (double)n * n * 6.0 > 9.0e18) return 0;
  return unf_layout(batch, heads, n).total;
}

int fa_forward_unfused(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                       int heads, int n, int d_k, float scale, int causal, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const int st = validate(q, k, v, o, lse, batch, heads, n, d_k, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!workspace) return FA_ERR_NULL;
  if ((uintptr_t)workspace % 16) return FA_ERR_ALIGN;
  if ((double)batch * heads * (double)n * n * 6.0 > 9.0e18) return FA_ERR_OVERFLOW;
  const UnfLayout ul = unf_layout(batch, heads, n);
  if (workspace_bytes < ul.total) return FA_ERR_SHAPE;
  const int64_t rows = (int64_t)batch * heads * n;
  const uintptr_t t_sz = (uintptr_t)(rows * d_k * 2);
  const Range rw{(uintptr_t)workspace, (uintptr_t)workspace + ul.total};
  const Range others[4] = {{(uintptr_t)q, (uintptr_t)q + t_sz}, {(uintptr_t)k, (uintptr_t)k + t_sz},
                           {(uintptr_t)v, (uintptr_t)v + t_sz}, {(uintptr_t)o, (uintptr_t)o + t_sz}};
  for (const Range& r : others)
    if (overlap(rw, r)) return FA_ERR_ALIAS;
  if (lse && overlap(rw, Range{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(rows * 4)})) return FA_ERR_ALIAS;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    fa::UnfArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.s = (float*)workspace;
    a.p = (uint16_t*)((char*)workspace + ul.p_off);
    a.bh = batch * heads;
    a.n = n;
    a.d = d_k;
    a.rows = (int)rows;
    a.causal = causal != 0;
    a.scale = scale;
    a.elt = static_cast<fa::Elt>(dtype);
    e = fa::launch_unfused(a, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

size_t fa_backward_workspace_size(int batch, int heads, int n) {
  if (batch < 1 || heads < 1 || n < 1) return 0;
  return bwd_layout(batch, heads, n).total;
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int n,
                int d_k, float scale, int causal, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads, n, d_k, scale,
                              causal, dtype, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads, n, d_k, scale, causal, dtype,
                 workspace, nullptr, 0, stream);
}

int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens,
                       int batch, int total, int max_seqlen, int heads, int d_k, float scale,
                       int causal, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace || !cu_seqlens)
    return FA_ERR_NULL;
  if (batch < 1 || heads < 1 || max_seqlen < 1 || total < 0) return FA_ERR_SHAPE;
  if (dtype < FA_F32 || dtype > FA_FP8_E4M3) return FA_ERR_DTYPE;
  if ((dtype != FA_F16 && dtype != FA_BF16) || (d_k != 64 && d_k != 128) ||
      (causal != 0 && causal != 1))
    return FA_ERR_UNSUPPORTED;
  for (uintptr_t p : {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)o, (uintptr_t)dout,
                      (uintptr_t)lse, (uintptr_t)dq, (uintptr_t)dk, (uintptr_t)dv,
                      (uintptr_t)workspace})
    if (p % 16) return FA_ERR_ALIGN;
  if ((uintptr_t)cu_seqlens % 4) return FA_ERR_ALIGN;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  const int64_t rs = (int64_t)heads * d_k;  // row stride, elements
  if (((int64_t)max_seqlen + 256) * rs * 2 > INT32_MAX) return FA_ERR_OVERFLOW;
  const int64_t bh = (int64_t)batch * heads;
  if (bh > kMaxGrid || bh * (((int64_t)max_seqlen + 127) / 128) > kMaxGrid) return FA_ERR_OVERFLOW;
  if ((int64_t)total * rs > (INT64_C(1) << 50)) return FA_ERR_OVERFLOW;
  const BwdLayout wl = bwd_layout(1, heads, total);
  if (workspace_bytes < wl.total) return FA_ERR_SHAPE;
  const uintptr_t t_sz = (uintptr_t)(total * rs * 2);
  const Range ins[7] = {{(uintptr_t)q, (uintptr_t)q + t_sz},       {(uintptr_t)k, (uintptr_t)k + t_sz},
                        {(uintptr_t)v, (uintptr_t)v + t_sz},       {(uintptr_t)o, (uintptr_t)o + t_sz},
                        {(uintptr_t)dout, (uintptr_t)dout + t_sz},
                        {(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)((int64_t)heads * total * 4)},
                        {(uintptr_t)cu_seqlens, (uintptr_t)cu_seqlens + (uintptr_t)(batch + 1) * 4}};
  const Range outs[4] = {{(uintptr_t)dq, (uintptr_t)dq + t_sz},
                         {(uintptr_t)dk, (uintptr_t)dk + t_sz},
                         {(uintptr_t)dv, (uintptr_t)dv + t_sz},
                         {(uintptr_t)workspace, (uintptr_t)workspace + wl.total}};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
  }
  if (total == 0) return FA_OK;  // no rows: nothing to compute
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads, max_seqlen, d_k, scale, causal,
                 dtype, workspace, cu_seqlens, total, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "batch, heads and n must be >= 1 (or workspace too small)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_UNSUPPORTED: return "unsupported d_k (64 or 128), causal flag (0 or 1), split count or backward dtype";
    case FA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FA_ERR_SCALE: return "scale not finite (or scale * log2(e) overflows), or a descale not finite and positive";
    case FA_ERR_ALIAS: return "an output or workspace overlaps an input or another output";
    case FA_ERR_OVERFLOW: return "problem exceeds the kernel's index or grid range";
    case FA_ERR_HIP: return "HIP runtime error (see fa_last_hip_error)";
    case FA_ERR_SCRATCH: return "split-KV partials exceed the fixed scratch of fa_forward_splitkv_noalloc (see fa_noalloc_scratch_bytes)";
    default: return "unknown status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

int fa_abi_version(void) { return kAbiVersion; }

}  // extern "C"
