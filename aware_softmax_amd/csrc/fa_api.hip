// C-ABI entry points of libfa.so: argument validation, kernel selection,
// launch on the caller's stream.  Declarations and contracts: include/fa.h.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace {

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

// The hipError_t behind the last FA_ERR_HIP returned on this thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

fa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = e;
  return FA_ERR_HIP;
}

// A launch's work-items in x must fit in 32 bits.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;

size_t elem_size(fa_dtype_t dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

bool is_16bit(fa_dtype_t dtype) { return dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16; }

// Head dims of the forward: 16-bit 32, 64, 96, 128, 256; fp32 32, 64, 96, 128.
fa_status_t check_dtype_headdim(int d, fa_dtype_t dtype) {
  if (dtype != FA_DTYPE_F32 && !is_16bit(dtype)) return FA_ERR_DTYPE;
  const bool ok = d == 32 || d == 64 || d == 96 || d == 128 || (d == 256 && is_16bit(dtype));
  return ok ? FA_OK : FA_ERR_UNSUPPORTED_HEADDIM;
}

// Head dims of the backward kernels.
bool bwd_headdim(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: sizes must be positive, consistent and within the supported range";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype is not supported by this entry point";
    case FA_ERR_UNSUPPORTED_HEADDIM: return "FA_ERR_UNSUPPORTED_HEADDIM: this entry point and dtype do not support this head dim";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: q/k/v/o must be 16-byte and lse 4-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP kernel launch failed";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or another output";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace is NULL, not 256-byte aligned or smaller than the size the call needs";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: the problem needs more scratch than the static array of fa_decode_static holds (FA_DECODE_STATIC_SCRATCH_BYTES)";
  }
  return "unknown fa_status_t";
}

const char* fa_version(void) { return "0.4.0 gfx950"; }

int fa_last_hip_error(const char** message) {
  if (message) *message = hipGetErrorString(g_last_hip_error);
  return (int)g_last_hip_error;
}

fa_status_t fa_fwd_tile(int d, fa_dtype_t dtype, int* block_q, int* block_k, int* waves) {
  if (!block_q || !block_k || !waves) return FA_ERR_NULL;
  const fa_status_t st = check_dtype_headdim(d, dtype);
  if (st != FA_OK) return st;
  const fa::TileConfig t = is_16bit(dtype) ? fa::mfma_tile(d) : fa::f32_tile(d);
  *block_q = t.block_q;
  *block_k = t.block_k;
  *waves = t.waves;
  return FA_OK;
}

fa_status_t fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                       int N, int d, int causal, float scale, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  const fa_status_t st = check_dtype_headdim(d, dtype);
  if (st != FA_OK) return st;
  // Sizes: element offsets are 64-bit in the kernels; the grid is one int.
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  const int64_t elems = bh * N * d;
  if (elems > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  const fa::TileConfig tile = is_16bit(dtype) ? fa::mfma_tile(d) : fa::f32_tile(d);
  const int64_t nqb = ((int64_t)N + tile.block_q - 1) / tile.block_q;
  if (bh * nqb * 64 * tile.waves > kMaxWorkItems) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) != 0 || ((uintptr_t)lse & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t tbytes = (size_t)elems * elem_size(dtype);
  const size_t kvbytes = (size_t)B * Hkv * N * d * elem_size(dtype);
  const size_t lbytes = (size_t)bh * N * sizeof(float);
  if (ranges_overlap(o, tbytes, q, tbytes) || ranges_overlap(o, tbytes, k, kvbytes) ||
      ranges_overlap(o, tbytes, v, kvbytes) || ranges_overlap(o, tbytes, lse, lbytes) ||
      ranges_overlap(lse, lbytes, q, tbytes) || ranges_overlap(lse, lbytes, k, kvbytes) ||
      ranges_overlap(lse, lbytes, v, kvbytes))
    return FA_ERR_ALIAS;

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)bh;
  p.N = N;
  p.d = d;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.group = H / Hkv;
  const hipError_t e = dtype == FA_DTYPE_BF16  ? fa::launch_fwd_bf16(p, stream)
                       : dtype == FA_DTYPE_F16 ? fa::launch_fwd_f16(p, stream)
                                               : fa::launch_fwd_f32(p, stream);
  return hip_status(e);
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                       int N, int d, int causal, float scale, float q_descale, float k_descale, float v_descale,
                       hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEADDIM;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  const int64_t elems = bh * N * d;
  if (elems > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  const fa::TileConfig tile = fa::mfma_tile(64);  // the fp8 kernel's workgroup shape (128 rows, 4 or 8 waves)
  const int64_t nqb = ((int64_t)N + tile.block_q - 1) / tile.block_q;
  if (bh * nqb * 64 * 2 * tile.waves > kMaxWorkItems) return FA_ERR_SHAPE;
  if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale) ||
      !(q_descale > 0.f) || !(k_descale > 0.f) || !(v_descale > 0.f))
    return FA_ERR_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) != 0 || ((uintptr_t)lse & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t qbytes = (size_t)elems;                      // e4m3: one byte per element
  const size_t kvbytes = (size_t)B * Hkv * N * d;
  const size_t obytes = (size_t)elems * 2;                  // bf16 output
  const size_t lbytes = (size_t)bh * N * sizeof(float);
  if (ranges_overlap(o, obytes, q, qbytes) || ranges_overlap(o, obytes, k, kvbytes) ||
      ranges_overlap(o, obytes, v, kvbytes) || ranges_overlap(o, obytes, lse, lbytes) ||
      ranges_overlap(lse, lbytes, q, qbytes) || ranges_overlap(lse, lbytes, k, kvbytes) ||
      ranges_overlap(lse, lbytes, v, kvbytes))
    return FA_ERR_ALIAS;

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)bh;
  p.N = N;
  p.d = d;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.group = H / Hkv;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  return hip_status(fa::launch_fwd_fp8(p, stream));
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, int causal, float scale, fa_dtype_t dtype, hipStream_t stream) {
  return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, stream);
}

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                          int B, int H, int Hkv, int total, int max_seqlen, int d, int causal, float scale,
                          fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hkv <= 0 || total <= 0 || max_seqlen <= 0 || d <= 0 || H % Hkv != 0)
    return FA_ERR_SHAPE;
  if (!is_16bit(dtype)) return FA_ERR_DTYPE;
  const fa_status_t st = check_dtype_headdim(d, dtype);
  if (st != FA_OK) return st;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX || max_seqlen > total) return FA_ERR_SHAPE;
  const int64_t elems = (int64_t)H * total * d;
  if (elems > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  const fa::TileConfig tile = fa::mfma_tile(d);
  const int64_t nqb = ((int64_t)max_seqlen + tile.block_q - 1) / tile.block_q;
  if (bh * nqb * 64 * tile.waves > kMaxWorkItems) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) != 0 ||
      (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t tbytes = (size_t)elems * 2;
  const size_t kvbytes = (size_t)Hkv * total * d * 2;
  const size_t lbytes = (size_t)H * total * sizeof(float);
  const size_t cbytes = (size_t)(B + 1) * sizeof(int);
  const void* ins[4] = {q, k, v, cu_seqlens};
  const size_t in_bytes[4] = {tbytes, kvbytes, kvbytes, cbytes};
  void* outs[2] = {o, lse};
  const size_t out_bytes[2] = {tbytes, lbytes};
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 4; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_ALIAS;
  if (ranges_overlap(o, tbytes, lse, lbytes)) return FA_ERR_ALIAS;

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)bh;
  p.N = max_seqlen;
  p.d = d;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.group = H / Hkv;
  p.cu_seqlens = cu_seqlens;
  p.H = H;
  p.total = total;
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(p, stream) : fa::launch_fwd_f16(p, stream);
  return hip_status(e);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || !bwd_headdim(d)) return 0;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX || bh * N * d > ((int64_t)1 << 40)) return 0;
  return fa::bwd_workspace_bytes((int)bh, N, d);
}

fa_status_t fa_bwd_tile(int d, int* block_k, int* block_q) {
  if (!block_k || !block_q) return FA_ERR_NULL;
  if (!bwd_headdim(d)) return FA_ERR_UNSUPPORTED_HEADDIM;
  *block_k = fa::bwd_block_k();
  *block_q = fa::bwd_block_q();
  return FA_OK;
}

fa_status_t fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                       int H, int Hkv, int N, int d, int causal, float scale, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || H % Hkv != 0) return FA_ERR_SHAPE;
  if (!is_16bit(dtype)) return FA_ERR_DTYPE;
  if (!bwd_headdim(d)) return FA_ERR_UNSUPPORTED_HEADDIM;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX) return FA_ERR_SHAPE;
  const int64_t elems = bh * N * d;
  if (elems > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  // The largest grid: one 256-thread workgroup per (query head, 128-row
  // block), two at d = 256 (one per half of the dK, dV columns).
  const int64_t nkb = ((int64_t)N + fa::bwd_block_k() - 1) / fa::bwd_block_k();
  if (bh * nkb * (d == 256 ? 2 : 1) * 256 > kMaxWorkItems) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
        (uintptr_t)dk | (uintptr_t)dv) & 15u) != 0 || ((uintptr_t)lse & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t stats = fa::bwd_workspace_bytes((int)bh, N, d);
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < stats) return FA_ERR_WORKSPACE;
  // a workspace of fa_bwd_gqa_workspace_bytes also holds the partials of
  // the head-split dK/dV pass
  const int hsplit = fa::bwd_head_split(B, H, Hkv, N);
  const size_t big = hsplit > 1 ? fa::bwd_gqa_workspace_bytes(B, H, Hkv, N, d) : stats;
  const bool split = hsplit > 1 && workspace_bytes >= big;
  const size_t need = split ? big : stats;
  const size_t tb = (size_t)elems * 2;
  const size_t kvb = (size_t)B * Hkv * N * d * 2;
  const size_t lb = (size_t)bh * N * sizeof(float);
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_bytes[6] = {tb, kvb, kvb, tb, tb, lb};
  void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_bytes[4] = {tb, kvb, kvb, need};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.workspace = workspace;
  p.BH = (int)bh;
  p.N = N;
  p.d = d;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.group = H / Hkv;
  if (split) {
    p.hsplit = hsplit;
    p.part = (float*)((char*)workspace + fa::bwd_part_offset(stats));
  }
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_bwd_bf16(p, stream) : fa::launch_bwd_f16(p, stream);
  return hip_status(e);
}

size_t fa_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || H % Hkv != 0 || !bwd_headdim(d)) return 0;
  if ((int64_t)B * H > INT_MAX || (int64_t)B * H * N * d > ((int64_t)1 << 40)) return 0;
  return fa::bwd_gqa_workspace_bytes(B, H, Hkv, N, d);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   int causal, float scale, fa_dtype_t dtype, hipStream_t stream) {
  return fa_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, d, causal, scale,
                    dtype, stream);
}

size_t fa_bwd_varlen_workspace_bytes(int H, int total, int d) {
  if (H <= 0 || total <= 0 || !bwd_headdim(d)) return 0;
  if ((int64_t)H * total * d > ((int64_t)1 << 40) || total > INT_MAX - 128) return 0;
  return fa::bwd_varlen_workspace_bytes(H, total, d);
}

fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, const int* cu_seqlens, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, int B, int H, int Hkv, int total, int max_seqlen, int d,
                          int causal, float scale, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !cu_seqlens || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hkv <= 0 || total <= 0 || max_seqlen <= 0 || d <= 0 || H % Hkv != 0)
    return FA_ERR_SHAPE;
  if (!is_16bit(dtype)) return FA_ERR_DTYPE;
  if (!bwd_headdim(d)) return FA_ERR_UNSUPPORTED_HEADDIM;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX || max_seqlen > total || total > INT_MAX - 128) return FA_ERR_SHAPE;
  const int64_t elems = (int64_t)H * total * d;
  if (elems > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  const int64_t nkb = ((int64_t)max_seqlen + fa::bwd_block_k() - 1) / fa::bwd_block_k();
  if (bh * nkb * (d == 256 ? 2 : 1) * 256 > kMaxWorkItems) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
        (uintptr_t)dk | (uintptr_t)dv) & 15u) != 0 || (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t need = fa::bwd_varlen_workspace_bytes(H, total, d);
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const size_t tb = (size_t)elems * 2;
  const size_t kvb = (size_t)Hkv * total * d * 2;
  const size_t lb = (size_t)H * total * sizeof(float);
  const void* ins[7] = {q, k, v, o, dout, lse, cu_seqlens};
  const size_t in_bytes[7] = {tb, kvb, kvb, tb, tb, lb, (size_t)(B + 1) * sizeof(int)};
  void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_bytes[4] = {tb, kvb, kvb, need};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 7; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.workspace = workspace;
  p.BH = (int)bh;
  p.N = max_seqlen;
  p.d = d;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.group = H / Hkv;
  p.cu_seqlens = cu_seqlens;
  p.H = H;
  p.total = total;
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_bwd_bf16(p, stream) : fa::launch_bwd_f16(p, stream);
  return hip_status(e);
}

fa_status_t fa_decode_plan(int B, int H, int Hkv, int N, int d, int num_splits, int* splits, int* chunk_keys,
                           size_t* workspace_bytes) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || num_splits < 0) return FA_ERR_SHAPE;
  if (H % Hkv != 0 || N > (1 << 30)) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED_HEADDIM;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX || (int64_t)B * Hkv * N * d > ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  const fa::DecodePlan pl = fa::decode_plan(B, H, Hkv, N, d, num_splits);
  if (pl.split_wgs * 256 > kMaxWorkItems) return FA_ERR_SHAPE;
  if (splits) *splits = pl.splits;
  if (chunk_keys) *chunk_keys = pl.chunk;
  if (workspace_bytes) *workspace_bytes = pl.workspace_bytes;
  return FA_OK;
}

size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int N, int d, int num_splits) {
  size_t ws = 0;
  return fa_decode_plan(B, H, Hkv, N, d, num_splits, nullptr, nullptr, &ws) == FA_OK ? ws : 0;
}

}  // extern "C"

namespace {

// fa_decode and fa_decode_static: validation (no HIP call), then the launch
// with the caller's workspace or, when static_scratch is set, the library's
// static scratch array of the current device.
fa_status_t decode_impl(const void* q, const void* k, const void* v, const int* cache_seqlens, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, bool static_scratch, int B, int H,
                        int Hkv, int N, int d, float scale, int num_splits, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  size_t need = 0;
  const fa_status_t st = fa_decode_plan(B, H, Hkv, N, d, num_splits, nullptr, nullptr, &need);
  if (st != FA_OK) return st;
  if (!is_16bit(dtype)) return FA_ERR_DTYPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) != 0 ||
      (((uintptr_t)lse | (uintptr_t)cache_seqlens) & 3u) != 0)
    return FA_ERR_ALIGN;
  if (static_scratch) {
    if (need > FA_DECODE_STATIC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  } else if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need) {
    return FA_ERR_WORKSPACE;
  }
  const size_t qb = (size_t)B * H * d * 2;
  const size_t kb = (size_t)B * Hkv * N * d * 2;
  const size_t lb = (size_t)B * H * sizeof(float);
  const void* ins[4] = {q, k, v, cache_seqlens};
  const size_t in_bytes[4] = {qb, kb, kb, cache_seqlens ? (size_t)B * sizeof(int) : 0};
  void* outs[3] = {o, lse, workspace};
  const size_t out_bytes[3] = {qb, lb, static_scratch ? 0 : need};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 4; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 3; ++b)
      if (ranges_overlap(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }
  if (static_scratch) {
    const hipError_t e = fa::decode_static_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e);
  }

  fa::DecodeParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.seqlens = cache_seqlens;
  p.o = o;
  p.lse = lse;
  p.workspace = workspace;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.num_splits = num_splits;
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_decode_bf16(p, stream) : fa::launch_decode_f16(p, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

fa_status_t fa_decode(const void* q, const void* k, const void* v, const int* cache_seqlens, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N, int d, float scale,
                      int num_splits, fa_dtype_t dtype, hipStream_t stream) {
  return decode_impl(q, k, v, cache_seqlens, o, lse, workspace, workspace_bytes, false, B, H, Hkv, N, d, scale,
                     num_splits, dtype, stream);
}

fa_status_t fa_decode_static(const void* q, const void* k, const void* v, const int* cache_seqlens, void* o,
                             float* lse, int B, int H, int Hkv, int N, int d, float scale, int num_splits,
                             fa_dtype_t dtype, hipStream_t stream) {
  return decode_impl(q, k, v, cache_seqlens, o, lse, nullptr, 0, true, B, H, Hkv, N, d, scale, num_splits, dtype,
                     stream);
}

fa_status_t fa_mfma_ceiling(float* sink, int iters, int blocks, int store, hipStream_t stream) {
  if (!sink) return FA_ERR_NULL;
  if (iters <= 0 || blocks <= 0 || (int64_t)blocks * 256 > kMaxWorkItems) return FA_ERR_SHAPE;
  if ((uintptr_t)sink % 4 != 0) return FA_ERR_ALIGN;
  return hip_status(fa::launch_mfma_ceiling(sink, iters, blocks, store, stream));
}

}  // extern "C"
