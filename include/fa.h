/*
 * fa.h -- C ABI of the fused exact-attention library (libfa.so, gfx950).
 *
 * The library computes, for every (batch b, head h),
 *     O = softmax(scale * Q K^T + mask) V     and     L = rowwise logsumexp
 * with the FlashAttention-2 forward: tiled over query blocks, keys and
 * values streamed through on-chip memory, running max m, running sum l and
 * an unnormalised accumulator rescaled by alpha = exp(m - m'), one division
 * by l at the end, and the N x N score matrix never written to memory.
 * Sources (page title and section):
 *   "FlashAttention-2: Why the Attention Bottleneck Wasn't Where Everyone
 *    Was Looking" -- "The hook" (the computed quantity), "FA2 change #1"
 *    (deferred division, L = m + log l), "FA2 change #2" (parallel over
 *    query blocks), "The causal masking freebie" (block classification);
 *   "FlashAttention: Move Less, Not Compute Less" -- "Tiling Is Easy;
 *    Softmax Couples the Entire Row" (online recurrences);
 *   "PidokuInfra 10 -- FlashAttention" -- section 4 (causal: query i sees
 *    keys 0..i; scale 1/sqrt(d) applied to QK^T before the softmax).
 *
 * Conventions shared by every entry point:
 *   - q, k, v, o are device pointers to contiguous row-major [B][H][N][d]
 *     tensors of the given dtype; lse is a device pointer to a contiguous
 *     [B][H][N] float32 tensor for both dtypes.
 *   - L is the natural-log logsumexp of the scaled, masked score row
 *     (L_i = m_i + ln l_i).
 *   - The causal mask is top-left aligned: query i attends to keys 0..i.
 *   - The caller owns all memory.  Nothing is allocated or freed, no state
 *     is kept between calls (calls are thread-safe and re-entrant), and no
 *     call synchronises: work is enqueued on `stream` (0 = the null stream)
 *     and the call returns.  Device-side faults surface at the caller's
 *     next synchronisation.
 *   - Arguments are validated before any HIP call; on a nonzero status no
 *     work has been enqueued.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_F32 = 0,  /* float32 in, float32 out, fp32 arithmetic */
  FA_DTYPE_BF16 = 1, /* bfloat16 in/out, fp32 accumulation and softmax */
  FA_DTYPE_F16 = 2   /* float16 in/out, fp32 accumulation and softmax */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,                 /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,                /* a size <= 0, sizes too large, or inconsistent */
  FA_ERR_DTYPE = 3,                /* dtype is not a fa_dtype_t value */
  FA_ERR_UNSUPPORTED_HEADDIM = 4,  /* d is not supported by the entry point for this dtype */
  FA_ERR_ALIGN = 5,                /* q/k/v/o not 16-byte or lse not 4-byte aligned */
  FA_ERR_SCALE = 6,                /* scale is NaN or infinite */
  FA_ERR_HIP = 7,                  /* the HIP launch reported an error */
  FA_ERR_ALIAS = 8,                /* an output overlaps an input or another output */
  FA_ERR_WORKSPACE = 9,            /* workspace missing, misaligned or too small */
  FA_ERR_SCRATCH = 10              /* the problem needs more than the library's static scratch */
} fa_status_t;

/* Size of the static device scratch array behind fa_decode_static. */
#define FA_DECODE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa_fwd -- attention forward for all B*H heads.
 *
 *   q, k, v  [in]  device, [B][H][N][d] of dtype, 16-byte aligned.
 *   o        [out] device, [B][H][N][d] of dtype, 16-byte aligned; must not
 *                  overlap q, k, v or lse.
 *   lse      [out] device, [B][H][N] float32, 4-byte aligned.
 *   B, H, N  sizes (> 0); any N >= 1 (ragged tails are masked).
 *   d        head dimension: 32, 64, 96, 128 or 256 for bf16 and fp16;
 *            32, 64, 96 or 128 for fp32 ("PidokuInfra 10 -- FlashAttention",
 *            sections 8-9: kernels commonly cover 64, 96, 128 and 256).
 *   causal   0: every query sees all N keys; nonzero: query i sees 0..i.
 *   scale    multiplies Q K^T before mask and softmax (finite; 1/sqrt(d)
 *            in the usual case; 0 and negative values are allowed).
 *   dtype    FA_DTYPE_BF16 or FA_DTYPE_F16 (MFMA path; P is rounded to the
 *            input type for the P.V product) or FA_DTYPE_F32 (fp32 path).
 *   stream   HIP stream the kernel is enqueued on.
 * Returns FA_OK or the first failed check (see fa_status_t).  The output
 * is deterministic: the same inputs give bitwise identical o and lse.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_fwd_gqa -- fa_fwd with grouped key/value heads: k and v are
 * [B][Hkv][N][d] and query head h reads key/value head h / (H / Hkv)
 * (Hkv = 1: one key/value head for all query heads; Hkv = H: fa_fwd).
 * "FlashAttention: Move Less, Not Compute Less", "What It Changes--and
 * What It Does Not": GQA cuts the number of key/value heads, and the
 * reference implementation carries GQA/MQA paths next to the causal one;
 * the sharing changes only which K and V tiles a workgroup streams.  q, o, lse and every other argument as for fa_fwd; H must be a
 * multiple of Hkv (else FA_ERR_SHAPE).
 */
fa_status_t fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, int causal, float scale,
                       fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_fwd_fp8 -- the forward on 8-bit inputs ("FlashAttention: Move Less,
 * Not Compute Less", section "FA1 to FA3", names FP8 as the next step;
 * the pages fix no quantisation, so this entry point takes the plainest
 * one): q, k, v hold OCP FP8 E4M3 bytes (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; 0x7F / 0xFF are NaN; largest finite 448), and each
 * tensor has one dequantisation factor, so element x means byte(x) times
 * its tensor's factor.  The result is the attention of the dequantised
 * tensors, as fa_fwd_gqa computes it: S = scale (q_descale q)(k_descale k)^T
 * with exact products and fp32 sums, P rounded to bf16 for P.V, V
 * dequantised exactly to bf16, O = v_descale P V / l.
 *   q         [in]  device, [B][H][N][d] e4m3 bytes, 16-byte aligned.
 *   k, v      [in]  device, [B][Hkv][N][d] e4m3 bytes, 16-byte aligned.
 *   o         [out] device, [B][H][N][d] bf16, 16-byte aligned.
 *   lse       [out] device, [B][H][N] float32 (natural log), 4-byte aligned.
 *   d         64 or 128 (else FA_ERR_UNSUPPORTED_HEADDIM).
 *   q_descale, k_descale, v_descale  finite and > 0 (else FA_ERR_SCALE).
 *   the other arguments and checks as for fa_fwd_gqa (outputs must not
 *   overlap the inputs or each other: FA_ERR_ALIAS).
 * Allocates nothing; one kernel is enqueued on `stream`.
 */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, int causal, float scale,
                       float q_descale, float k_descale, float v_descale, hipStream_t stream);

/*
 * fa_fwd_varlen -- the forward over a batch of B sequences of different
 * lengths packed without padding ("FlashAttention: Move Less, Not Compute
 * Less", "What It Changes--and What It Does Not": the reference
 * implementation has variable-length paths; "PidokuInfra 10 --
 * FlashAttention", sections 8-9: padding sequences instead wastes the
 * kernel's work).  Every head holds the `total` rows of all sequences one
 * after another; sequence b is rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1
 * and attends only within itself (causal: row i of the sequence sees its
 * rows 0..i).
 *
 *   q, o        [in]/[out] device, [H][total][d] of dtype, 16-byte aligned.
 *   k, v        [in]  device, [Hkv][total][d] of dtype, 16-byte aligned
 *               (query head h reads key/value head h / (H / Hkv)).
 *   lse         [out] device, [H][total] float32, 4-byte aligned.
 *   cu_seqlens  [in]  device, B + 1 int32, 4-byte aligned: 0 =
 *               cu_seqlens[0] <= cu_seqlens[1] <= ... <= cu_seqlens[B] =
 *               total.  Read only by the kernel (the host never waits for
 *               it); offsets are clamped to [0, total] on the device, so
 *               malformed offsets cannot address memory outside the
 *               tensors, but their results are undefined.
 *   max_seqlen  the longest sequence (1 <= max_seqlen <= total); rows of a
 *               longer sequence past max_seqlen are not written.
 *   dtype       FA_DTYPE_BF16 or FA_DTYPE_F16.
 *   d, causal, scale, stream   as for fa_fwd.
 * Empty sequences are allowed.  Returns FA_OK or the first failed check.
 */
fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen,
                          int d, int causal, float scale, fa_dtype_t dtype, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* fa_status_string(fa_status_t status);

/*
 * fa_fwd_tile -- the tile configuration fa_fwd uses for (d, dtype):
 * query rows per workgroup, keys per streamed tile and wavefronts per
 * workgroup, as launched on large grids (16-bit: 256 rows and 8 waves for
 * d = 32 to 128, 128 rows and 8 waves at d = 256; fp32: 128 rows, 4
 * waves).  On small grids (at most 1024 workgroups of 128 rows) d <= 96
 * runs two wave groups splitting the keys of each 128-row block (8 waves;
 * at d = 96 only where 256-row blocks would leave compute units idle), and
 * fp32 grids of at most 256 blocks of 64 rows run 16- or 32-row blocks.
 * Host-only; makes no HIP call.  Returns FA_OK or
 * FA_ERR_NULL / FA_ERR_DTYPE / FA_ERR_UNSUPPORTED_HEADDIM.
 */
fa_status_t fa_fwd_tile(int d, fa_dtype_t dtype, int* block_q, int* block_k, int* waves);

/*
 * fa_bwd_workspace_bytes -- size of the device workspace fa_bwd needs for
 * these sizes: two fp32 [B][H][Npad] row vectors (the row statistics D and
 * L / scale of every query), Npad = N rounded up to a multiple of 64.
 * Host-only; makes no HIP call.  Returns 0 for non-positive sizes or an
 * unsupported head dimension.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd_gqa_workspace_bytes -- the workspace with which fa_bwd_gqa (and
 * fa_bwd) may split the query heads of each key/value-head group over
 * several workgroups of the dK/dV pass ("FA2 change #2" parallelises that
 * pass over key blocks; with grouped heads a key block also sums over the
 * group's heads, and on small grids the heaviest causal blocks would
 * otherwise set the run time).  It is fa_bwd_workspace_bytes(B, H, N, d)
 * rounded up to 256 bytes plus fp32 partial dK and dV for each head
 * subset, or exactly fa_bwd_workspace_bytes when these sizes do not split
 * (a group of odd size, or more than 256 dK/dV workgroups).  Passing at
 * least this many bytes enables the split; passing fa_bwd_workspace_bytes
 * keeps the one-workgroup-per-key-block pass.  Either way the result is
 * deterministic.  Host-only; 0 for invalid sizes or head dimension.
 */
size_t fa_bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d);

/*
 * fa_bwd -- attention backward for all B*H heads: given the upstream
 * gradient dO of O, writes dQ, dK and dV.
 *
 * "FlashAttention: Move Less, Not Compute Less", "Why More Arithmetic Can
 * Finish Sooner": the backward does not read a stored S or P; it rebuilds
 * P = exp(scale Q K^T + mask - L) tile by tile on chip from Q, K and the
 * row statistic L of the forward ("FlashAttention-2: ...", "FA2 change #1").
 * With D_i = dO_i . O_i and dS = P * (dO V^T - D):
 *     dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
 * "FA2 change #2", last paragraph, splits the work over key columns (each
 * worker owning dK_j, dV_j) and accumulates dQ with atomic adds; here dK
 * and dV are formed that way, and dQ by a second, query-parallel pass that
 * rebuilds P and dP for its rows instead of atomics (no atomics at all).
 *
 *   q, k, v, o, dout  [in]  device, [B][H][N][d] of dtype, 16-byte aligned; o is
 *                     the forward output for the same q, k, v, causal, scale.
 *   lse       [in]  device, [B][H][N] float32 (the forward's L), 4-byte aligned.
 *   dq, dk, dv [out] device, [B][H][N][d] of dtype, 16-byte aligned; must not
 *                     overlap each other, the inputs or the workspace.
 *   workspace [scratch] device, at least fa_bwd_workspace_bytes(B, H, N, d)
 *                     bytes (passed as workspace_bytes), 256-byte aligned,
 *                     owned by the caller; overwritten, contents undefined
 *                     afterwards.  It needs no initialisation.
 *   B, H, N, causal, scale   as for fa_fwd.
 *   d         head dimension: 32, 64, 96, 128 or 256 (else
 *             FA_ERR_UNSUPPORTED_HEADDIM).  At 256 the dK/dV pass runs
 *             two workgroups per key block, one per half of the columns,
 *             each rebuilding S and dP over the full d ("PidokuInfra 10 --
 *             FlashAttention", section 5: the on-chip budget of a d = 256
 *             tile).
 *   dtype     FA_DTYPE_BF16 or FA_DTYPE_F16 (P and dS are rounded to it for
 *             the MFMAs); FA_DTYPE_F32 returns FA_ERR_DTYPE.
 *   stream    HIP stream; three kernels are enqueued in order on it.
 * Returns FA_OK or the first failed check.  The outputs are deterministic:
 * the same inputs give bitwise identical dq, dk and dv.
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, int causal, float scale, fa_dtype_t dtype,
                   hipStream_t stream);

/*
 * fa_bwd_gqa -- fa_bwd with grouped key/value heads (the layouts of
 * fa_fwd_gqa): k, v [in] and dk, dv [out] are [B][Hkv][N][d]; q, o, dout,
 * dq are [B][H][N][d] and lse [B][H][N].  dK and dV of a key/value head
 * are the sums over the H / Hkv query heads that read it (the chain rule
 * through the shared K and V); they are summed on chip by the workgroup
 * that owns the key block, so the result stays free of atomics and
 * deterministic.  Every other argument as for fa_bwd; H must be a
 * multiple of Hkv (else FA_ERR_SHAPE).  With a workspace of at least
 * fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d) bytes on a small grid the
 * heads of a group may be split over several dK/dV workgroups that write
 * fp32 partial sums to the workspace; a fourth kernel then adds the
 * partials in a fixed order and rounds once (four kernels are enqueued
 * instead of three).
 */
fa_status_t fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       int B, int H, int Hkv, int N, int d, int causal, float scale, fa_dtype_t dtype,
                       hipStream_t stream);

/*
 * fa_bwd_varlen_workspace_bytes -- the workspace of fa_bwd_varlen: two
 * fp32 [H][ld] row vectors, ld = total rounded up to 64, plus 64.  Host-only;
 * 0 for invalid sizes.
 */
size_t fa_bwd_varlen_workspace_bytes(int H, int total, int d);

/*
 * fa_bwd_varlen -- the backward of fa_fwd_varlen (same packed layouts,
 * cu_seqlens and max_seqlen): q, o, dout, dq [H][total][d]; k, v, dk, dv
 * [Hkv][total][d]; lse [H][total]; every sequence's gradients depend only
 * on its own rows.  workspace: at least fa_bwd_varlen_workspace_bytes(H,
 * total, d) bytes, 256-byte aligned.  dtype FA_DTYPE_BF16 or FA_DTYPE_F16;
 * d 32, 64, 96, 128 or 256; the other arguments and the checks as for fa_bwd_gqa and
 * fa_fwd_varlen (cu_seqlens clamped to [0, total] on the device).
 */
fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, const int* cu_seqlens, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int total,
                          int max_seqlen, int d, int causal, float scale, fa_dtype_t dtype,
                          hipStream_t stream);

/*
 * fa_bwd_tile -- keys per workgroup of the dK/dV pass and queries per
 * streamed tile of it.  Host-only.  Returns FA_OK or FA_ERR_NULL /
 * FA_ERR_UNSUPPORTED_HEADDIM.
 */
fa_status_t fa_bwd_tile(int d, int* block_k, int* block_q);

/*
 * Decode: one new query row per sequence against a cache of N keys and
 * values ("PidokuInfra 10 -- FlashAttention", section 5, "The decode
 * variant: FlashDecoding").  Query head h of batch b attends to every key
 * of key/value head h / (H / Hkv) (Hkv = H: multi-head; Hkv < H: groups of
 * H / Hkv query heads share one key/value head); there is no mask (the new
 * token is the last position and sees the whole cache).  The keys are split
 * into chunks processed by separate workgroups, each producing an
 * unnormalised partial (m, l, o~); a second kernel merges the partials with
 * the online-softmax rescale and divides once.
 *
 * Layouts: q, o contiguous [B][H][d]; k, v contiguous [B][Hkv][N][d]; lse
 * contiguous [B][H] float32 (natural-log logsumexp of the scaled scores).
 */

/*
 * fa_decode_plan -- the split fa_decode uses for these sizes.
 *   num_splits  0 picks the count automatically (enough workgroups to fill
 *               the GPU); n > 0 asks for n splits, reduced to the number of
 *               key chunks of one workgroup iteration if larger (1 gives the
 *               unsplit kernel: one workgroup walks all N keys).
 *   splits, chunk_keys, workspace_bytes  [out] the split count, keys per
 *               split (the last split may be shorter) and the workspace
 *               fa_decode needs.  Any of them may be NULL.
 * Host-only.  Returns FA_OK, FA_ERR_SHAPE (a size <= 0, H not a multiple of
 * Hkv, N > 2^30, num_splits < 0, or sizes too large), or
 * FA_ERR_UNSUPPORTED_HEADDIM.
 */
fa_status_t fa_decode_plan(int B, int H, int Hkv, int N, int d, int num_splits, int* splits,
                           int* chunk_keys, size_t* workspace_bytes);

/* fa_decode_workspace_bytes -- the workspace of fa_decode_plan, 0 on error. */
size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int N, int d, int num_splits);

/*
 * fa_decode -- split-K decode attention.
 *   q         [in]  device, [B][H][d] of dtype, 16-byte aligned.
 *   k, v      [in]  device, [B][Hkv][N][d] of dtype, 16-byte aligned: a
 *             cache of capacity N per sequence.
 *   cache_seqlens [in] device, B int32, 4-byte aligned, or NULL: sequence
 *             b attends to the first cache_seqlens[b] rows of its cache
 *             (clamped to [0, N] on the device); NULL means all N.  A
 *             sequence with no key gets o = 0 and lse = -inf.
 *   o         [out] device, [B][H][d] of dtype, 16-byte aligned.
 *   lse       [out] device, [B][H] float32, 4-byte aligned.
 *   workspace [scratch] device, at least fa_decode_workspace_bytes(...)
 *             bytes (passed as workspace_bytes), 256-byte aligned, owned by
 *             the caller; overwritten, needs no initialisation.
 *   B, H, Hkv, N, d   batch, query heads, key/value heads (H % Hkv == 0),
 *             cached keys (1 <= N <= 2^30), head dim (32, 64, 96, 128
 *             or 256).
 *   scale     finite; multiplies q . k.
 *   num_splits  as for fa_decode_plan.
 *   dtype     FA_DTYPE_BF16 or FA_DTYPE_F16 (fp32 products and softmax).
 *   stream    HIP stream; two kernels are enqueued in order on it.
 * Outputs must not overlap each other, the inputs or the workspace
 * (FA_ERR_ALIAS).  No atomics: results are deterministic for a given split.
 * Returns FA_OK or the first failed check.
 */
fa_status_t fa_decode(const void* q, const void* k, const void* v, const int* cache_seqlens, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N, int d,
                      float scale, int num_splits, fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_decode_static -- fa_decode without a workspace argument and without
 * any allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The split partials go to a static device array of
 * FA_DECODE_STATIC_SCRATCH_BYTES (16 MiB) that the library holds on every
 * device it runs on until the process ends; its device address is looked
 * up once per device (hipGetSymbolAddress) on the first call there.
 *   Arguments, layouts, checks and results as for fa_decode (the same
 *   kernels and split plan: outputs are bitwise those of fa_decode with
 *   the same num_splits), minus workspace / workspace_bytes.
 *   A problem whose fa_decode_workspace_bytes(B, H, Hkv, N, d, num_splits)
 *   exceeds FA_DECODE_STATIC_SCRATCH_BYTES returns FA_ERR_SCRATCH before
 *   any HIP call (e.g. B * H * splits * (d + 2) * 4 bytes > 16 MiB).
 * Every call on one device shares that device's array and leaves its
 * partials in it; nothing in it needs to start at zero (every partial the
 * merge reads is written by the same call first).  Calls that overlap in
 * time on one device -- on different streams, or from different threads
 * without ordering -- race on the array and give undefined results; calls
 * on one stream are ordered and safe.
 */
fa_status_t fa_decode_static(const void* q, const void* k, const void* v, const int* cache_seqlens, void* o,
                             float* lse, int B, int H, int Hkv, int N, int d, float scale, int num_splits,
                             fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_last_hip_error -- the hipError_t behind the last FA_ERR_HIP an entry
 * point returned on the calling thread (0 if none), and, if message is not
 * NULL, the runtime's description of it (static storage).  Host-only.
 */
int fa_last_hip_error(const char** message);

/*
 * fa_mfma_ceiling -- measurement helper, not part of attention: `blocks`
 * workgroups of four waves each run `iters` x 4 dependent-chain
 * v_mfma_f32_32x32x16_bf16 instructions (32768 FLOP each) with no memory
 * traffic, so that the attention kernels' rate can be set against the
 * dense bf16 rate the chip sustains under matrix load (clock and power
 * included) as well as against the nominal peak.  FLOPs per call:
 * blocks * 4 * iters * 4 * 32768.
 *   sink    device buffer of blocks * 256 floats, written only if store != 0
 *           (the flag keeps the compiler from dropping the loop).
 *   stream  HIP stream; one kernel is enqueued on it.
 * Returns FA_ERR_NULL (sink NULL), FA_ERR_SHAPE (iters or blocks <= 0, or
 * blocks * 256 beyond 2^32 - 1), FA_ERR_ALIGN (sink not 4-byte aligned),
 * FA_ERR_HIP (launch failed) or FA_OK.
 */
fa_status_t fa_mfma_ceiling(float* sink, int iters, int blocks, int store, hipStream_t stream);

/* Library version string, e.g. "0.1.0 gfx950" (static storage). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
