// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a forward launch needs; pointers are device pointers in the
// [B][H][N][d] / [B][H][N] layouts of fa.h.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;       // B * H (query heads)
  int N;        // sequence length (queries = keys)
  int d;        // head dim
  int causal;   // nonzero: query i sees keys 0..i
  float scale;  // multiplies Q K^T
  int group;    // query heads per key/value head (H / Hkv); k, v are [B][Hkv][N][d]
  // Variable length (16-bit forward only): when cu_seqlens (device, B + 1
  // ints) is set, N is the longest sequence, BH = B * H, and q, o are
  // [H][total][d], k, v [H / group][total][d], lse [H][total].
  const int* cu_seqlens = nullptr;
  int H = 0;
  int total = 0;
  // FP8 forward only: q, k, v are e4m3 bytes whose values are byte x factor.
  float q_descale = 1.f;
  float k_descale = 1.f;
  float v_descale = 1.f;
};

// Tile shape per (dtype, d).
struct TileConfig {
  int block_q;
  int block_k;
  int waves;
};

TileConfig mfma_tile(int d);  // the 16-bit (MFMA) forward, bf16 and fp16
TileConfig f32_tile(int d);

// Everything a backward launch needs (device pointers, layouts of fa.h).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;  // bwd_workspace_bytes(BH, N, d) bytes
  int BH;           // B * H (query heads)
  int N;
  int d;
  int causal;
  float scale;
  int group;        // query heads per key/value head; k, v, dk, dv are [B][H / group][N][d]
  // Variable length: cu_seqlens (device, B + 1 ints) set, N = the longest
  // sequence, BH = B * H; every tensor is packed per head ([H][total][d],
  // [H / group][total][d], lse [H][total]); workspace
  // bwd_varlen_workspace_bytes(H, total, d).
  const int* cu_seqlens = nullptr;
  int H = 0;
  int total = 0;
  // Grouped heads, fixed length: with part set, the dK/dV pass splits each
  // group's query heads over hsplit workgroups that write fp32 partials to
  // part ([2][hsplit][B * Hkv][N][d]), summed by a reduction kernel.
  int hsplit = 1;
  float* part = nullptr;
};

// Everything a split-K decode launch needs: q, o [B][H][d]; k, v
// [B][Hkv][N][d]; lse [B][H]; workspace at least decode_plan(...).workspace_bytes.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens;  // device [B] keys per sequence, or null: all N
  void* o;
  float* lse;
  void* workspace;
  int B;
  int H;
  int Hkv;
  int N;
  int d;
  float scale;
  int num_splits;  // 0: automatic
};

// How the keys of one (batch, key/value head) are split: `splits` chunks of
// `chunk` keys (the last one shorter), `heads_per_wg` query heads of a group
// per workgroup.  Workspace: fp32 partial o~ [B*H][splits][d] at offset 0,
// fp32 (m, l) [B*H][splits][2] at ml_offset.
struct DecodePlan {
  int heads_per_wg;
  int chunk;
  int splits;
  int64_t split_wgs;
  size_t ml_offset;
  size_t workspace_bytes;
};
DecodePlan decode_plan(int B, int H, int Hkv, int N, int d, int num_splits);
int decode_rows_per_iter(int d, int heads_per_wg);

// Launchers: enqueue the kernel(s) on `stream`; return the first
// hipError_t a launch reported.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t stream);
// e4m3 q, k, v (fixed length, d 64 or 128), bf16 o.
hipError_t launch_fwd_fp8(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
// Device address, on the current device, of fa_decode_static's scratch
// array (FA_DECODE_STATIC_SCRATCH_BYTES bytes); looked up once per device.
hipError_t decode_static_scratch(void** ptr);
hipError_t launch_decode_f16(const DecodeParams& p, hipStream_t stream);

// Backward workspace: -L/scale and -D, fp32 [BH][Npad] each; Npad = N
// rounded up to the query tile of the dK/dV pass.
size_t bwd_workspace_bytes(int BH, int N, int d);
size_t bwd_varlen_workspace_bytes(int H, int total, int d);  // -L/scale and -D, fp32 [H][ld] each
int bwd_block_k();  // keys per workgroup of the dK/dV pass
// Head split of the grouped-head dK/dV pass (1: none) and the workspace it
// needs: the statistics, then (256-byte aligned, at bwd_part_offset) the
// fp32 partials.
int bwd_head_split(int B, int H, int Hkv, int N);
size_t bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d);
size_t bwd_part_offset(size_t stats_bytes);
int bwd_block_q();  // queries per streamed tile of the dK/dV pass

// Matrix-core-only ceiling kernel (4 MFMA 32x32x16 bf16 per iteration per
// wave, 256 threads per block); `sink` holds blocks*256 floats.
hipError_t launch_mfma_ceiling(float* sink, int iters, int blocks, int store, hipStream_t stream);

}  // namespace fa
