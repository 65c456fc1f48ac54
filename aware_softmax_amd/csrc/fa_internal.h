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
  int BH;       // B * H
  int N;        // sequence length (queries = keys)
  int d;        // head dim
  int causal;   // nonzero: query i sees keys 0..i
  float scale;  // multiplies Q K^T
};

// Tile shape per (dtype, d).
struct TileConfig {
  int block_q;
  int block_k;
  int waves;
};

TileConfig bf16_tile(int d);
TileConfig f32_tile(int d);

// Launchers: enqueue the kernel on `stream`; return the launch's hipError_t.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);

}  // namespace fa
