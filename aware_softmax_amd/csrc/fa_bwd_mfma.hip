// FlashAttention-2 backward, bfloat16 or float16 in/out (a template
// parameter), fp32 accumulation, gfx950 MFMA.
//
// What is computed (per batch*head), the chain rule through
// O = softmax(scale * Q K^T + mask) V with P rebuilt from the saved row
// statistic L instead of stored ("FlashAttention: Move Less, Not Compute
// Less", "Why More Arithmetic Can Finish Sooner"; "FlashAttention-2: Why
// the Attention Bottleneck Wasn't Where Everyone Was Looking", "FA2 change
// #1": only L = m + log l is kept for the backward):
//   P  = exp(scale * Q K^T - L)          (0 where masked)
//   dV = P^T dO,   dP = dO V^T,   D_i = dO_i . O_i,   dS = P * (dP - D)
//   dK = scale * dS^T Q,   dQ = scale * dS K
//
// How.  "FA2 change #2" (last paragraph) parallelises the backward over key
// columns: each worker owns dK_j and dV_j, and the dQ rows that every
// worker touches are accumulated with atomic adds.  The key-column part is
// kept; the dQ atomics are not: on MI355X fp32 atomic adds of one 64 x d
// partial dQ per (key block, query tile) took as long as all five matrix
// products together (about one lane per clock per CU).  dQ is instead
// formed by a second, query-parallel kernel that rebuilds S, P and dP for
// its rows -- two more matrix products in place of the atomics, the pages'
// trade of recomputation for memory traffic once more -- which also makes
// dQ deterministic.
//
// Three kernels:
//   bwd_pre   D_i = dO_i . O_i (fp32) and L_i / scale, stored negated: the
//             initial values of the dP and S accumulators below;
//   bwd_dkdv  one workgroup per (head, 128-key block), 4 wave64s with 32
//             keys each; 64-query tiles of Q and dO (plus L, D) streamed
//             through triple-buffered LDS; dK, dV in registers (at d = 256
//             two workgroups per key block, one per half of the columns of
//             dK and dV, and double-buffered LDS);
//   bwd_dq    one workgroup per (head, 128-query block), 4 wave64s with 32
//             queries each; 32-key tiles of K and V streamed through
//             triple-buffered LDS (48 KB); dQ in registers.  At 242 VGPRs
//             two workgroups share a CU (two waves per SIMD).
//
// MI355X mapping (v_mfma_f32_32x32x16_bf16 throughout; one wave per SIMD in
// bwd_dkdv, whose dK and dV accumulators take 128 registers per lane, two
// in bwd_dq):
//   * the MFMA accumulator layout that computes scores is directly the B
//     operand of the next product: in bwd_dkdv S and dP have queries as rows
//     and the wave's 32 keys as columns, so P and dS packed to bf16 feed
//     dV^T += dO^T P and dK^T += Q^T dS; in bwd_dq S^T and dP^T have keys as
//     rows and the wave's 32 queries as columns, so dS^T feeds
//     dQ^T += K^T dS^T (the order of the 16 contraction indices of a step
//     is permuted identically on both operands);
//   * the transposed operands (dO^T, Q^T, K^T) come from the row-major LDS
//     tiles through ds_read_b64_tr_b16;
//   * LDS tiles are XOR-swizzled per 16-byte chunk so that both the
//     row-fragment reads (ds_read_b128) and the transposing reads are free
//     of bank conflicts, and are filled by LDS-DMA (global_load_lds) two
//     tiles ahead;
//   * the exponentials and packing of a tile ride on its MFMAs: in
//     bwd_dkdv those of the first 32-query block on the MFMAs that compute
//     the second block's scores, the second block's on the first gradient
//     MFMAs; in bwd_dq on the gradient MFMAs.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_internal.h"
#include "fa_schedule.h"

namespace fa {
namespace {

template <class T>
using vec8 = T __attribute__((ext_vector_type(8)));
template <class T>
using vec4 = T __attribute__((ext_vector_type(4)));
template <class T>
using vec2 = T __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 128;     // bwd_dkdv: keys per workgroup (32 per wave)
constexpr int kBQ = 64;       // bwd_dkdv: queries per streamed tile
constexpr int kBQdq = 128;    // bwd_dq: queries per workgroup (32 per wave)
constexpr int kBKdq = 32;     // bwd_dq: keys per streamed tile
constexpr int kRing = 3;      // LDS buffers per streamed tensor (bwd_dq; bwd_dkdv up to d = 128)
constexpr int64_t kHeadSplitMaxWgs = 256;  // dK/dV grids up to one round on 256 CUs split the group's heads
constexpr float kLog2e = 1.44269504088896340736f;

// Variable-length layout (cu set): B sequences packed into `total` rows per
// head; q, o, dO, dQ [H][total][D], k, v, dK, dV [H / group][total][D],
// L [H][total], workspace statistics [H][ld] (ld = total rounded up to 64,
// plus 64, so that a 64-row statistics tile never leaves its head).
// Sequence b is rows cu[b] .. cu[b + 1] - 1 (offsets clamped to
// [0, total], so no access leaves the tensors whatever the array holds).
// cu null: the fixed-length layouts [BH][N][D] and [BH][Npad].
inline int varlen_ld(int total) { return (total + kBQ - 1) / kBQ * kBQ + kBQ; }

struct VarLen {
  const int* cu;
  int H;
  int total;
  int ld;
};
__device__ __forceinline__ int seq_start(const VarLen& vl, int b) { return min(max(vl.cu[b], 0), vl.total); }
__device__ __forceinline__ int seq_len(const VarLen& vl, int b, int r0) {
  return min(max(vl.cu[b + 1], r0), vl.total) - r0;
}

// Calls fn(integral_constant<int, i>) for i = 0 .. N-1, fully unrolled.
template <class Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, I...>) {
  (fn(std::integral_constant<int, I>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  static_for_impl(fn, std::make_integer_sequence<int, N>{});
}
template <int I>
using ic = std::integral_constant<int, I>;

// Elements per LDS tile row: d rounded up to a power-of-two number of
// 16-byte chunks (d = 32 -> 64, 96 -> 128), so that the XOR swizzle below
// permutes whole rows.  The pad chunks are filled with copies of real
// chunks and never read: the MFMA loops run over d only.
template <int D>
constexpr int lds_row_elems() {
  return D == 32 ? 64 : D == 96 ? 128 : D;
}

// Physical 16-byte chunk mask of row r of an LDS tile whose rows are ROWB
// bytes (chunk c is stored at c ^ mask).  Conflict-free for
//   * 16 lanes reading one chunk of 16 consecutive rows (ds_read_b128), and
//   * 32 lanes reading 4 chunks of 4 consecutive rows (transposing reads).
template <int ROWB>
__device__ __forceinline__ int swz_mask(int r) {
  static_assert(ROWB == 512 || ROWB == 256 || ROWB == 128, "rows of 64, 128 or 256 bf16");
  // 512-byte rows: the 16 bank groups repeat every 16 chunks, so the
  // 256-byte mask (4 bits) serves them as well.
  if constexpr (ROWB >= 256)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// LDS operand reads by inline asm: completion is tracked only by the
// explicit lgkmcnt waits that precede each use, so several fragments stay in
// flight while the MFMAs run (hipcc's own wait insertion would drain the
// queue before every read).  LDS reads complete in order, so a wait that
// counts only the reads issued after a fragment is exact for it.  The loops
// below issue no other LDS operation.
template <int OFF, class T>
__device__ __forceinline__ void ds_b128(vec8<T>& f, unsigned addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_b128f(f32x4& f, unsigned addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr64(s16x4& f, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "i"(OFF));
}
template <class T>
__device__ __forceinline__ vec8<T> join(const s16x4& lo, const s16x4& hi) {
  return __builtin_bit_cast(vec8<T>, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Two fp32 values rounded (to nearest even) to the element type, packed.
template <class T>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, vec2<T>));
}
__device__ __forceinline__ f32x16 mfma(const vec8<__bf16>& a, const vec8<__bf16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(const vec8<_Float16>& a, const vec8<_Float16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// dK^T / dV^T accumulation with the accumulator pinned to AGPRs (C and D
// of the MFMA in the accumulation register file).  Left to itself the
// compiler keeps part of the scores there as well and shuttles them with
// v_accvgpr_mov (48 per tile at d = 128); pinned, dK and dV take 128 AGPRs,
// everything else fits the VGPRs, and the backward is 8-10 % faster (B2 H16
// N4096 d128 causal, same box).  The asm is opaque to the compiler's hazard
// checks, so it carries its own: two wait states first (the B operand may
// just have been written by VALU), and mfma_drain before the accumulators
// are read.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const vec8<__bf16>& a, const vec8<__bf16>& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16& acc, const vec8<_Float16>& a, const vec8<_Float16>& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last accumulating MFMA and any other access of
// its accumulator.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Waits until all but this wave's last KEEP vector memory operations (the
// LDS-DMA copies of the tile after next, issued this iteration) and all its
// LDS operations are complete, then the workgroup barrier.  Vector memory
// operations of a wave complete in issue order.
template <int KEEP>
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(KEEP) : "memory");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned lds_u32;
// Word 3 of a gfx9-family buffer descriptor: the plain 32-bit data format.
constexpr int kBufferWord3 = 0x00020000;
__device__ void raw_buffer_load_lds(i32x4 rsrc, lds_u32* lds, int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer descriptor of the `bytes` bytes at p, kept in scalar registers
// (every argument is uniform over the wave; readfirstlane says so).
__device__ __forceinline__ i32x4 buffer_desc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return {__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
          __builtin_amdgcn_readfirstlane(bytes), kBufferWord3};
}

// LDS-DMA of rows [r0, r0 + kRows) of a row-major [N][D] 16-bit matrix into
// a swizzled LDS tile.  One wave instruction writes 1 KiB of LDS
// contiguously (lane l at byte 16 l); the swizzle is applied by choosing
// which logical chunk each lane fetches.  The tile's first row is the base
// of a buffer descriptor and each lane adds a constant byte offset, so a
// copy costs no vector ALU work; rows past N - 1 fall outside the
// descriptor's range and read as zeros (they are masked wherever they
// enter).  Wave w issues instructions [w IPW, (w + 1) IPW).
template <int D, int kRows>
struct RowTileDma {
  static constexpr int ROWB = 2 * lds_row_elems<D>(), CPR = ROWB / 16, RPI = 1024 / ROWB;
  static constexpr int IPW = kRows * ROWB / 1024 / kWaves;
  static_assert(kRows * ROWB % (1024 * kWaves) == 0, "DMA splits evenly over waves");
  unsigned off[IPW];  // byte offset of this lane's chunk from the tile's first row
  __device__ RowTileDma(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int row = (wave * IPW + i) * RPI + lane / CPR;
      const int slot = (lane % CPR) ^ swz_mask<ROWB>(row);  // logical chunk of this LDS slot
      const int chunk = slot < D / 8 ? slot : slot - D / 8;   // pad slots: a copy of a real chunk
      off[i] = (unsigned)(row * D * 2 + chunk * 16);
    }
  }
  template <class T>
  __device__ i32x4 desc(const T* X, int r0, int N) const {
    return buffer_desc(X + (size_t)r0 * D, min(max(N - r0, 0), kRows) * D * 2);
  }
  // instruction i of this wave
  __device__ void copy(const i32x4& rs, char* tile, int wave, int i) const {
    raw_buffer_load_lds(rs, (lds_u32*)(tile + (wave * IPW + i) * 1024), 16, (int)off[i], 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// bwd_pre: one row per LPR lanes (CPL 16-byte chunks of dO and O each; LPR
// the largest power of two dividing the row's chunk count).
template <int D>
constexpr int pre_lanes_per_row() {
  return (D / 8) & -(D / 8);
}
// Writes -D_i and -L_i / scale (in the units of the raw score q.k): the
// initial values of the dP and S accumulators of the two main kernels, so
// that their MFMAs produce dP - D and q.k - L / scale directly.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ Og, const T* __restrict__ dOg,
                                                      const float* __restrict__ Lg, float* __restrict__ Lsg,
                                                      float* __restrict__ Dng, int N, int Npad, float l_to_score,
                                                      VarLen vl) {
  constexpr int LPR = pre_lanes_per_row<D>();
  constexpr int CPL = D / 8 / LPR;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int c = tid % LPR;
  const size_t row = (size_t)blockIdx.x * RPB + tid / LPR;  // in [0, BH * Npad), or [0, H * ld)
  // fixed length: head bh, row i of N (padded to Npad); variable length:
  // head bh, packed row i of total (padded to ld)
  const int stride = vl.cu ? vl.ld : Npad;
  const int rows = vl.cu ? vl.total : N;
  const int bh = (int)(row / stride);
  const int i = (int)(row % stride);
  float acc = 0.f;
  if (i < rows) {
#pragma unroll
    for (int x = 0; x < CPL; ++x) {
      const size_t off = ((size_t)bh * rows + i) * D + (c + x * LPR) * 8;
      const vec8<T> a = *(const vec8<T>*)(Og + off);
      const vec8<T> b = *(const vec8<T>*)(dOg + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
  }
#pragma unroll
  for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (c == 0) {
    Dng[row] = -acc;
    Lsg[row] = i < rows ? -Lg[(size_t)bh * rows + i] * l_to_score : 0.f;
  }
}

// ---------------------------------------------------------------------------
// bwd_dkdv.
template <int D>
struct DkdvLayout {
  static constexpr int ROWB = 2 * lds_row_elems<D>();
  // Buffers per streamed tensor: three (DMA two tiles ahead), two at
  // d = 256, whose 32 KiB tiles leave room for no third.
  static constexpr int RING = D > 128 ? 2 : kRing;
  static constexpr int QTILE = kBQ * ROWB;    // one Q or dO tile
  static constexpr int STTILE = 2 * kBQ * 4;  // -L/scale[64], -D[64]
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + RING * QTILE;
  static constexpr int OFF_ST = OFF_DO + RING * QTILE;
  static constexpr int TOTAL = OFF_ST + RING * STTILE;
  static_assert(TOTAL <= 160 * 1024, "fits the 160 KiB LDS");
};

// bwd_dkdv column halves: at d = 256 the dK and dV accumulators of 32 keys
// (256 registers per lane) do not fit beside the K and V fragments, so
// each (key block) is processed by two workgroups that rebuild the same S
// and dP over the full d and accumulate dK and dV for one half of the
// columns each (phase A is done twice: 1.5x the matrix work of one pass).
template <int D>
constexpr int dkdv_halves() {
  return D > 128 ? 2 : 1;
}

// Per 64-query tile and wave (32 keys):
//   A  S = Q K^T - L/scale and dP = dO V^T - D  (4 DT MFMAs; row fragments
//      of the Q and dO tiles, several in flight);
//   V  P = 2^(c S), dS = P dP, both packed to bf16 (VALU only), in eight
//      groups of 4 rows: those of query block 0 ride on the second half of
//      A (block 1's MFMAs), those of block 1 on the first two steps of B;
//   B  dV^T += dO^T P and dK^T += Q^T dS        (8 DBO MFMAs, transposing reads;
//      DBO = the 32-column blocks of the workgroup's columns of dK and dV).
// Iteration t runs A(t) and B(t) with V(t) spread over both; the DMA of
// the tile RING - 1 ahead is in flight meanwhile; one barrier per
// iteration.
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                     const T* __restrict__ dOg, const float* __restrict__ Lsg, const float* __restrict__ Dng,
                     T* __restrict__ dKg, T* __restrict__ dVg, int BHkv, int N, int Npad, int nkb, float c,
                     float scale, int group, VarLen vl, int hsplit, float* __restrict__ part) {
  using Ly = DkdvLayout<D>;
  constexpr int DT = D / 16;
  constexpr int NH = dkdv_halves<D>();
  constexpr int DBO = D / 32 / NH;  // 32-column blocks of dK, dV per workgroup
  constexpr int ROWB = Ly::ROWB;
  constexpr int RING = Ly::RING;
  constexpr int PF = RING - 1;  // tiles in flight ahead of the one being read
  constexpr int NA = 4 * DT;   // phase A MFMAs
  constexpr int LA = 4;        // phase A fragments in flight
  constexpr int NB = 8 * DBO;  // phase B MFMAs
  constexpr int LB = 4;       // phase B fragments in flight
  static_assert(NA % 8 == 0, "eight VALU groups ride on the phase A MFMAs");
  __shared__ __attribute__((aligned(1024))) char smem[Ly::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  // One workgroup per (key/value head, key block); it sums dK and dV over
  // the `group` query heads that share the key/value head (consecutive
  // query heads bhk * group .. bhk * group + group - 1).
  // With hsplit > 1 (fixed length only) the group's query heads are split
  // into hsplit subsets of hc heads, one workgroup per (key/value head,
  // subset, key block), and each writes its partial dK, dV in fp32 to
  // `part` ([hsplit][BHkv][N][D] each) for bwd_reduce_kernel to sum.
  // With NH = 2 (d = 256) the column half dh is the fastest index of the
  // head dimension, so both halves of a key block are neighbours in the
  // schedule and read the same Q, dO tiles close in time.
  int vbh2, jb;
  map_block(blockIdx.x, BHkv * hsplit * NH * nkb, nkb, CAUSAL ? Order::HeavyFirst : Order::Plain, &vbh2, &jb);
  const int vbh = vbh2 / NH;
  const int dcol = (vbh2 - vbh * NH) * (D / NH);  // first dK, dV column of this workgroup
  const int bhk = vbh / hsplit;
  const int sub = vbh - bhk * hsplit;
  const int hc = group / hsplit;  // query heads of this workgroup: hs .. hs + hc - 1 of the group
  const int hs = sub * hc;
  const int kb0 = jb * kBKV;
  // Rows of this key/value head (and sequence): `head` is the element
  // offset of its K/V row 0; query head r of the group has Q/dO row 0 at
  // q_off(r) and statistics row 0 at st_off(r).
  size_t head;
  int hk = bhk, r0 = 0;
  if (vl.cu) {
    const int n_kv = vl.H / group;
    const int B = BHkv / n_kv;  // head-major: hk = bhk / B (each XCD gets the same heads of every sequence)
    hk = bhk / B;
    const int b = bhk - hk * B;
    r0 = seq_start(vl, b);
    N = seq_len(vl, b, r0);
    if (kb0 >= N) return;  // past the end of this sequence (the whole workgroup)
    Npad = (N + kBQ - 1) / kBQ * kBQ;
    head = ((size_t)hk * vl.total + r0) * D;
  } else {
    head = (size_t)bhk * (size_t)N * D;
  }
  auto q_off = [&](int r) -> size_t {
    return vl.cu ? ((size_t)(hk * group + r) * vl.total + r0) * D : (size_t)(bhk * group + r) * (size_t)N * D;
  };
  auto st_off = [&](int r) -> size_t {
    return vl.cu ? (size_t)(hk * group + r) * vl.ld + r0 : (size_t)(bhk * group + r) * Npad;
  };
  const int kw0 = kb0 + 32 * wave;  // first key of this wave
  const int key = kw0 + col;        // this lane's key (MFMA column)
  const T* Kh = Kg + head;
  const T* Vh = Vg + head;

  // K and V fragments of the wave's keys: B operands of S = Q K^T and
  // dP = dO V^T (lane: key `col`, d = 16t + 8 half .. + 7).
  vec8<T> kf[DT], vf[DT];
  {
    const size_t r = (size_t)min(key, N - 1) * D + half * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      kf[t] = *(const vec8<T>*)(Kh + r + 16 * t);
      vf[t] = *(const vec8<T>*)(Vh + r + 16 * t);
    }
  }

  // Query tiles it0 .. nqt - 1 of each head of the group, streamed as one
  // sequence v = r * span + (it - it0) (r: head within the group).
  const int nqt = Npad / kBQ;
  const int it0 = CAUSAL ? kb0 / kBQ : 0;
  const int span = nqt - it0;
  const int total = hc * span;
  // Tile v goes to ring buffer (v + ring_off) mod RING, the offset chosen
  // so that the first head's first unmasked tile lands in buffer 0 (the
  // unrolled loop below starts there).
  const int it_s0 = CAUSAL ? min(it0 + 2, nqt) : 0;
  const int ring_off = (RING - (it_s0 - it0) % RING) % RING;
  auto ring = [&](int v) { return __builtin_amdgcn_readfirstlane((v + ring_off) % RING); };
  using QDma = RowTileDma<D, kBQ>;
  const QDma qdma(wave, lane);
  constexpr int kDmaPerWave = 1 + 2 * QDma::IPW;  // statistics, Q, dO
  static_assert(kDmaPerWave <= NA, "the copies of a tile ride on phase A's MFMAs");
  // Descriptors of tile v: its 64 statistics (-L/scale for waves 0 and 2,
  // -D for waves 1 and 3: the duplicate copy writes the same bytes and keeps
  // the number of DMA instructions per wave uniform for the waits), Q, dO.
  struct TileDesc {
    i32x4 st, q, dO;
  };
  auto tile_desc = [&](int v) {
    const int rr = __builtin_amdgcn_readfirstlane(v / span);
    const int r = hs + rr;
    const int it = it0 + v - rr * span;
    const size_t qhead = q_off(r);
    return TileDesc{buffer_desc((wave & 1 ? Dng : Lsg) + st_off(r) + it * kBQ, kBQ * 4),
                    qdma.desc(Qg + qhead, it * kBQ, N), qdma.desc(dOg + qhead, it * kBQ, N)};
  };
  // DMA instruction k of this wave for a tile with descriptors t into ring buffer b
  auto dma_op = [&](const TileDesc& t, int b, auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0)
      raw_buffer_load_lds(t.st, (lds_u32*)(smem + Ly::OFF_ST + b * Ly::STTILE + (wave & 1) * 4 * kBQ), 4, lane * 4,
                          0, 0, 0);
    else if constexpr (k <= QDma::IPW)
      qdma.copy(t.q, smem + Ly::OFF_Q + b * Ly::QTILE, wave, k - 1);
    else
      qdma.copy(t.dO, smem + Ly::OFF_DO + b * Ly::QTILE, wave, k - 1 - QDma::IPW);
  };
  auto dma_tile = [&](int v) {
    const TileDesc t = tile_desc(v);
    static_for<kDmaPerWave>([&](auto kc) { dma_op(t, ring(v), kc); });
  };

  // Lane-constant LDS byte offsets within a tile.
  // Row fragments: row 32 qb + col, logical chunk 2t + half, stored at
  // (2t) ^ (half ^ mask): t enters as a XOR of bits 5.. of the offset.
  unsigned rf_lane[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = 32 * qb + col;
    rf_lane[qb] = (unsigned)(r * ROWB + ((half ^ swz_mask<ROWB>(r)) << 4));
  }
  // Transposing reads: lane gets column 32b + col of rows 16u + 4 half +
  // {0..3} (lo) and 16u + 8 + 4 half + {0..3} (hi); the swizzle does not
  // depend on u, which enters as an immediate offset.
  unsigned trq[DBO][2];
  {
    const int tr_e = (lane & 15) >> 2, tr_t = lane & 3, tr_cg = (lane >> 4) & 1;
#pragma unroll
    for (int b = 0; b < DBO; ++b)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * half + tr_e + 8 * hi;
        const int chunk = dcol / 8 + 4 * b + 2 * tr_cg + (tr_t >> 1);
        trq[b][hi] = (unsigned)(r * ROWB + ((chunk ^ swz_mask<ROWB>(r)) << 4) + (tr_t & 1) * 8);
      }
  }
  const unsigned sbase = lds_addr(smem);
  // Absolute LDS addresses in ring buffer 0 (Q and dO): the row fragments
  // of 16-wide d step t, the transposing reads, the statistics.  The ring
  // buffer (when known at compile time), the query block and the 16-query
  // step then enter as instruction immediates.  At d = 256 (no registers
  // to spare) the addresses are formed per read and the ring buffer stays
  // a run-time value.
  constexpr bool kAbs = D <= 128;
  unsigned rq[kAbs ? DT : 1], rdo[kAbs ? DT : 1], tq[DBO][2], tdo[DBO][2];
#pragma unroll
  for (int t = 0; t < (kAbs ? DT : 0); ++t) {
    rq[t] = sbase + Ly::OFF_Q + (rf_lane[0] ^ (unsigned)(t << 5));
    rdo[t] = sbase + Ly::OFF_DO + (rf_lane[0] ^ (unsigned)(t << 5));
  }
#pragma unroll
  for (int b = 0; b < DBO; ++b)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      tq[b][hi] = sbase + Ly::OFF_Q + trq[b][hi];
      tdo[b][hi] = sbase + Ly::OFF_DO + trq[b][hi];
    }
  const unsigned ast0 = sbase + Ly::OFF_ST + 16 * half;

  f32x16 dkT[DBO], dvT[DBO];
#pragma unroll
  for (int b = 0; b < DBO; ++b) {
    dkT[b] = f32x16{};
    dvT[b] = f32x16{};
  }
  f32x16 S[2], dP[2];  // [query block]
  unsigned pw[2][8], dw[2][8];

  // visible iff key <= query (causal), query < N and key < N: with lo = the
  // smallest visible query index, query q is visible iff lo <= q < N.
  const int lo = key >= N ? INT_MAX / 2 : (CAUSAL ? key : 0);

  // VALU group k: P and dS of query block k / 4, rows 8 (k % 4) + 4 half +
  // {0..3}, i.e. the bf16 pairs of 16-query step k / 2 of phase B.
  auto vgroup = [&](auto kc, auto mask_c, int it) {
    constexpr int k = decltype(kc)::value, qb = k / 4, g = k % 4;
    constexpr bool MASK = decltype(mask_c)::value;
    float p[4], ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = __builtin_amdgcn_exp2f(S[qb][4 * g + e] * c);
      if constexpr (MASK) {
        const int qi = it * kBQ + 32 * qb + 8 * g + 4 * half + e;
        const unsigned keep = ~(unsigned)(((qi - lo) | (N - 1 - qi)) >> 31);
        pe = __uint_as_float(__float_as_uint(pe) & keep);
      }
      p[e] = pe;
      ds[e] = pe * dP[qb][4 * g + e];
    }
    pw[qb][2 * g] = pack2<T>(p[0], p[1]);
    pw[qb][2 * g + 1] = pack2<T>(p[2], p[3]);
    dw[qb][2 * g] = pack2<T>(ds[0], ds[1]);
    dw[qb][2 * g + 1] = pack2<T>(ds[2], ds[3]);
  };

  // One tile: phase A, then phase B with the VALU groups of step u + 1
  // riding on the MFMAs of step u (groups 0 and 1 run before step 0).
  // bc: the ring buffer of tile v, as an int or as integral_constant (then
  // every buffer offset is an instruction immediate).
  auto iteration = [&](int v, int it, auto mask_c, auto bc) {
    constexpr bool CT = !std::is_integral_v<decltype(bc)>;
    int b;
    if constexpr (CT)
      b = decltype(bc)::value;
    else
      b = bc;
    // The copies of tile v + PF ride on phase A's MFMAs, one every
    // kDmaStride.  Past the last tile they repeat it into the buffer of tile
    // v - 1 (already consumed, never read again): no branch in the MFMA
    // stream, and the waits below count the same instructions.
    const TileDesc nt = tile_desc(min(v + PF, total - 1));
    const int nb = CT ? (b + PF) % RING : ring(v + PF);
    constexpr int kDmaStride = PF == 1 ? 1 : NA / kDmaPerWave;  // one tile ahead: copy early
    // buffer offsets: immediates (BQ, BS) or run-time additions (bq, bs)
    constexpr int BQ = [] {
      if constexpr (CT) return decltype(bc)::value * Ly::QTILE;
      else return 0;
    }();
    constexpr int BS = [] {
      if constexpr (CT) return decltype(bc)::value * Ly::STTILE;
      else return 0;
    }();
    const unsigned bq = CT ? 0u : (unsigned)(b * Ly::QTILE);
    {
      const unsigned ast = ast0 + (CT ? 0u : (unsigned)(b * Ly::STTILE));
      // initial accumulators: register 4 g + e of query block qb holds query
      // 32 qb + 8 g + 4 half + e
      f32x4 init[2][2][4];  // [S or dP][qb][g]
      static_for<8>([&](auto kc) {
        constexpr int k = decltype(kc)::value, qb = k / 4, g = k % 4;
        ds_b128f<BS + (32 * qb + 8 * g) * 4>(init[0][qb][g], ast);
        ds_b128f<BS + (kBQ + 32 * qb + 8 * g) * 4>(init[1][qb][g], ast);
      });
      vec8<T> fa[LA];
      auto issue = [&](auto fc) {
        constexpr int F = decltype(fc)::value, qb = F / (2 * DT), t = (F / 2) % DT, X = F % 2;
        if constexpr (kAbs)
          ds_b128<BQ + qb * 32 * ROWB>(fa[F % LA], (X ? rdo[t] : rq[t]) + bq);
        else
          ds_b128<0>(fa[F % LA], sbase + (X ? Ly::OFF_DO : Ly::OFF_Q) + (unsigned)(b * Ly::QTILE) +
                                     (rf_lane[qb] ^ (unsigned)(t << 5)));
      };
      static_for<(LA < NA ? LA : NA)>(issue);
      asm volatile("s_waitcnt lgkmcnt(%16)"
                   : "+v"(init[0][0][0]), "+v"(init[0][0][1]), "+v"(init[0][0][2]), "+v"(init[0][0][3]),
                     "+v"(init[0][1][0]), "+v"(init[0][1][1]), "+v"(init[0][1][2]), "+v"(init[0][1][3]),
                     "+v"(init[1][0][0]), "+v"(init[1][0][1]), "+v"(init[1][0][2]), "+v"(init[1][0][3]),
                     "+v"(init[1][1][0]), "+v"(init[1][1][1]), "+v"(init[1][1][2]), "+v"(init[1][1][3])
                   : "i"(LA));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S[qb][4 * g + e] = init[0][qb][g][e];
            dP[qb][4 * g + e] = init[1][qb][g][e];
          }
      static_for<NA>([&](auto fc) {
        constexpr int F = decltype(fc)::value, qb = F / (2 * DT), t = (F / 2) % DT, X = F % 2;
        constexpr int last = (F + LA - 1 < NA - 1) ? F + LA - 1 : NA - 1;
        asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(fa[F % LA]) : "i"(last - F));
        if constexpr (X == 0)
          S[qb] = mfma(fa[F % LA], kf[t], S[qb]);
        else
          dP[qb] = mfma(fa[F % LA], vf[t], dP[qb]);
        if constexpr (F + LA < NA) issue(ic<F + LA>{});
        if constexpr (F % kDmaStride == 0 && F / kDmaStride < kDmaPerWave)
          dma_op(nt, nb, ic<F / kDmaStride>{});
        // groups 0-3 (query block 0, complete after the first half) ride on
        // the second half's MFMAs, one after each quarter of it
        constexpr int Q4 = DT / 2;
        if constexpr (F >= 2 * DT && (F - 2 * DT) % Q4 == Q4 - 1) vgroup(ic<(F - 2 * DT) / Q4>{}, mask_c, it);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    {
      s16x4 lo_[LB], hi_[LB];
      auto issue = [&](auto fc) {
        constexpr int F = decltype(fc)::value, u = F / (2 * DBO), bb = (F / 2) % DBO, X = F % 2;
        ds_tr64<BQ + u * 16 * ROWB>(lo_[F % LB], (X ? tq[bb][0] : tdo[bb][0]) + bq);
        ds_tr64<BQ + u * 16 * ROWB>(hi_[F % LB], (X ? tq[bb][1] : tdo[bb][1]) + bq);
      };
      static_for<(LB < NB ? LB : NB)>(issue);
      static_for<NB>([&](auto fc) {
        constexpr int F = decltype(fc)::value, u = F / (2 * DBO), bb = (F / 2) % DBO, X = F % 2;
        constexpr int last = (F + LB - 1 < NB - 1) ? F + LB - 1 : NB - 1;
        constexpr int qb = u / 2, h2 = u % 2;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo_[F % LB]), "+v"(hi_[F % LB]) : "i"(2 * (last - F)));
        if constexpr (X == 0) {
          const vec8<T> pf = __builtin_bit_cast(
              vec8<T>, (u32x4){pw[qb][4 * h2], pw[qb][4 * h2 + 1], pw[qb][4 * h2 + 2], pw[qb][4 * h2 + 3]});
          mfma_acc(dvT[bb], join<T>(lo_[F % LB], hi_[F % LB]), pf);
        } else {
          const vec8<T> dsf = __builtin_bit_cast(
              vec8<T>, (u32x4){dw[qb][4 * h2], dw[qb][4 * h2 + 1], dw[qb][4 * h2 + 2], dw[qb][4 * h2 + 3]});
          mfma_acc(dkT[bb], join<T>(lo_[F % LB], hi_[F % LB]), dsf);
        }
        if constexpr (F + LB < NB) issue(ic<F + LB>{});
        // groups 4 + 2u and 5 + 2u (query block 1, used from step 2 on)
        // after the first and second half of step u < 2's MFMAs
        constexpr int per = 2 * DBO, f = F % per;
        if constexpr (u < 2 && (f == per / 2 - 1 || f == per - 1))
          vgroup(ic<4 + 2 * u + (f == per - 1 ? 1 : 0)>{}, mask_c, it);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // tile v + 1 must be complete; with three buffers the copies of tile
    // v + 2 stay in flight
    if (PF == 2 && v + 2 < total)
      dma_barrier<kDmaPerWave>();
    else
      dma_barrier<0>();
  };

  // Tiles [it0, it_s) and [it_e, nqt) may hide scores (the causal diagonal,
  // the ragged end); tiles in between need no mask for any wave.
  const int it_s = it_s0;
  int it_e = kb0 + kBKV <= N ? N / kBQ : 0;
  it_e = max(it_e, it_s);

  dma_tile(0);
  if (PF == 2 && 1 < total) {
    dma_tile(1);
    dma_barrier<kDmaPerWave>();
  } else {
    dma_barrier<0>();
  }
  for (int rr = 0; rr < hc; ++rr) {
    int v = rr * span;
    int it = it0;
    for (; it < it_s; ++it, ++v) iteration(v, it, std::true_type{}, ring(v));
    // Unmasked tiles: up to buffer 0 with the buffer a run-time value, then
    // the loop unrolled by the ring period (the buffers compile-time), then
    // the rest.
    for (; kAbs && it < it_e && ring(v) != 0; ++it, ++v) iteration(v, it, std::false_type{}, ring(v));
    for (; kAbs && it + RING <= it_e; it += RING, v += RING) {
      iteration(v, it, std::false_type{}, ic<0>{});
      iteration(v + 1, it + 1, std::false_type{}, ic<1>{});
      if constexpr (RING > 2) iteration(v + 2, it + 2, std::false_type{}, ic<(RING > 2 ? 2 : 0)>{});
    }
    for (; it < it_e; ++it, ++v) iteration(v, it, std::false_type{}, ring(v));
    for (; it < nqt; ++it, ++v) iteration(v, it, std::true_type{}, ring(v));
  }

  mfma_drain();
  // ---- dK = scale * (dK^T)^T, dV: lane writes key `key`, d = 32 b + 8 g + 4 half + {0..3}.
  if (part && key < N) {  // fp32 partials of this head subset
    const size_t plane = (size_t)hsplit * BHkv * N * D;
    float* pk = part + (((size_t)sub * BHkv + bhk) * N + key) * D + dcol + 4 * half;
    float* pv = pk + plane;
#pragma unroll
    for (int b = 0; b < DBO; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ok, ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[e] = dkT[b][4 * g + e] * scale;
          ov[e] = dvT[b][4 * g + e];
        }
        *(f32x4*)(pk + 32 * b + 8 * g) = ok;
        *(f32x4*)(pv + 32 * b + 8 * g) = ov;
      }
  } else if (key < N) {
    T* dkrow = dKg + head + (size_t)key * D + dcol + 4 * half;
    T* dvrow = dVg + head + (size_t)key * D + dcol + 4 * half;
#pragma unroll
    for (int b = 0; b < DBO; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        vec4<T> ok, ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[e] = (T)(dkT[b][4 * g + e] * scale);
          ov[e] = (T)dvT[b][4 * g + e];
        }
        *(vec4<T>*)(dkrow + 32 * b + 8 * g) = ok;
        *(vec4<T>*)(dvrow + 32 * b + 8 * g) = ov;
      }
  }
}

// dK, dV = the sums of the hsplit fp32 partials, rounded once to T
// (`part` as written by bwd_dkdv_kernel with hsplit > 1).  Eight
// consecutive elements per thread; the subsets are added in order, so the
// result is deterministic.
template <class T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part, T* __restrict__ dK,
                                                         T* __restrict__ dV, size_t elems, int hsplit) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= elems) return;
  const size_t plane = (size_t)hsplit * elems;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float* src = part + t * plane + i;
    f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
    for (int s = 1; s < hsplit; ++s) {
      a += *(const f32x4*)(src + s * elems);
      b += *(const f32x4*)(src + s * elems + 4);
    }
    vec8<T> out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] = (T)a[e];
      out[4 + e] = (T)b[e];
    }
    *(vec8<T>*)((t ? dV : dK) + i) = out;
  }
}

// ---------------------------------------------------------------------------
// bwd_dq.
template <int D>
struct DqLayout {
  static constexpr int ROWB = 2 * lds_row_elems<D>();
  static constexpr int KTILE = kBKdq * ROWB;  // one K or V tile
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = OFF_K + kRing * KTILE;
  static constexpr int TOTAL = OFF_V + kRing * KTILE;
  static_assert(TOTAL <= 160 * 1024, "fits the 160 KiB LDS");
};

// Per key tile (32 keys here; the code takes any multiple of 32) and wave
// (32 queries; lane = query, registers = keys):
//   A  S^T = K Q^T - L/scale and dP^T = V dO^T - D  (2 KB DT MFMAs, KB =
//      32-key halves per tile; row fragments of the K and V tiles; Q and
//      dO fragments resident);
//   V  P = 2^(c S^T), dS^T = P dP^T, packed to the element type;
//   C  dQ^T += K^T dS^T                               (2 KB DB MFMAs, transposing reads).
// Iteration j runs A(j + 1) with V(j) riding on its MFMAs, then C(j).
// Three waves per SIMD at d = 32 (+8 % on B2 H16 N4096 d32 causal); at
// d = 64 the same bound costs spills and 5 %.  One at d = 256, where the
// Q and dO fragments and dQ take 256 registers per lane.
template <int D>
constexpr int dq_waves() {
  return D <= 32 ? 3 : D <= 128 ? 2 : 1;
}
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(dq_waves<D>(), dq_waves<D>())))
void bwd_dq_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                   const T* __restrict__ dOg, const float* __restrict__ Lsg, const float* __restrict__ Dng,
                   T* __restrict__ dQg, int BH, int N, int Npad, int nqb, float c, float scale, int group,
                   VarLen vl) {
  using Ly = DqLayout<D>;
  constexpr int DT = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROWB = Ly::ROWB;
  constexpr int KB = kBKdq / 32;  // 32-key halves per tile
  constexpr int NA = 2 * KB * DT;  // phase A MFMAs
  constexpr int LA = 4;
  constexpr int NC = 2 * KB * DB;  // phase C MFMAs
  constexpr int LC = 4;
  __shared__ __attribute__((aligned(1024))) char smem[Ly::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL ? Order::HeavyLast : Order::Plain, &bh, &qb);
  const int q0 = qb * kBQdq;
  // Rows of query head bh (and its sequence): Q/dO/dQ row 0 at `head`, the
  // K/V rows of its key/value head at `kvhead`, statistics row 0 at `st`.
  size_t head, kvhead, st;
  if (vl.cu) {
    const int B = BH / vl.H;  // head-major, as in bwd_dkdv
    const int h = bh / B, b = bh - h * B;
    const int r0 = seq_start(vl, b);
    N = seq_len(vl, b, r0);
    if (q0 >= N) return;  // past the end of this sequence (the whole workgroup)
    Npad = (N + kBQ - 1) / kBQ * kBQ;
    head = ((size_t)h * vl.total + r0) * D;
    kvhead = ((size_t)(h / group) * vl.total + r0) * D;
    st = (size_t)h * vl.ld + r0;
  } else {
    head = (size_t)bh * (size_t)N * D;
    kvhead = (size_t)(bh / group) * (size_t)N * D;  // key/value head of query head bh
    st = (size_t)bh * Npad;
  }
  const int qw = q0 + 32 * wave;
  const int qi = qw + col;  // this lane's query (MFMA column)
  const T* Qh = Qg + head;
  const T* Kh = Kg + kvhead;
  const T* Vh = Vg + kvhead;
  const T* dOh = dOg + head;

  // Q and dO fragments of the wave's queries: B operands of S^T = K Q^T and
  // dP^T = V dO^T (lane: query `col`, d = 16t + 8 half .. + 7).
  vec8<T> qf[DT], dof[DT];
  {
    const size_t r = (size_t)min(qi, N - 1) * D + half * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      qf[t] = *(const vec8<T>*)(Qh + r + 16 * t);
      dof[t] = *(const vec8<T>*)(dOh + r + 16 * t);
    }
  }
  const int qs = min(qi, Npad - 1);
  const float ls = Lsg[st + qs];  // -L / scale
  const float dn = Dng[st + qs];  // -D

  int nkt = (N + kBKdq - 1) / kBKdq;
  if (CAUSAL) nkt = min(nkt, (q0 + kBQdq - 1) / kBKdq + 1);
  auto ring = [&](int j) { return __builtin_amdgcn_readfirstlane(j % kRing); };
  using KDma = RowTileDma<D, kBKdq>;
  const KDma kdma(wave, lane);
  constexpr int kDmaPerWave = 2 * KDma::IPW;  // K, V
  static_assert(kDmaPerWave <= NA, "the copies of a tile ride on phase A's MFMAs");
  // DMA instruction k of this wave for key tile j into ring buffer b
  auto dma_op = [&](int j, int b, auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k < KDma::IPW)
      kdma.copy(kdma.desc(Kh, j * kBKdq, N), smem + Ly::OFF_K + b * Ly::KTILE, wave, k);
    else
      kdma.copy(kdma.desc(Vh, j * kBKdq, N), smem + Ly::OFF_V + b * Ly::KTILE, wave, k - KDma::IPW);
  };
  auto dma_tile = [&](int j) { static_for<kDmaPerWave>([&](auto kc) { dma_op(j, ring(j), kc); }); };

  unsigned rf_lane[KB];  // K / V row fragments: row 32 kb + col, chunk 2t + half
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int r = 32 * kb + col;
    rf_lane[kb] = (unsigned)(r * ROWB + ((half ^ swz_mask<ROWB>(r)) << 4));
  }
  unsigned trk[DB][2];  // K^T transposing reads
  {
    const int tr_e = (lane & 15) >> 2, tr_t = lane & 3, tr_cg = (lane >> 4) & 1;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * half + tr_e + 8 * hi;
        const int chunk = 4 * b + 2 * tr_cg + (tr_t >> 1);
        trk[b][hi] = (unsigned)(r * ROWB + ((chunk ^ swz_mask<ROWB>(r)) << 4) + (tr_t & 1) * 8);
      }
  }
  const unsigned sbase = lds_addr(smem);
  // Absolute LDS addresses in ring buffer 0: K and V row fragments of
  // 16-wide d step t, the K^T transposing reads; the ring buffer (when
  // known at compile time) and the 16-key step enter as immediates.  (At
  // d = 256, one wave per SIMD, the 32 row-fragment addresses would not fit
  // beside the Q, dO and dQ registers: they are formed per read.)
  constexpr bool kAbs = D <= 128;
  unsigned rk[kAbs ? DT : 1], rv[kAbs ? DT : 1], tk[DB][2];
#pragma unroll
  for (int t = 0; t < (kAbs ? DT : 0); ++t) {
    rk[t] = sbase + Ly::OFF_K + (rf_lane[0] ^ (unsigned)(t << 5));
    rv[t] = sbase + Ly::OFF_V + (rf_lane[0] ^ (unsigned)(t << 5));
  }
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) tk[b][hi] = sbase + Ly::OFF_K + trk[b][hi];

  f32x16 dqT[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) dqT[b] = f32x16{};
  f32x16 S[KB], dP[KB];  // [32-key half]
  unsigned dw[KB][8];

  // visible iff key <= qi (causal) and key < N: key <= hi_key
  const int hi_key = CAUSAL ? min(qi, N - 1) : N - 1;

  // VALU group k: dS^T of key half k / 4, rows 8 (k % 4) + 4 half + {0..3},
  // i.e. the bf16 pairs of 16-key step k / 2 of phase C.
  auto vgroup = [&](auto kc, auto mask_c, int j) {
    constexpr int k = decltype(kc)::value, kb = k / 4, g = k % 4;
    constexpr bool MASK = decltype(mask_c)::value;
    float ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = __builtin_amdgcn_exp2f(S[kb][4 * g + e] * c);
      if constexpr (MASK) {
        const int kk = j * kBKdq + 32 * kb + 8 * g + 4 * half + e;
        const unsigned keep = ~(unsigned)((hi_key - kk) >> 31);
        pe = __uint_as_float(__float_as_uint(pe) & keep);
      }
      ds[e] = pe * dP[kb][4 * g + e];
    }
    dw[kb][2 * g] = pack2<T>(ds[0], ds[1]);
    dw[kb][2 * g + 1] = pack2<T>(ds[2], ds[3]);
  };

  // bc: the ring buffer of tile j, as an int or as integral_constant (then
  // every buffer offset is an instruction immediate).
  auto iteration = [&](int j, auto mask_c, auto bc) {
    constexpr bool CT = !std::is_integral_v<decltype(bc)>;
    int b;
    if constexpr (CT)
      b = decltype(bc)::value;
    else
      b = bc;
    // The copies of tile j + 2 ride on phase A's MFMAs, one every
    // kDmaStride; past the last tile they repeat it into the buffer of tile
    // j - 1 (consumed, never read again).
    const int jn = min(j + 2, nkt - 1);
    const int nb = CT ? (b + 2) % kRing : ring(j + 2);
    constexpr int kDmaStride = NA / kDmaPerWave;
    constexpr int BK = [] {
      if constexpr (CT) return decltype(bc)::value * Ly::KTILE;
      else return 0;
    }();
    const unsigned bk = CT ? 0u : (unsigned)(b * Ly::KTILE);
    {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S[kb][r] = ls;
          dP[kb][r] = dn;
        }
      vec8<T> fa[LA];
      auto issue = [&](auto fc) {
        constexpr int F = decltype(fc)::value, kb = F / (2 * DT), t = (F / 2) % DT, X = F % 2;
        if constexpr (kAbs)
          ds_b128<BK + kb * 32 * ROWB>(fa[F % LA], (X ? rv[t] : rk[t]) + bk);
        else
          ds_b128<0>(fa[F % LA], sbase + (X ? Ly::OFF_V : Ly::OFF_K) + (unsigned)(b * Ly::KTILE) +
                                     (rf_lane[kb] ^ (unsigned)(t << 5)));
      };
      static_for<(LA < NA ? LA : NA)>(issue);
      static_for<NA>([&](auto fc) {
        constexpr int F = decltype(fc)::value, kb = F / (2 * DT), t = (F / 2) % DT, X = F % 2;
        constexpr int last = (F + LA - 1 < NA - 1) ? F + LA - 1 : NA - 1;
        asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(fa[F % LA]) : "i"(last - F));
        if constexpr (X == 0)
          S[kb] = mfma(fa[F % LA], qf[t], S[kb]);
        else
          dP[kb] = mfma(fa[F % LA], dof[t], dP[kb]);
        if constexpr (F + LA < NA) issue(ic<F + LA>{});
        if constexpr (F % kDmaStride == 0 && F / kDmaStride < kDmaPerWave)
          dma_op(jn, nb, ic<F / kDmaStride>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    vgroup(ic<0>{}, mask_c, j);
    vgroup(ic<1>{}, mask_c, j);
    {
      s16x4 lo_[LC], hi_[LC];
      auto issue = [&](auto fc) {
        constexpr int F = decltype(fc)::value, u = F / DB, bb = F % DB;
        ds_tr64<BK + u * 16 * ROWB>(lo_[F % LC], tk[bb][0] + bk);
        ds_tr64<BK + u * 16 * ROWB>(hi_[F % LC], tk[bb][1] + bk);
      };
      static_for<(LC < NC ? LC : NC)>(issue);
      static_for<NC>([&](auto fc) {
        constexpr int F = decltype(fc)::value, u = F / DB, bb = F % DB;
        constexpr int last = (F + LC - 1 < NC - 1) ? F + LC - 1 : NC - 1;
        constexpr int kb = u / 2, h2 = u % 2;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo_[F % LC]), "+v"(hi_[F % LC]) : "i"(2 * (last - F)));
        const vec8<T> dsf = __builtin_bit_cast(
            vec8<T>, (u32x4){dw[kb][4 * h2], dw[kb][4 * h2 + 1], dw[kb][4 * h2 + 2], dw[kb][4 * h2 + 3]});
        dqT[bb] = mfma(join<T>(lo_[F % LC], hi_[F % LC]), dsf, dqT[bb]);
        if constexpr (F + LC < NC) issue(ic<F + LC>{});
        // groups 2 (u + 1) and 2 (u + 1) + 1 ride on step u's MFMAs
        constexpr int f = F % DB;
        if constexpr (u < 2 * KB - 1 && DB >= 2 && (f == DB / 2 - 1 || f == DB - 1))
          vgroup(ic<2 * (u + 1) + (f == DB - 1 ? 1 : 0)>{}, mask_c, j);
        if constexpr (u < 2 * KB - 1 && DB == 1) {
          vgroup(ic<2 * (u + 1)>{}, mask_c, j);
          vgroup(ic<2 * (u + 1) + 1>{}, mask_c, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // tile j + 1 must be complete; the copies of tile j + 2 stay in flight
    if (j + 2 < nkt)
      dma_barrier<kDmaPerWave>();
    else
      dma_barrier<0>();
  };

  // Key tiles [0, j_e) need no mask for any wave: every key precedes every
  // query of the workgroup (causal) and lies inside the sequence.
  int j_e = N / kBKdq;
  if (CAUSAL) j_e = min(j_e, q0 / kBKdq);
  j_e = max(0, min(j_e, nkt));

  dma_tile(0);
  if (1 < nkt) {
    dma_tile(1);
    dma_barrier<kDmaPerWave>();
  } else {
    dma_barrier<0>();
  }
  // Unmasked tiles in a loop unrolled by the ring period (tile 0 is in
  // buffer 0, so the buffers are compile-time there), then the rest.
  int j = 0;
  for (; kAbs && j + kRing <= j_e; j += kRing) {
    iteration(j, std::false_type{}, ic<0>{});
    iteration(j + 1, std::false_type{}, ic<1>{});
    iteration(j + 2, std::false_type{}, ic<2>{});
  }
  for (; j < j_e; ++j) iteration(j, std::false_type{}, ring(j));
  for (; j < nkt; ++j) iteration(j, std::true_type{}, ring(j));

  // ---- dQ = scale * (dQ^T)^T: lane writes query qi, d = 32 b + 8 g + 4 half + {0..3}.
  if (qi < N) {
    T* row = dQg + head + (size_t)qi * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        vec4<T> o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (T)(dqT[b][4 * g + e] * scale);
        *(vec4<T>*)(row + 32 * b + 8 * g) = o;
      }
  }
}

template <class T, int D>
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  // Fixed length: statistics [BH][npad]; variable length: [H][ld].
  const int npad = (p.N + kBQ - 1) / kBQ * kBQ;
  VarLen vl{p.cu_seqlens, p.H, p.total, p.cu_seqlens ? varlen_ld(p.total) : 0};
  const size_t stat_rows = p.cu_seqlens ? (size_t)p.H * vl.ld : (size_t)p.BH * npad;
  // P = 2^(c (q.k - L / scale)) with c = scale log2(e).  |c| is kept at
  // least 1e-30 so that L / scale stays finite; below that every
  // c q.k rounds to 0 anyway and P = e^-L as for scale = 0.
  float c = p.scale * kLog2e;
  if (fabsf(c) < 1e-30f) c = c < 0.f ? -1e-30f : 1e-30f;
  float* ls = (float*)p.workspace;
  float* dn = ls + stat_rows;
  const T* q = (const T*)p.q;
  const T* k = (const T*)p.k;
  const T* v = (const T*)p.v;
  const T* dout = (const T*)p.dout;
  {
    constexpr int RPB = 256 / pre_lanes_per_row<D>();
    static_assert(kBQ % RPB == 0, "statistics rows split evenly over the pre kernel's workgroups");
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)(stat_rows / RPB)), dim3(256), 0, stream,
                       (const T*)p.o, dout, p.lse, ls, dn, p.N, npad, kLog2e / c, vl);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (p.N + kBKV - 1) / kBKV;
    const int bhkv = p.BH / p.group;
    const int hsplit = p.part ? p.hsplit : 1;
    const dim3 grid((unsigned)(bhkv * hsplit * dkdv_halves<D>() * nkb)), block(kThreads);
    if (p.causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), grid, block, 0, stream, q, k, v, dout, ls, dn, (T*)p.dk,
                         (T*)p.dv, bhkv, p.N, npad, nkb, c, p.scale, p.group, vl, hsplit, p.part);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), grid, block, 0, stream, q, k, v, dout, ls, dn, (T*)p.dk,
                         (T*)p.dv, bhkv, p.N, npad, nkb, c, p.scale, p.group, vl, hsplit, p.part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (hsplit > 1) {
      const size_t elems = (size_t)bhkv * p.N * D;
      const unsigned blocks = (unsigned)((elems / 8 + 255) / 256);
      hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3(blocks), dim3(256), 0, stream, (const float*)p.part, (T*)p.dk,
                         (T*)p.dv, elems, hsplit);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  {
    const int nqb = (p.N + kBQdq - 1) / kBQdq;
    const dim3 grid((unsigned)(p.BH * nqb)), block(kThreads);
    if (p.causal)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), grid, block, 0, stream, q, k, v, dout, ls, dn, (T*)p.dq,
                         p.BH, p.N, npad, nqb, c, p.scale, p.group, vl);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), grid, block, 0, stream, q, k, v, dout, ls, dn, (T*)p.dq,
                         p.BH, p.N, npad, nqb, c, p.scale, p.group, vl);
    return hipGetLastError();
  }
}

}  // namespace

size_t bwd_workspace_bytes(int BH, int N, int d) {
  (void)d;
  const size_t npad = ((size_t)N + kBQ - 1) / kBQ * kBQ;
  return (size_t)BH * npad * 2 * sizeof(float);
}

// Head split of the grouped-head dK/dV pass: with few (key/value head,
// key block) workgroups the heaviest causal blocks -- which stream every
// query tile of every head of the group -- set the run time, so the group's
// heads are divided over hsplit workgroups that write fp32 partials.
int bwd_head_split(int B, int H, int Hkv, int N) {
  if (Hkv <= 0 || H % Hkv != 0) return 1;
  const int group = H / Hkv;
  const int64_t wgs = (int64_t)B * Hkv * (((int64_t)N + kBKV - 1) / kBKV);
  if (group % 2 != 0 || wgs > kHeadSplitMaxWgs) return 1;
  return (group % 4 == 0 && wgs * 4 <= 2 * kHeadSplitMaxWgs) ? 4 : 2;
}

size_t bwd_part_offset(size_t stats_bytes) { return (stats_bytes + 255) & ~(size_t)255; }

size_t bwd_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  const size_t stats = bwd_workspace_bytes(B * H, N, d);
  const int hs = bwd_head_split(B, H, Hkv, N);
  if (hs == 1) return stats;
  return bwd_part_offset(stats) + 2 * (size_t)hs * B * Hkv * N * d * sizeof(float);
}

size_t bwd_varlen_workspace_bytes(int H, int total, int d) {
  (void)d;
  return (size_t)H * varlen_ld(total) * 2 * sizeof(float);
}

int bwd_block_k() { return kBKV; }
int bwd_block_q() { return kBQ; }

template <class T>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_bwd<T, 32>(p, stream);
    case 64: return launch_bwd<T, 64>(p, stream);
    case 96: return launch_bwd<T, 96>(p, stream);
    case 128: return launch_bwd<T, 128>(p, stream);
    case 256: return launch_bwd<T, 256>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  return launch_bwd_t<__bf16>(p, stream);
}
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t stream) {
  return launch_bwd_t<_Float16>(p, stream);
}

}  // namespace fa
