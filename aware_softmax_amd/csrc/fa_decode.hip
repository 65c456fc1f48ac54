// Decode attention with the key dimension split across workgroups
// ("PidokuInfra 10 -- FlashAttention", section 5, "The decode variant:
// FlashDecoding"), bfloat16 or float16 in/out (a template parameter), fp32
// softmax state, gfx950.
//
// What is computed: one query row per (batch b, head h) against the N
// cached keys and values of its key/value head hk = h / (H / Hkv)
// (H = Hkv is ordinary multi-head attention; H / Hkv > 1 shares one
// key/value head among a group of query heads):
//     o_bh = sum_j softmax_j(scale * q_bh . k_j) v_j,   lse_bh = logsumexp_j(...)
// No mask: the decoded token is the newest position and sees every cached
// key (the causal mask with the query at the end of the sequence).
//
// How (the same section): with one query per sequence, a grid over
// (batch, head) alone has too few workgroups to fill the GPU and each must
// walk all N keys serially.  The keys are split into S chunks; each
// workgroup computes an unnormalised partial (m, l, o~) over its chunk, and
// a second kernel merges the S partials with the online-softmax rescale
// ("FlashAttention: Move Less, Not Compute Less", "Tiling Is Easy; Softmax
// Couples the Entire Row": partials are brought to the common max M by
// exp(m_s - M) before summing), then divides once.
//
// MI355X mapping.  The work is a matrix-vector product per head, bound by
// reading K and V from HBM once; it runs on the VALU (v_dot2_f32_bf16), not
// on MFMA.  A group of LPR lanes (4, 8 or 16) shares one key row, each lane
// holding CPL 16-byte chunks (8 bf16 each) of it, so one wave instruction
// reads 64 x 16 = 1 KiB of K or V in runs of at least 64 contiguous bytes;
// the row's dot product is finished by a DPP reduction inside the lane
// group, which leaves the score in every lane of the group.  Each lane keeps its own online-softmax state (m, l and its
// 8 elements of o~) over the rows it has seen, so the hot loop has no
// cross-lane max at all; the states of a workgroup are merged once at the
// end.  A group of G query heads that share a key/value head is served by
// one workgroup, so K and V are read once for all G.
#include <atomic>
#include <mutex>

#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <class T>
using vec2 = T __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kMfmaMaxHeads = 32;  // heads per workgroup of the MFMA decode (one MFMA column block)
constexpr float kLn2 = 0.69314718055994530942f;

// Row split per head dim: CPL 16-byte chunks per lane, LPR lanes per row
// (d = 32: 4 x 1, 64: 8 x 1, 96: 4 x 3, 128: 16 x 1, 256: 16 x 2); lane cc
// holds chunks cc, cc + LPR, ..., cc + (CPL - 1) LPR of its row.
template <int D>
struct Shape {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "head dim");
  static constexpr int CPL = D == 96 ? 3 : D == 256 ? 2 : 1;
  static constexpr int LPR = D / 8 / CPL;  // lanes per key row
  static constexpr int RPI = 64 / LPR;     // key rows per wave instruction
};

// Largest query-head group one workgroup serves (a divisor of H / Hkv):
// each head keeps 8 CPL fp32 of o~ per lane.
template <int D>
constexpr int max_group() {
  return D >= 256 ? 4 : 8;
}
int max_group_rt(int d) { return d >= 256 ? max_group<256>() : max_group<128>(); }

// Row-group instructions per wave and iteration (K and V each): 8 loads of
// 16 bytes in flight per tensor for groups of up to 4 heads, 4 for larger
// groups; 16 at d = 128 with one or two heads (measured on B8 H32 N32768:
// +1 % with one head, +4 % with two, against 8).
template <int D, int G>
constexpr int unroll() {
  constexpr int loads = (D == 128 && G <= 2) ? 16 : G <= 4 ? 8 : 4;
  return loads / Shape<D>::CPL > 0 ? loads / Shape<D>::CPL : 1;
}

// Rows of one workgroup iteration: every wave reads unroll() instructions
// of RPI rows.
template <int D, int G>
constexpr int rows_per_iter() {
  return kWaves * unroll<D, G>() * Shape<D>::RPI;
}

// Dot product of two packed pairs with an fp32 accumulate (v_dot2), and the
// two fp32 values of a packed pair: bf16 is the high half of an fp32, fp16
// converts exactly.
__device__ __forceinline__ float dot2(__bf16, unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(vec2<__bf16>, a), __builtin_bit_cast(vec2<__bf16>, b), c,
                                         false);
}
__device__ __forceinline__ float dot2(_Float16, unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(vec2<_Float16>, a), __builtin_bit_cast(vec2<_Float16>, b), c,
                                false);
}
__device__ __forceinline__ f32x2 unpack2(__bf16, unsigned u) {
  return f32x2{__builtin_bit_cast(float, u << 16), __builtin_bit_cast(float, u & 0xffff0000u)};
}
// The empty asm keeps the conversion a separate v_cvt_f32_f16: fused into
// the following FMAs it becomes v_fma_mix_f32, which measured half the
// decode throughput (3.3 against 6.4 TB/s with 4 heads per group).
__device__ __forceinline__ f32x2 unpack2(_Float16, unsigned u) {
  f32x2 r = __builtin_convertvector(__builtin_bit_cast(vec2<_Float16>, u), f32x2);
  asm volatile("" : "+v"(r));
  return r;
}

// Sum over the LPR lanes of a key row; every lane of the group gets the sum.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "lane group of 4, 8 or 16");
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1]: sums over each 4-lane quad.
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  // row_half_mirror: lane i of an 8-lane half reads lane 7 - i (the other quad).
  if constexpr (LPR >= 8)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  if constexpr (LPR == 16)  // row_mirror: lane i of a 16-lane row reads lane 15 - i.
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

// Split kernel.  Workgroup index -> (split s, head group hg, b * Hkv + hk).
// part_o  [B*H][S][D]  fp32 unnormalised o~ of each split;
// part_ml [B*H][S][2]  fp32 (m, l) of each split, m in log2 units of the
//                      scaled scores (c = scale * log2 e folded in).
template <class T, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int* __restrict__ seqlens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int H, int Hkv, int N, int S, int chunk, float c) {
  constexpr int LPR = Shape<D>::LPR;
  constexpr int RPI = Shape<D>::RPI;
  constexpr int CPL = Shape<D>::CPL;
  constexpr int E = 8 * CPL;  // elements of a row per lane
  constexpr int U = unroll<D, G>();
  constexpr int ROWS_WAVE = U * RPI;  // rows per wave and iteration
  constexpr float kNegInf = -__builtin_inff();

  const int group = H / Hkv;
  const int n_hg = group / G;
  int wg = blockIdx.x;
  const int s = wg % S;
  wg /= S;
  const int hg = wg % n_hg;
  const int bhk = wg / n_hg;  // b * Hkv + hk
  const int b = bhk / Hkv;
  const int hk = bhk - b * Hkv;
  const int h0 = hk * group + hg * G;  // first query head of this workgroup

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cc = lane % LPR;  // first 16-byte chunk of the row this lane holds
  const int rr = lane / LPR;  // row within a wave instruction

  // Query fragments: the lane's chunks cc + x LPR of each head's query.
  unsigned qf[G][4 * CPL];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int x = 0; x < CPL; ++x) {
      const u32x4 t = *(const u32x4*)(q + ((size_t)b * H + h0 + i) * D + (cc + x * LPR) * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) qf[i][4 * x + w] = t[w];
    }

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = 0.f;
  }

  // Keys of sequence b: the first seqlens[b] rows of the cache (clamped to
  // [0, N]), all N without seqlens.  A split past the end has no keys and
  // writes the empty partial (m = -inf, l = 0, o~ = 0).
  const int n_b = seqlens ? min(max(seqlens[b], 0), N) : N;
  const int k_begin = s * chunk;
  const int k_end = min(n_b, k_begin + chunk);
  const size_t head_off = (size_t)bhk * N * D;
  const T* kh = k + head_off + cc * 8;
  const T* vh = v + head_off + cc * 8;

  for (int r0 = k_begin + wave * ROWS_WAVE; r0 < k_end; r0 += kWaves * ROWS_WAVE) {
    u32x4 kf[U][CPL], vf[U][CPL];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r0 + u * RPI + rr;
      ok[u] = row < k_end;
      const int rc = ok[u] ? row : k_end - 1;  // clamped rows are loaded but scored -inf
#pragma unroll
      for (int x = 0; x < CPL; ++x)
        kf[u][x] = __builtin_nontemporal_load((const u32x4*)(kh + (size_t)rc * D + x * LPR * 8));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r0 + u * RPI + rr;
      const int rc = row < k_end ? row : k_end - 1;
#pragma unroll
      for (int x = 0; x < CPL; ++x)
        vf[u][x] = __builtin_nontemporal_load((const u32x4*)(vh + (size_t)rc * D + x * LPR * 8));
    }
    // V rows as fp32.
    float vv[U][E];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float sc[U];
      float tmax = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < CPL; ++x)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc = dot2(T{}, qf[i][4 * x + t], kf[u][x][t], acc);
        acc = row_sum<LPR>(acc);
        sc[u] = ok[u] ? acc * c : kNegInf;
        tmax = fmaxf(tmax, sc[u]);
      }
      const float m_new = fmaxf(m[i], tmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;  // no visible row yet: nothing to add
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_use);
      m[i] = m_new;
      float ls = 0.f;
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = __builtin_amdgcn_exp2f(sc[u] - m_use);
        ls += p[u];
      }
      l[i] = l[i] * alpha + ls;
      if (i == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int x = 0; x < CPL; ++x)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const f32x2 pr = unpack2(T{}, vf[u][x][t]);
              vv[u][8 * x + 2 * t] = pr[0];
              vv[u][8 * x + 2 * t + 1] = pr[1];
            }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float acc = o[i][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) acc = fmaf(p[u], vv[u][e], acc);
        o[i][e] = acc;
      }
    }
  }

  // Merge the RPI row groups of the wave (lanes cc, cc + LPR, ...), then the
  // waves through LDS.  A state with no visible row has m = -inf, l = 0,
  // o~ = 0 and gets weight 0.
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float mm = m[i];
#pragma unroll
    for (int sh = LPR; sh < 64; sh <<= 1) mm = fmaxf(mm, __shfl_xor(mm, sh));
    const float w = __builtin_amdgcn_exp2f(m[i] - (mm == kNegInf ? 0.f : mm));
    float ll = l[i] * w;
    float oo[E];
#pragma unroll
    for (int e = 0; e < E; ++e) oo[e] = o[i][e] * w;
#pragma unroll
    for (int sh = LPR; sh < 64; sh <<= 1) {
      ll += __shfl_xor(ll, sh);
#pragma unroll
      for (int e = 0; e < E; ++e) oo[e] += __shfl_xor(oo[e], sh);
    }
    if (rr == 0) {
#pragma unroll
      for (int x = 0; x < CPL; ++x)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_o[wave][i][(cc + x * LPR) * 8 + e] = oo[8 * x + e];
      if (cc == 0) {
        sm_m[wave][i] = mm;
        sm_l[wave][i] = ll;
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += kThreads) {
    const int i = t / D;
    const int e = t - i * D;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][i]);
    const float mref = mm == kNegInf ? 0.f : mm;  // -inf: the split has no key
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[w][i] - mref);
      ll = fmaf(wt, sm_l[w][i], ll);
      oo = fmaf(wt, sm_o[w][i][e], oo);
    }
    const size_t row = ((size_t)b * H + h0 + i) * S + s;
    part_o[row * D + e] = oo;
    if (e == 0) {
      part_ml[row * 2] = mm;
      part_ml[row * 2 + 1] = ll;
    }
  }
}

// Combine kernel: one workgroup of D threads per (b, h).  M = max_s m_s,
// l = sum_s 2^(m_s - M) l_s, o = sum_s 2^(m_s - M) o~_s / l, and
// lse = ln 2 * (M + log2 l) (m is in log2 units).
template <class T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, T* __restrict__ o,
                                                           float* __restrict__ lse, int S) {
  const int bh = blockIdx.x;
  const int e = threadIdx.x;
  const float* ml = part_ml + (size_t)bh * S * 2;
  const float* po = part_o + (size_t)bh * S * D + e;
  float mm = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < S; ++s) mm = fmaxf(mm, ml[2 * s]);
  const float mref = mm == -__builtin_inff() ? 0.f : mm;  // -inf: the sequence has no key
  float ll = 0.f, oo = 0.f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float wt = __builtin_amdgcn_exp2f(ml[2 * s] - mref);
    ll = fmaf(wt, ml[2 * s + 1], ll);
    oo = fmaf(wt, po[(size_t)s * D], oo);
  }
  // No key at all: o = 0 and lse = -inf (an empty softmax row).
  o[(size_t)bh * D + e] = (T)(ll > 0.f ? oo / ll : 0.f);
  if (e == 0) lse[bh] = ll > 0.f ? (mm + __builtin_amdgcn_logf(ll)) * kLn2 : -__builtin_inff();
}

// Largest divisor of the query-head group that one workgroup serves.
// d = 64 or 128 with 5 or more heads per key/value head runs the MFMA decode,
// which serves up to 32 heads of a group per workgroup.  Measured on B8
// N32768 d128 (same box): 8 heads per key/value head 4.1-4.3 -> 6.0-6.3
// TB/s, 6 heads 5.1 -> 6.2 (d = 64, 8 heads: 3.8 -> 5.2-5.5); at 4 heads
// the VALU kernel stays ahead (6.45 against 6.3 TB/s).
bool mfma_path(int group, int d) { return (d == 64 || d == 128) && group >= 5; }

int heads_per_wg(int group, int d) {
  if (mfma_path(group, d)) {
    for (int g = kMfmaMaxHeads; g > 1; --g)
      if (group % g == 0) return g;
  }
  for (int g = max_group_rt(d); g > 1; --g)
    if (group % g == 0) return g;
  return 1;
}

// ---------------------------------------------------------------------------
// MFMA decode (d = 64 or 128, 5 to 32 query heads of a group per workgroup).  The
// VALU kernel above spends about 11 VALU instructions per head and key on
// the dot product, its lane reduction, the softmax and P.V; with 8 heads per
// key/value head that issue rate, not HBM, bounds it.  Here the group's
// heads are the 32 query columns of the forward's tiles: S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16 (columns past the group are zero),
// the softmax runs in-lane per head column as in the forward, and P is
// rounded to the element type for the MFMA (the forward's precision, not
// the VALU kernel's fp32 P).  Each of the 4 waves takes its own 32-key tile
// of a 128-key LDS stage (staged through registers, the next stage's loads
// in flight during the current one); the waves' (m, l, o~) are merged once
// at the end and written as the split's partial for the combine kernel.
namespace mf {
constexpr int kKeys = 32;               // keys per wave tile
constexpr int kStage = kWaves * kKeys;  // keys per LDS stage
template <int D>
struct Layout {
  static constexpr int KS = D + 8;   // K row stride (elements, +16 B)
  static constexpr int VS = D + 16;  // V row stride (elements, +32 B)
  static constexpr int K_ELEMS = kStage * KS;
  static constexpr int STAGE = K_ELEMS + kStage * VS;
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int CPT = kStage * CPR / kThreads;
  static_assert(kStage * CPR % kThreads == 0, "stage splits evenly over threads");
};
}  // namespace mf

template <class T>
using vec8 = T __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma32(const vec8<__bf16>& a, const vec8<__bf16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const vec8<_Float16>& a, const vec8<_Float16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// Lane l receives x from lane l ^ 32; returns the max or the sum of the two.
__device__ __forceinline__ float swap_halves(float x, bool want_max) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]);
  const float b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}
// Two transposing 8-byte LDS reads -> the 8 elements of one V^T operand.
template <class T>
__device__ __forceinline__ vec8<T> read_vt(const T* p0, const T* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  return __builtin_bit_cast(vec8<T>, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <class T, int D>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int* __restrict__ seqlens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int H, int Hkv, int N, int S, int chunk, float c,
    int G) {
  using namespace mf;
  using Ly = Layout<D>;
  constexpr int KS = Ly::KS, VS = Ly::VS, K_ELEMS = Ly::K_ELEMS, STAGE = Ly::STAGE, CPR = Ly::CPR, CPT = Ly::CPT;
  constexpr float kNegInf = -__builtin_inff();
  constexpr int DT = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) T smem[STAGE];

  const int group = H / Hkv;
  const int n_hg = group / G;
  int wg = blockIdx.x;
  const int s = wg % S;
  wg /= S;
  const int hg = wg % n_hg;
  const int bhk = wg / n_hg;  // b * Hkv + hk
  const int b = bhk / Hkv;
  const int hk = bhk - b * Hkv;
  const int h0 = hk * group + hg * G;  // first query head of this workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // head column h0 + col
  const int half = lane >> 5;

  // Q^T fragments (B operand): head h0 + col, d = 16 t + 8 half .. + 7.
  vec8<T> qf[DT];
  if (col < G) {
    const vec8<T>* src = (const vec8<T>*)(q + ((size_t)b * H + h0 + col) * D + half * 8);
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = src[2 * t];
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = vec8<T>{};
  }

  const int n_b = seqlens ? min(max(seqlens[b], 0), N) : N;
  const int k_begin = s * chunk;
  const int k_end = min(n_b, k_begin + chunk);
  const int nst = k_end > k_begin ? (k_end - k_begin + kStage - 1) / kStage : 0;
  const size_t head_off = (size_t)bhk * N * D;
  const T* kh = k + head_off;
  const T* vh = v + head_off;

  f32x16 oacc[DB];
#pragma unroll
  for (int bb = 0; bb < DB; ++bb) oacc[bb] = f32x16{};
  float m_run = kNegInf;
  float l_part = 0.f;

  vec8<T> kreg[CPT], vreg[CPT];
  auto gload = [&](int j) {
    const int r0 = k_begin + j * kStage;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / CPR;
      const int c8 = ci % CPR;
      const int key = r0 + row;
      if (key < k_end) {
        const size_t off = (size_t)key * D + c8 * 8;
        kreg[i] = __builtin_nontemporal_load((const vec8<T>*)(kh + off));
        vreg[i] = __builtin_nontemporal_load((const vec8<T>*)(vh + off));
      } else {
        kreg[i] = vec8<T>{};
        vreg[i] = vec8<T>{};
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / CPR;
      const int c8 = ci % CPR;
      *(vec8<T>*)(smem + row * KS + c8 * 8) = kreg[i];
      *(vec8<T>*)(smem + K_ELEMS + row * VS + c8 * 8) = vreg[i];
    }
  };

  const int tr_e = (lane & 15) >> 2;
  const int tr_t = lane & 3;
  const int tr_cg = (lane >> 4) & 1;

  if (nst > 0) {
    gload(0);
    lstore();
  }
  __syncthreads();
  for (int j = 0; j < nst; ++j) {
    if (j + 1 < nst) gload(j + 1);
    const int kt0 = k_begin + j * kStage + wave * kKeys;  // this wave's 32 keys
    if (kt0 < k_end) {
      // S^T[key][head]: register r of lane (col, half) is key kt0 + 8 (r/4) + 4 half + r%4.
      const T* krow = smem + (wave * kKeys + col) * KS + half * 8;
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t) sacc = mfma32(*(const vec8<T>*)(krow + 16 * t), qf[t], sacc);
      const int lim = k_end - kt0 - half * 4;  // key offsets >= lim lie past the split
      float sv[16];  // scaled scores (log2 units); c may be negative
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        sv[r] = off < lim ? sacc[r] * c : kNegInf;
        mx = fmaxf(mx, sv[r]);
      }
      mx = swap_halves(mx, true);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      float lsum = l_part * alpha;
      vec8<T> pf[2];  // B operands of the two 16-key steps
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        unsigned w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = sv[u * 8 + e], x1 = sv[u * 8 + e + 1];
          const float p0 = x0 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x0 - m_use);
          const float p1 = x1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x1 - m_use);
          const vec2<T> pr = __builtin_convertvector((f32x2){p0, p1}, vec2<T>);
          // the converted values in fp32 (a v_dot2 would wait for the matrix pipe)
          lsum += (float)pr[0] + (float)pr[1];
          w[e >> 1] = __builtin_bit_cast(unsigned, pr);
        }
        pf[u] = __builtin_bit_cast(vec8<T>, (u32x4){w[0], w[1], w[2], w[3]});
      }
      l_part = lsum;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) oacc[bb] *= alpha;
      }
      const T* vl = smem + K_ELEMS + wave * kKeys * VS;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const T* vrow = vl + (u * 16 + half * 4 + tr_e) * VS + tr_cg * 16 + 4 * tr_t;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) oacc[bb] = mfma32(read_vt(vrow + bb * 32, vrow + bb * 32 + 8 * VS), pf[u], oacc[bb]);
      }
    }
    __syncthreads();
    if (j + 1 < nst) lstore();
    __syncthreads();
  }

  // Merge the 4 waves: [16 DB + 2][4 waves][64 lanes] fp32 in the stage
  // (free after the loop's last barrier); wave w then merges d block w.
  constexpr int NV = 16 * DB + 2;
  static_assert(NV * kThreads * 4 <= (int)sizeof(smem), "merge buffer fits the stage");
  static_assert(DB <= kWaves, "at most one output block per wave");
  float* xb = (float*)smem;
#pragma unroll
  for (int bb = 0; bb < DB; ++bb)
#pragma unroll
    for (int r = 0; r < 16; ++r) xb[(bb * 16 + r) * kThreads + tid] = oacc[bb][r];
  xb[16 * DB * kThreads + tid] = m_run;
  xb[(16 * DB + 1) * kThreads + tid] = l_part;
  __syncthreads();
  float mw[kWaves], mm = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = xb[16 * DB * kThreads + w * 64 + lane];
    mm = fmaxf(mm, mw[w]);
  }
  const float mref = mm == kNegInf ? 0.f : mm;  // no key in the split: all weights 0
  float ll = 0.f, oo[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) oo[r] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float wt = __builtin_amdgcn_exp2f(mw[w] - mref);
    ll = fmaf(wt, xb[(16 * DB + 1) * kThreads + w * 64 + lane], ll);
    if (wave < DB) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oo[r] = fmaf(wt, xb[(wave * 16 + r) * kThreads + w * 64 + lane], oo[r]);
    }
  }
  const float l_tot = swap_halves(ll, false);
  if (wave < DB && col < G) {
    const size_t row = ((size_t)b * H + h0 + col) * S + s;
    float* dst = part_o + row * D + wave * 32 + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) *(float4*)(dst + 8 * g) = make_float4(oo[4 * g], oo[4 * g + 1], oo[4 * g + 2], oo[4 * g + 3]);
    if (wave == 0 && half == 0) {
      part_ml[row * 2] = mm;
      part_ml[row * 2 + 1] = l_tot;
    }
  }
}

template <int D>
int rows_per_iter_rt(int G) {
  switch (G) {
    case 1: return rows_per_iter<D, 1>();
    case 2: return rows_per_iter<D, 2>();
    case 3: return rows_per_iter<D, 3>();
    case 4: return rows_per_iter<D, 4>();
    case 5: return rows_per_iter<D, 5>();
    case 6: return rows_per_iter<D, 6>();
    case 7: return rows_per_iter<D, 7>();
    default: return rows_per_iter<D, 8>();
  }
}

int rows_per_iter_d(int d, int G) {
  if ((d == 64 || d == 128) && G >= 5) return mf::kStage;  // the MFMA decode's LDS stage
  switch (d) {
    case 32: return rows_per_iter_rt<32>(G);
    case 64: return rows_per_iter_rt<64>(G);
    case 96: return rows_per_iter_rt<96>(G);
    case 128: return rows_per_iter_rt<128>(G);
    default: return rows_per_iter_rt<256>(G);
  }
}

template <class T, int D, int G>
hipError_t launch_g(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  const float c = p.scale * kLog2e;
  float* po = (float*)p.workspace;
  float* pml = (float*)((char*)p.workspace + plan.ml_offset);
  hipLaunchKernelGGL((decode_split_kernel<T, D, G>), dim3(plan.split_wgs), dim3(kThreads), 0, stream,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, p.seqlens, po, pml, p.H, p.Hkv, p.N,
                     plan.splits, plan.chunk, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.B * p.H), dim3(D), 0, stream, (const float*)po,
                     (const float*)pml, (T*)p.o, p.lse, plan.splits);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_mfma(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  const float c = p.scale * kLog2e;
  float* po = (float*)p.workspace;
  float* pml = (float*)((char*)p.workspace + plan.ml_offset);
  hipLaunchKernelGGL((decode_mfma_kernel<T, D>), dim3(plan.split_wgs), dim3(kThreads), 0, stream, (const T*)p.q,
                     (const T*)p.k, (const T*)p.v, p.seqlens, po, pml, p.H, p.Hkv, p.N, plan.splits, plan.chunk, c,
                     plan.heads_per_wg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.B * p.H), dim3(D), 0, stream, (const float*)po,
                     (const float*)pml, (T*)p.o, p.lse, plan.splits);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_d(const DecodeParams& p, const DecodePlan& plan, hipStream_t stream) {
  if constexpr (D == 64 || D == 128) {
    if (plan.heads_per_wg >= 5) return launch_mfma<T, D>(p, plan, stream);
  }
  if constexpr (max_group<D>() == 4) {
    switch (plan.heads_per_wg) {
      case 1: return launch_g<T, D, 1>(p, plan, stream);
      case 2: return launch_g<T, D, 2>(p, plan, stream);
      case 3: return launch_g<T, D, 3>(p, plan, stream);
      default: return launch_g<T, D, 4>(p, plan, stream);
    }
  } else {
    switch (plan.heads_per_wg) {
      case 1: return launch_g<T, D, 1>(p, plan, stream);
      case 2: return launch_g<T, D, 2>(p, plan, stream);
      case 3: return launch_g<T, D, 3>(p, plan, stream);
      case 4: return launch_g<T, D, 4>(p, plan, stream);
      case 5: return launch_g<T, D, 5>(p, plan, stream);
      case 6: return launch_g<T, D, 6>(p, plan, stream);
      case 7: return launch_g<T, D, 7>(p, plan, stream);
      default: return launch_g<T, D, 8>(p, plan, stream);
    }
  }
}

}  // namespace

// Split plan.  Chunks are whole workgroup iterations; with num_splits = 0
// the count aims at kTargetWgs workgroups in all, two per CU: measured over
// batch 1-16, 8-64 heads, group sizes 1-8 and N = 8K-128K, one or two
// resident workgroups per CU (each wave with 8-16 KiB of loads in flight)
// already saturate HBM, and more splits only add partials and tail.
DecodePlan decode_plan(int B, int H, int Hkv, int N, int d, int num_splits) {
  constexpr int64_t kTargetWgs = 512;
  DecodePlan pl{};
  const int group = H / Hkv;
  pl.heads_per_wg = heads_per_wg(group, d);
  const int rows = rows_per_iter_d(d, pl.heads_per_wg);
  const int64_t iters = ((int64_t)N + rows - 1) / rows;
  const int64_t base = (int64_t)B * Hkv * (group / pl.heads_per_wg);
  int64_t want = num_splits > 0 ? num_splits : (kTargetWgs + base - 1) / base;
  if (want > iters) want = iters;
  if (want < 1) want = 1;
  const int64_t iters_per_split = (iters + want - 1) / want;
  pl.chunk = (int)(iters_per_split * rows);
  pl.splits = (int)(((int64_t)N + pl.chunk - 1) / pl.chunk);
  pl.split_wgs = base * pl.splits;
  const size_t rows_bh = (size_t)B * H * pl.splits;
  pl.ml_offset = (rows_bh * d * sizeof(float) + 255) & ~(size_t)255;
  pl.workspace_bytes = pl.ml_offset + rows_bh * 2 * sizeof(float);
  return pl;
}

int decode_rows_per_iter(int d, int heads_per_wg) { return rows_per_iter_d(d, heads_per_wg); }

template <class T>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  const DecodePlan plan = decode_plan(p.B, p.H, p.Hkv, p.N, p.d, p.num_splits);
  switch (p.d) {
    case 32: return launch_d<T, 32>(p, plan, stream);
    case 64: return launch_d<T, 64>(p, plan, stream);
    case 96: return launch_d<T, 96>(p, plan, stream);
    case 128: return launch_d<T, 128>(p, plan, stream);
    case 256: return launch_d<T, 256>(p, plan, stream);
  }
  return hipErrorInvalidValue;
}

// Scratch of fa_decode_static: the split partials (o~, m, l) of
// decode_plan's workspace layout, for callers that cannot allocate.  One
// copy per device, held by the loaded code object until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// is only a stand-in for the device symbol): its device address is looked
// up once per device with hipGetSymbolAddress and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) { return launch_decode_t<__bf16>(p, stream); }
hipError_t launch_decode_f16(const DecodeParams& p, hipStream_t stream) { return launch_decode_t<_Float16>(p, stream); }

}  // namespace fa
