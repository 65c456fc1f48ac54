// FlashAttention-2 forward, bfloat16 or float16 in/out, fp32 softmax state,
// gfx950 MFMA (v_mfma_f32_32x32x16_bf16 / _f16; the element type is a
// template parameter, everything else is shared).
//
// What is computed (per batch*head, per query row i):
//   O_i = sum_j softmax_j(scale * q_i . k_j + mask_ij) v_j,  L_i = logsumexp_j(...)
// How ("FlashAttention-2: Why the Attention Bottleneck Wasn't Where Everyone
// Was Looking", sections "FA2 change #1" to "#3" and "The causal masking
// freebie"; "FlashAttention: Move Less, Not Compute Less", section "Tiling Is
// Easy; Softmax Couples the Entire Row"):
//   * one workgroup per (head, block of kBQ query rows); the Q block and the
//     running state (m, l, unnormalised O) stay in registers while key/value
//     tiles of kBK rows stream through LDS (outer loop over query blocks);
//   * split-Q: each wave64 owns 32 query rows of the block and the whole
//     key tile, so no partial results cross waves;
//   * per tile: S^T = K Q^T on MFMA, mask only on tiles that cross the
//     diagonal or the ragged end, m' = max(m, rowmax), alpha = 2^(m - m'),
//     P = 2^(S*c - m'), l = alpha*l + rowsum(P), O^T = alpha*O^T + V^T P^T
//     on MFMA; one reciprocal of l per row at the end, L = ln2*(m + log2 l);
//   * tiles entirely above a wave's diagonal are never computed.
//
// MI355X mapping (both kernels):
//   * scores are computed transposed (keys x queries) with
//     v_mfma_f32_32x32x16_bf16, so each lane holds 32 scores of ONE query:
//     row max and row sum are in-lane plus one permlane32 swap;
//   * the fp32 score accumulator, exponentiated and packed to bf16, is
//     directly the B operand of the P.V MFMA (the key order inside a 16-key
//     step is permuted consistently on both operands);
//   * V^T operands come from the row-major V tile through ds_read_b64_tr_b16
//     (the gfx950 transposing LDS read), so V is stored in LDS as it sits in
//     HBM;
//   * exp is the hardware exp2 with scale*log2(e) folded into one FMA.
// Two kernels (and an e4m3 variant of each):
//   * d = 256, and d = 96 on grids of fewer 256-row blocks than CUs: 4
//     waves, 128 query rows per workgroup, K/V tiles staged through
//     registers into padded, double-buffered LDS rows;
//   * d = 32, 64, 96, 128 ("duo"): 8 waves (two per SIMD), 256 query rows
//     (128 with two wave groups over the key tiles on small grids, d = 32
//     and 64), K/V tiles copied HBM -> LDS by LDS-DMA into XOR-swizzled
//     rings (d = 32 and 96 in the LDS rows of d = 64 and 128), the 32
//     softmax slots of an interval spread one to four per MFMA; steady
//     tiles skip the row max (fixed reference max with an overflow check,
//     see below).
#include <math.h>
#include <stdlib.h>

#include "fa_internal.h"
#include "fa_schedule.h"
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {
namespace {

template <class T>
using vec8 = T __attribute__((ext_vector_type(8)));
template <class T>
using vec4 = T __attribute__((ext_vector_type(4)));
template <class T>
using vec2 = T __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The two 16-bit element types: MFMA, the fp32 pair -> element pair
// conversion (round to nearest even) and the fp32 sum of a converted pair.
// Row sums of P are fp32 adds, not v_dot2 of the packed pair with (1, 1):
// on gfx950 a v_dot2 waits for the SIMD's matrix pipe, so beside the other
// wave's MFMAs it runs several times slower than the adds that replace it
// (measured: a softmax instruction mix ran 1.8x faster beside an MFMA
// stream with adds).
__device__ __forceinline__ f32x16 mfma32(const vec8<__bf16>& a, const vec8<__bf16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const vec8<_Float16>& a, const vec8<_Float16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
template <class T>
__device__ __forceinline__ vec2<T> cvt2(float a, float b) {
  return __builtin_convertvector((f32x2){a, b}, vec2<T>);
}
// Sum of the two converted values, exactly as the P.V product sees them
// (for bf16 a shift and a mask recover them as fp32).
template <class T>
__device__ __forceinline__ float sum2(vec2<T> pr) {
  return (float)pr[0] + (float)pr[1];
}

constexpr int kBQ = 128;  // query rows per workgroup
constexpr int kBK = 64;   // keys per streamed tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kBQ / kWaves;  // 32 = one MFMA column block
static_assert(kRowsPerWave == 32, "one 32-wide MFMA block of queries per wave");

// One LDS stage holds G consecutive key tiles, one per wave group: with
// G = 2 the workgroup's two groups of 4 waves take alternate tiles of the
// same query rows and merge their (m, l, O) once at the end.
// V tile row stride in elements.  A transposing 8-byte read is served 32
// lanes at a time over the LDS's 64 banks, and those lanes read 64 bytes
// from each of 4 consecutive rows; they are conflict-free when the row
// stride is 64 or 192 bytes modulo 256, so rows of 32 or 96 elements are
// left as they are and the others get 32 elements of pad.
constexpr int v_row_elems(int d) { return (d % 128 == 32 || d % 128 == 96) ? d : d + 32; }

template <int D, int G, int OS = 1>
struct Layout {
  static constexpr int THREADS = kThreads * G * OS;
  static constexpr int KEYS = kBK * G;  // keys per stage
  static constexpr int KS = D + 8;      // K tile row stride in elements (+16 B)
  static constexpr int VS = v_row_elems(D);  // V tile row stride in elements
  static constexpr int K_ELEMS = KEYS * KS;
  static constexpr int V_ELEMS = KEYS * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS_PER_ROW = D / 8;                    // 16-byte chunks
  static constexpr int CHUNKS_PER_THREAD = KEYS * D / 8 / THREADS;
  static_assert(KEYS * D / 8 % THREADS == 0, "tile splits evenly over threads");
};

__device__ inline float swap_halves(float x, bool want_max) {
  // Lane l receives x from lane l ^ 32; returns max or sum of the two.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]);
  const float b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}

template <class T>
__device__ inline vec8<T> read_vt(const T* p0, const T* p1) {
  // Two transposing 8-byte LDS reads -> the 8 bf16 of one MFMA A operand.
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(vec8<T>, v);
}

// Raw LDS addressing: 32-bit byte addresses kept in VGPRs, so each operand
// read is one ds_read with a compile-time immediate offset.
__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Offset, within a 64-key tile, of score i of a lane (i = 16*kb + r for the
// two 32-key MFMA halves kb and accumulator register r), without the
// lane's 4*half: kb*32 + (r/4)*8 + r%4.
__device__ constexpr int score_key_offset(int i) { return (i >> 4) * 32 + ((i >> 2) & 3) * 8 + (i & 3); }

// Where the rows of query head bh live.  Fixed length: q, o [BH][N][D],
// k, v [BH / group][N][D], L [BH][N].  Variable length (cu_seqlens, B + 1
// offsets into `total` packed rows per head): q, o [H][total][D], k, v
// [H / group][total][D], L [H][total]; bh = h B + b (head-major: the
// schedule gives each XCD a contiguous range of bh, so every XCD gets the
// same heads of every sequence and the same share of the work whatever the
// lengths), and sequence b holds rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1
// of every head.  Query heads of a group are consecutive, so head h reads
// key/value head h / group.
struct HeadRows {
  size_t q, kv, l;  // element offsets of row 0 of the Q/O head, the K/V head, the L row
  int n;            // rows of the sequence
};
__device__ inline HeadRows head_rows(int bh, int BH, int group, int N, int D, const int* cu_seqlens, int H,
                                     int total) {
  HeadRows r;
  if (cu_seqlens) {
    const int B = BH / H;
    const int h = bh / B, b = bh - h * B;
    // offsets clamped to [0, total], so no row outside the packed tensors is
    // ever addressed, whatever the array holds
    const int r0 = min(max(cu_seqlens[b], 0), total);
    r.n = min(max(cu_seqlens[b + 1], r0), total) - r0;
    r.l = (size_t)h * total + r0;
    r.q = r.l * D;
    r.kv = ((size_t)(h / group) * total + r0) * D;
  } else {
    r.n = N;
    r.l = (size_t)bh * N;
    r.q = r.l * D;
    r.kv = (size_t)(bh / group) * N * D;
  }
  return r;
}

// Online-softmax update of one 64-key tile for the lane's query row
// ("FlashAttention-2: ...", "FA2 change #1"; "FlashAttention: Move Less,
// Not Compute Less", "Tiling Is Easy"): sv holds the lane's 32 raw scores
// q.k (the other 32 of the row sit in lane ^ 32).  m_run is the running
// max in log2 units (scores times c = scale*log2 e), l_part the lane's
// partial row sum.  Writes P = 2^(s*c - m') as bf16 MFMA B-operand
// fragments and returns alpha = 2^(m - m') for rescaling O.
//   MASK: the tile crosses the causal diagonal or the end of the sequence;
//   scores with key offset > lim_causal (causal) or >= lim_n are replaced
//   by -inf before any arithmetic.  Unmasked tiles run no per-score compare
//   or select at all.  c must be > 0 (a zero scale is raised to 1e-30 by
//   the caller: every P of a row is then exactly 1 in fp32, as for scale 0,
//   while -inf * c stays -inf for hidden keys).
template <bool MASK, bool CAUSAL, class T>
__device__ inline float tile_softmax(float (&sv)[32], float c, int lim_causal, int lim_n, float& m_run,
                                     float& l_part, vec8<T> (&pfrag)[4]) {
  if (MASK) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int off = score_key_offset(i);
      if ((CAUSAL && off > lim_causal) || off >= lim_n) sv[i] = -INFINITY;
    }
  }
  float mx[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) mx[q] = fmaxf(sv[2 * q], sv[2 * q + 1]);
#pragma unroll
  for (int i = 8; i < 32; i += 8)
#pragma unroll
    for (int q = 0; q < 4; ++q) mx[q] = fmaxf(mx[q], fmaxf(sv[i + 2 * q], sv[i + 2 * q + 1]));
  const float mrow = swap_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])), true);
  float m_new, m_use;
  if (MASK) {  // a row may see no key of this tile (mrow = -inf)
    const float mc = (mrow == -INFINITY) ? -INFINITY : mrow * c;
    m_new = fmaxf(m_run, mc);
    m_use = (m_new == -INFINITY) ? 0.f : m_new;
  } else {
    m_new = fmaxf(m_run, mrow * c);
    m_use = m_new;
  }
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  m_run = m_new;
  float lsum = l_part * alpha;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    unsigned w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float x0 = sv[u * 8 + e], x1 = sv[u * 8 + e + 1];
      // c > 0 (the kernels raise a zero scale to 1e-30), so a hidden
      // score gives 2^(-inf) = 0 with no select
      const float p0 = __builtin_amdgcn_exp2f(fmaf(x0, c, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(x1, c, -m_use));
      const vec2<T> pr = cvt2<T>(p0, p1);
      lsum += sum2(pr);
      w[e >> 1] = __builtin_bit_cast(unsigned, pr);
    }
    pfrag[u] = __builtin_bit_cast(vec8<T>, (u32x4){w[0], w[1], w[2], w[3]});
  }
  l_part = lsum;
  return alpha;
}

// Any d that is a multiple of 32 (one 32-wide output block per step); two
// workgroups per CU up to d = 128, one at d = 256 (O^T alone is 128 fp32
// per lane there, and two K/V stages take 137 KB of LDS).
//
// G = 2 (grids too small to fill the chip): 8 waves in two groups of 4 over
// the same 128 query rows; group g takes the key tiles 2j + g, so the
// longest chain of dependent tiles -- the last causal row block scans every
// key -- is halved.  At the end group 1 hands its running max, partial sums
// and O^T to group 0 through LDS, which rescales both to the common max
// (the merge rule of the online softmax) and writes the output.
//
// Register budget (launch bound): 4 workgroups per CU at d = 32, 3 at
// d = 64, 2 up to d = 128 -- without it hipcc gave the non-causal d = 64
// kernel 178 VGPRs (two workgroups per CU) and ran it 15 % slower.
//
// OS = 2 (d = 256): 8 waves, two per 32 query rows; both compute S and the
// softmax of their rows, and each keeps O^T for one half of d (64 fp32 per
// lane instead of 128), which fits two waves per SIMD without spilling.
// Q.K^T is done twice (1.5x the MFMA work); measured 521 -> 640 TFLOP/s on
// B8 H32 N8192 d256 causal (same box, identical output bits).
template <class T, int D, bool CAUSAL, int G, int OS = 1>
__global__ __launch_bounds__(kThreads * G * OS, (D >= 256 || G == 2 || OS == 2) ? 1 : D <= 32 ? 4 : D <= 64 ? 3 : 2) void fwd_mfma_kernel(
    const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
    T* __restrict__ Og, float* __restrict__ Lg, int BH, int N, int nqb, float c, int negate,
    int group, const int* __restrict__ cu_seqlens, int H, int total) {
  using Ly = Layout<D, G, OS>;
  static_assert(G == 1 || OS == 1, "one kind of split at a time");
  constexpr int DT = D / 16;       // 16-wide d steps of the QK^T contraction
  constexpr int DB = D / 32 / OS;  // 32-wide d blocks of the output held by this wave
  __shared__ __attribute__((aligned(16))) T smem[2 * Ly::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = (tid >> 6) & (kWaves - 1);  // query rows of the wave
  const int grp = G == 1 ? 0 : tid >> 8;       // key tiles of the wave
  const int dh = OS == 1 ? 0 : tid >> 8;       // d range of O held by the wave
  const int col = lane & 31;   // query column of the transposed tiles
  const int half = lane >> 5;  // which 4-key group of each 8 (MFMA layout)
  c = fmaxf(c, 1e-30f);        // tile_softmax needs c > 0 (scale 0: every P is 1)

  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL ? Order::HeavyLast : Order::Plain, &bh, &qb);
  const int q0 = qb * kBQ;
  HeadRows hr = head_rows(bh, BH, group, N, D, cu_seqlens, H, total);
  if (cu_seqlens) {
    N = hr.n;
    if (q0 >= N) return;  // past the end of this sequence (the whole workgroup)
  }
  const size_t head = hr.q;
  const T* Qh = Qg + head;
  const T* Kh = Kg + hr.kv;
  const T* Vh = Vg + hr.kv;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop
  const int qw = q0 + wave * kRowsPerWave;  // first query row of this wave
  const int qi = qw + col;                  // this lane's query row
  vec8<T> qf[DT];
  if (qi < N) {
    const vec8<T>* src = (const vec8<T>*)(Qh + (size_t)qi * D + half * 8);
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = src[2 * t];
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = vec8<T>{};
  }
  if (negate) {  // scale < 0: use -Q and |scale| (negation is exact)
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 u = __builtin_bit_cast(u32x4, qf[t]) ^ 0x80008000u;
      qf[t] = __builtin_bit_cast(vec8<T>, u);
    }
  }

  int nkt = (N + Ly::KEYS - 1) / Ly::KEYS;  // LDS stages
  if (CAUSAL) nkt = min(nkt, (q0 + kBQ - 1) / Ly::KEYS + 1);

  // ---- running state: O^T blocks (d x queries), m in log2 units, partial l
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // ---- global -> register prefetch, register -> LDS store
  vec8<T> kreg[Ly::CHUNKS_PER_THREAD], vreg[Ly::CHUNKS_PER_THREAD];
  auto gload = [&](int j) {
    const int kt0 = j * Ly::KEYS;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS_PER_THREAD; ++i) {
      const int ci = tid + Ly::THREADS * i;
      const int row = ci / Ly::CHUNKS_PER_ROW;
      const int c8 = ci % Ly::CHUNKS_PER_ROW;
      const int key = kt0 + row;
      if (key < N) {
        const size_t off = (size_t)key * D + c8 * 8;
        kreg[i] = *(const vec8<T>*)(Kh + off);
        vreg[i] = *(const vec8<T>*)(Vh + off);
      } else {
        kreg[i] = vec8<T>{};
        vreg[i] = vec8<T>{};
      }
    }
  };
  auto lstore = [&](int buf) {
    T* Kl = smem + buf * Ly::STAGE;
    T* Vl = Kl + Ly::K_ELEMS;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS_PER_THREAD; ++i) {
      const int ci = tid + Ly::THREADS * i;
      const int row = ci / Ly::CHUNKS_PER_ROW;
      const int c8 = ci % Ly::CHUNKS_PER_ROW;
      *(vec8<T>*)(Kl + row * Ly::KS + c8 * 8) = kreg[i];
      *(vec8<T>*)(Vl + row * Ly::VS + c8 * 8) = vreg[i];
    }
  };

  // Lane-constant parts of the transposed V read: within each 16-lane group
  // lane (e, t) fetches 4 d-values of key row e; the hardware transpose hands
  // lane i the d-column i of those 4 keys.
  const int tr_e = (lane & 15) >> 2;
  const int tr_t = lane & 3;
  const int tr_cg = (lane >> 4) & 1;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) gload(j + 1);
    const int kt0 = j * Ly::KEYS + grp * kBK;  // this group's tile
    const bool skip = (CAUSAL && kt0 > qw + kRowsPerWave - 1) || (G > 1 && kt0 >= N);
    if (!skip) {
      const T* Kl = smem + buf * Ly::STAGE + grp * kBK * Ly::KS;
      const T* Vl = smem + buf * Ly::STAGE + Ly::K_ELEMS + grp * kBK * Ly::VS;

      // S^T[key][query] for two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const T* krow = Kl + (kb * 32 + col) * Ly::KS + half * 8;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const vec8<T> kf = *(const vec8<T>*)(krow + t * 16);
          s[kb] = mfma32(kf, qf[t], s[kb]);
        }
      }

      // Online softmax; masking only on tiles crossing this wave's diagonal
      // or the ragged end.
      float sv[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] = s[0][r];
        sv[16 + r] = s[1][r];
      }
      const bool need_mask = (CAUSAL && kt0 + kBK - 1 > qw) || (kt0 + kBK > N);
      const int lim_causal = qi - kt0 - half * 4;
      const int lim_n = N - kt0 - half * 4;
      vec8<T> pfrag[4];
      const float alpha = need_mask
                              ? tile_softmax<true, CAUSAL>(sv, c, lim_causal, lim_n, m_run, l_part, pfrag)
                              : tile_softmax<false, CAUSAL>(sv, c, lim_causal, lim_n, m_run, l_part, pfrag);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
      }

      // O^T += V^T P^T, four 16-key steps.
#pragma unroll
      for (int u = 0; u < kBK / 16; ++u) {
        const vec8<T> pf = pfrag[u];
        const T* vrow = Vl + (u * 16 + half * 4 + tr_e) * Ly::VS + tr_cg * 16 + 4 * tr_t;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const int bd = (dh * DB + b) * 32;  // output d block
          const vec8<T> vf = read_vt(vrow + bd, vrow + bd + 8 * Ly::VS);
          oacc[b] = mfma32(vf, pf, oacc[b]);
        }
      }
    }
    if (j + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (G == 2) {
    // Merge the two groups (the stages are free after the loop's last
    // barrier): [16 DB + 2][4 waves][64 lanes] fp32, lane-consecutive so
    // that every write and read is conflict-free.  Both groups hold the same
    // rows in the same lanes; a row's max is the same in its two lanes.
    constexpr int NV = 16 * DB + 2;
    static_assert(NV * kThreads * 4 <= (int)sizeof(smem), "merge buffer fits the stages");
    float* xb = (float*)smem + wave * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) xb[(b * 16 + r) * kThreads] = oacc[b][r];
      xb[16 * DB * kThreads] = m_run;
      xb[(16 * DB + 1) * kThreads] = l_part;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xb[16 * DB * kThreads];
    const float l1 = xb[(16 * DB + 1) * kThreads];
    const float mm = fmaxf(m_run, m1);
    const float mu = mm == -INFINITY ? 0.f : mm;  // a row no group saw: both factors 0
    const float a0 = __builtin_amdgcn_exp2f(m_run - mu);
    const float a1 = __builtin_amdgcn_exp2f(m1 - mu);
    l_part = a0 * l_part + a1 * l1;
    m_run = mm;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] = a0 * oacc[b][r] + a1 * xb[(b * 16 + r) * kThreads];
  }

  // ---- epilogue: one reciprocal per row, bf16 store, L = ln2 (m + log2 l)
  const float l_tot = swap_halves(l_part, false);
  if (qi < N) {
    const float inv = 1.f / l_tot;
    T* orow = Og + head + (size_t)qi * D + half * 4 + dh * DB * 32;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        vec4<T> out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (T)(oacc[b][g * 4 + e] * inv);
        *(vec4<T>*)(orow + b * 32 + g * 8) = out;
      }
    if (half == 0 && dh == 0) Lg[hr.l + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// FP8 forward (d = 64 or 128): q, k, v are OCP e4m3 bytes, each tensor with
// one dequantisation factor (its values are byte value x factor).  The
// attention computed is that of the dequantised tensors:
//   * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 -- the products of two e4m3
//     values are exact in fp32 -- with the Q and K factors folded into c;
//   * V is widened to bf16 (exact: every e4m3 value is a bf16 value) while
//     it is staged into LDS, so the softmax, P.V (P in bf16, as in the
//     16-bit kernels) and the merge run as in fwd_mfma_kernel;
//   * the V factor joins the final 1/l.
// Same workgroup shape as fwd_mfma_kernel (4 waves x 32 query rows, 64-key
// tiles, G = 2 splitting the key tiles on small grids).  The MFMA takes 64
// contraction values per lane pair: lane (row, half) holds bytes
// 64 t + 32 half .. + 31 of its row of K (A) or Q (B); any assignment of
// contraction indices to (half, byte) gives the same sum as long as A and B
// use the same one.
template <int D, int G>
struct LayoutF8 {
  static constexpr int THREADS = kThreads * G;
  static constexpr int KEYS = kBK * G;           // keys per stage
  static constexpr int KSB = D + 16;             // K tile row stride in bytes (fp8)
  static constexpr int VS = v_row_elems(D);      // V tile row stride in bf16 elements
  static constexpr int K_BYTES = KEYS * KSB;
  static constexpr int STAGE_BYTES = K_BYTES + KEYS * VS * 2;
  static constexpr int CHUNKS_PER_ROW = D / 16;  // 16-byte chunks of fp8
  static constexpr int CHUNKS_PER_THREAD = KEYS * D / 16 / THREADS;
  static_assert(KEYS * D / 16 % THREADS == 0, "tile splits evenly over threads");
  static_assert(STAGE_BYTES % 16 == 0, "stages stay 16-byte aligned");
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // formats of A and B: fp8 e4m3 (cbsz = blgp = 0); no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(kThreads * G, G == 2 ? 1 : 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Qg, const uint8_t* __restrict__ Kg, const uint8_t* __restrict__ Vg,
    __bf16* __restrict__ Og, float* __restrict__ Lg, int BH, int N, int nqb, float c, int negate, float v_descale,
    int group) {
  using T = __bf16;
  using Ly = LayoutF8<D, G>;
  constexpr int DT8 = D / 64;  // 64-wide d steps of the QK^T contraction
  constexpr int DB = D / 32;   // 32-wide d blocks of the output
  __shared__ __attribute__((aligned(16))) char smem[2 * Ly::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = (tid >> 6) & (kWaves - 1);  // query rows of the wave
  const int grp = G == 1 ? 0 : tid >> 8;       // key tiles of the wave
  const int col = lane & 31;
  const int half = lane >> 5;
  c = fmaxf(c, 1e-30f);  // tile_softmax needs c > 0 (scale 0: every P is 1)

  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL ? Order::HeavyLast : Order::Plain, &bh, &qb);
  const int q0 = qb * kBQ;
  const size_t head = (size_t)bh * N * D;                 // Q/O rows (elements = bytes for fp8)
  const size_t kvhead = (size_t)(bh / group) * N * D;
  const uint8_t* Qh = Qg + head;
  const uint8_t* Kh = Kg + kvhead;
  const uint8_t* Vh = Vg + kvhead;

  // ---- Q fragments (B operand): 32 bytes of the lane's query row per d step
  const int qw = q0 + wave * kRowsPerWave;
  const int qi = qw + col;
  i32x8 qf[DT8];
#pragma unroll
  for (int t = 0; t < DT8; ++t) {
    if (qi < N) {
      const u32x4* src = (const u32x4*)(Qh + (size_t)qi * D + 64 * t + 32 * half);
      const u32x4 lo = src[0], hi = src[1];
      qf[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
      qf[t] = i32x8{};
    }
    if (negate) qf[t] ^= (int)0x80808080u;  // scale < 0: -Q (flips the sign bits; exact)
  }

  int nkt = (N + Ly::KEYS - 1) / Ly::KEYS;  // LDS stages
  if (CAUSAL) nkt = min(nkt, (q0 + kBQ - 1) / Ly::KEYS + 1);

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // ---- global -> register prefetch (16 fp8 per chunk), register -> LDS
  u32x4 kreg[Ly::CHUNKS_PER_THREAD], vreg[Ly::CHUNKS_PER_THREAD];
  auto gload = [&](int j) {
    const int kt0 = j * Ly::KEYS;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS_PER_THREAD; ++i) {
      const int ci = tid + Ly::THREADS * i;
      const int row = ci / Ly::CHUNKS_PER_ROW;
      const int c16 = ci % Ly::CHUNKS_PER_ROW;
      const int key = kt0 + row;
      if (key < N) {
        const size_t off = (size_t)key * D + c16 * 16;
        kreg[i] = *(const u32x4*)(Kh + off);
        vreg[i] = *(const u32x4*)(Vh + off);
      } else {
        kreg[i] = u32x4{};
        vreg[i] = u32x4{};
      }
    }
  };
  auto lstore = [&](int buf) {
    char* Kl = smem + buf * Ly::STAGE_BYTES;
    T* Vl = (T*)(Kl + Ly::K_BYTES);
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS_PER_THREAD; ++i) {
      const int ci = tid + Ly::THREADS * i;
      const int row = ci / Ly::CHUNKS_PER_ROW;
      const int c16 = ci % Ly::CHUNKS_PER_ROW;
      *(u32x4*)(Kl + row * Ly::KSB + c16 * 16) = kreg[i];
      // 16 e4m3 -> 16 bf16 (exact): decode pairs to fp32, pack pairs to bf16
      unsigned w[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(vreg[i][x], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(vreg[i][x], true);
        w[2 * x] = __builtin_bit_cast(unsigned, cvt2<T>(lo[0], lo[1]));
        w[2 * x + 1] = __builtin_bit_cast(unsigned, cvt2<T>(hi[0], hi[1]));
      }
      u32x4* dst = (u32x4*)(Vl + row * Ly::VS + c16 * 16);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
  };

  const int tr_e = (lane & 15) >> 2;
  const int tr_t = lane & 3;
  const int tr_cg = (lane >> 4) & 1;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) gload(j + 1);
    const int kt0 = j * Ly::KEYS + grp * kBK;
    const bool skip = (CAUSAL && kt0 > qw + kRowsPerWave - 1) || (G > 1 && kt0 >= N);
    if (!skip) {
      const char* Kl = smem + buf * Ly::STAGE_BYTES + grp * kBK * Ly::KSB;
      const T* Vl = (const T*)(smem + buf * Ly::STAGE_BYTES + Ly::K_BYTES) + grp * kBK * Ly::VS;

      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const char* krow = Kl + (kb * 32 + col) * Ly::KSB + 32 * half;
#pragma unroll
        for (int t = 0; t < DT8; ++t) {
          const u32x4 lo = *(const u32x4*)(krow + 64 * t);
          const u32x4 hi = *(const u32x4*)(krow + 64 * t + 16);
          const i32x8 kf{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          s[kb] = mfma_f8(kf, qf[t], s[kb]);
        }
      }

      float sv[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] = s[0][r];
        sv[16 + r] = s[1][r];
      }
      const bool need_mask = (CAUSAL && kt0 + kBK - 1 > qw) || (kt0 + kBK > N);
      const int lim_causal = qi - kt0 - half * 4;
      const int lim_n = N - kt0 - half * 4;
      vec8<T> pfrag[4];
      const float alpha = need_mask
                              ? tile_softmax<true, CAUSAL>(sv, c, lim_causal, lim_n, m_run, l_part, pfrag)
                              : tile_softmax<false, CAUSAL>(sv, c, lim_causal, lim_n, m_run, l_part, pfrag);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
      }

#pragma unroll
      for (int u = 0; u < kBK / 16; ++u) {
        const vec8<T> pf = pfrag[u];
        const T* vrow = Vl + (u * 16 + half * 4 + tr_e) * Ly::VS + tr_cg * 16 + 4 * tr_t;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const vec8<T> vf = read_vt(vrow + b * 32, vrow + b * 32 + 8 * Ly::VS);
          oacc[b] = mfma32(vf, pf, oacc[b]);
        }
      }
    }
    if (j + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (G == 2) {
    // Merge the two groups, as in fwd_mfma_kernel.
    constexpr int NV = 16 * DB + 2;
    static_assert(NV * kThreads * 4 <= (int)sizeof(smem), "merge buffer fits the stages");
    float* xb = (float*)smem + wave * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) xb[(b * 16 + r) * kThreads] = oacc[b][r];
      xb[16 * DB * kThreads] = m_run;
      xb[(16 * DB + 1) * kThreads] = l_part;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xb[16 * DB * kThreads];
    const float l1 = xb[(16 * DB + 1) * kThreads];
    const float mm = fmaxf(m_run, m1);
    const float mu = mm == -INFINITY ? 0.f : mm;
    const float a0 = __builtin_amdgcn_exp2f(m_run - mu);
    const float a1 = __builtin_amdgcn_exp2f(m1 - mu);
    l_part = a0 * l_part + a1 * l1;
    m_run = mm;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] = a0 * oacc[b][r] + a1 * xb[(b * 16 + r) * kThreads];
  }

  // ---- epilogue: O = V factor x O~ / l -> bf16, L = ln2 (m + log2 l)
  const float l_tot = swap_halves(l_part, false);
  if (qi < N) {
    const float inv = v_descale / l_tot;
    T* orow = Og + head + (size_t)qi * D + half * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        vec4<T> out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (T)(oacc[b][g * 4 + e] * inv);
        *(vec4<T>*)(orow + b * 32 + g * 8) = out;
      }
    if (half == 0) Lg[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// Helpers of the d = 128 kernel.

constexpr float kRaise = 8.f;  // reference-max slack, log2 units (P <= 2^8)

// Calls fn(integral_constant<int, i>) for i = 0 .. N-1, fully unrolled.
template <class Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, I...>) {
  (fn(std::integral_constant<int, I>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  static_for_impl(fn, std::make_integer_sequence<int, N>{});
}

// One V^T fragment (two transposing 8-byte reads) or K fragment (one
// 16-byte read) by inline asm, so completion is tracked only by the
// explicit waits below (hipcc's own wait insertion drops to lgkmcnt(0)
// while LDS-DMA loads are in flight).
template <int OFF_LO, int OFF_HI>
__device__ __forceinline__ void read_v(s16x4& lo, s16x4& hi, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "i"(OFF_LO));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(addr), "i"(OFF_HI));
}
template <int OFF, class T>
__device__ __forceinline__ void read_k(vec8<T>& f, unsigned addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "i"(OFF));
}

// Update of one unmasked tile against the current reference max m, with no
// per-tile max at all.  O = O~/l and L = m + log l hold for any reference m
// ("FlashAttention: Move Less, Not Compute Less", "Tiling Is Easy"); m only
// has to keep 2^(s c - m) in range.  It is set from a real row max on the
// row's first tile and raised only when a tile's probabilities overflow the
// budget checked in fast_finish, so it never exceeds the running row max by
// more than the raise slack and nothing underflows.  The 16 score pairs go
// through three stages spread over the 32 MFMA slots of an interval:
//   slot 2r:     t = s c - m of pair r, and pack + row-sum pair r - 1;
//   slot 2r + 1: p = 2^t of pair r;
// pair 15 is packed by fast_finish.  The row sum here adds the fp32 P, not
// the packed values the P.V product uses (the exact update and the masked
// one add those): a steady tile's weights are then off by at most the
// unit roundoff relative, an error that averages over the many keys of a
// row that reaches the steady loop, for two fp32 adds per pair instead of
// four.  Measured: B8 H32 N8192 d128 causal 1108 -> 1155 TFLOP/s.
struct FastSoftmax {
  float t[2], p[2];
  float ps[4];
  unsigned w[16];
};

template <class T, int K>
__device__ __forceinline__ void fast_slot(FastSoftmax& st, const f32x16 (&s)[2], float c, float m) {
  auto sv = [&](int i) { return s[i >> 4][i & 15]; };
  constexpr int r = K / 2;
  if constexpr (K % 2 == 0) {
    if constexpr (r >= 1) {
      constexpr int q = r - 1;
      const vec2<T> pr = cvt2<T>(st.p[0], st.p[1]);
      const float pp = st.p[0] + st.p[1];
      st.ps[q & 3] = q < 4 ? pp : st.ps[q & 3] + pp;
      st.w[q] = __builtin_bit_cast(unsigned, pr);
      asm volatile("" ::"v"(st.w[q]), "v"(st.ps[q & 3]));
    }
    st.t[0] = fmaf(sv(2 * r), c, -m);
    st.t[1] = fmaf(sv(2 * r + 1), c, -m);
    asm volatile("" ::"v"(st.t[0]), "v"(st.t[1]));
  } else {
    st.p[0] = __builtin_amdgcn_exp2f(st.t[0]);
    st.p[1] = __builtin_amdgcn_exp2f(st.t[1]);
    asm volatile("" ::"v"(st.p[0]), "v"(st.p[1]));
  }
}

// Packs pair 15 and returns the lane's partial row sum of the tile.
template <class T>
__device__ __forceinline__ float fast_finish(FastSoftmax& st, vec8<T> (&pfrag)[4]) {
  const vec2<T> pr = cvt2<T>(st.p[0], st.p[1]);
  st.ps[3] += st.p[0] + st.p[1];
  st.w[15] = __builtin_bit_cast(unsigned, pr);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    pfrag[u] = __builtin_bit_cast(vec8<T>, (u32x4){st.w[4 * u], st.w[4 * u + 1], st.w[4 * u + 2], st.w[4 * u + 3]});
  return (st.ps[0] + st.ps[1]) + (st.ps[2] + st.ps[3]);
}

// Probability budget of a fast tile: a lane's partial row sum above 2^16
// (or not finite) sends the tile through the exact update instead.  Below
// it every probability is at most 2^16, so O stays far from fp32 overflow.
constexpr float kFastBudget = 65536.f;

// Masked tile update in place on the score accumulator.  A score is
// visible when its key offset (within the lane's keys of the tile) is below
// lim; hidden scores become -inf through a sign-mask bit select (integer
// ALU only, so no per-score lane masks occupy scalar registers).  With c > 0,
// 2^(-inf) = 0 drops them from P; a row with no visible key keeps its state.
template <class T>
__device__ inline float softmax_masked_inplace(f32x16 (&s)[2], float c, int lim, float& m_run, float& l_part,
                                               vec8<T> (&pfrag)[4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const unsigned keep = (unsigned)((score_key_offset(i) - lim) >> 31);
    const unsigned u = __float_as_uint(s[i >> 4][i & 15]);
    s[i >> 4][i & 15] = __uint_as_float((u & keep) | (0xff800000u & ~keep));
    mx = fmaxf(mx, s[i >> 4][i & 15]);
  }
  const float mrow = swap_halves(mx, true);
  const float m_tile = mrow * c;
  const bool raise = m_tile > m_run + kRaise;  // false when m_tile = -inf
  const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.f;
  if (raise) m_run = m_tile;
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    unsigned w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int i = u * 8 + e;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i >> 4][i & 15], c, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[(i + 1) >> 4][(i + 1) & 15], c, -m_use));
      const vec2<T> pr = cvt2<T>(p0, p1);
      ps[e >> 1] += sum2(pr);
      w[e >> 1] = __builtin_bit_cast(unsigned, pr);
    }
    pfrag[u] = __builtin_bit_cast(vec8<T>, (u32x4){w[0], w[1], w[2], w[3]});
  }
  l_part = l_part * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
  return alpha;
}

// ---------------------------------------------------------------------------
// duo (d = 128): 8 waves per workgroup, two per SIMD, 32 query rows per
// wave, 256 per workgroup, one workgroup per CU.
//
// Each wave software-pipelines its own tiles: within one barrier interval it
// runs the 16 P.V MFMAs of one tile and the 16 Q.K MFMAs of the next, and
// the 32 slots of the softmax update of the tile in between ride on those
// MFMAs, one slot of VALU work after each (the matrix unit computes while
// the exponentials issue; the other wave of the SIMD fills the gaps).  The
// HBM -> LDS copies (LDS-DMA, 1 KiB per wave instruction) are spread over
// the same MFMAs two intervals ahead of use, into rings of four K and four
// V tiles (128 KiB); one workgroup barrier per interval.  All eight waves
// follow the same order (P.V of tile j-1 first, then Q.K of tile j+1); the
// two waves of a SIMD interleave through the hardware's own arbitration.
// The steady loop is unrolled by the ring period (4), so every LDS address
// is a per-lane base plus a compile-time immediate.
//
// The reference max m of a row is not the running max.  O = O~/l and
// L = m + log l do not depend on which reference m is used (the
// online-softmax identity of "FlashAttention: Move Less, Not Compute Less",
// "Tiling Is Easy"); m only has to keep P = 2^(s*c - m) in range.  It is set
// from the real row max on the first and on masked tiles (raised only when
// a tile's max exceeds it by more than kRaise), and steady tiles use it as
// it stands, with no per-tile max: their probabilities are checked after the
// fact (fast_check) and the rare tile whose row sum exceeds the budget is
// redone against its real max (fast_redo).  The choice of m changes rounding
// only.
namespace duo {

// LDS-DMA through a buffer descriptor: the tile's base address sits in
// scalar registers and each lane adds only its constant byte offset (no
// 64-bit address arithmetic per copy on the VALU); rows past the end of
// the sequence fall outside the descriptor's range and read as zeros.
// Word 3 selects the plain 32-bit data format of gfx9-family descriptors.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned lds_u32;
constexpr int kBufferWord3 = 0x00020000;
// A lane source offset beyond every descriptor's range: the copy writes
// zeros to LDS and reads nothing.
constexpr unsigned kPadOffset = 0x40000000u;
__device__ void raw_buffer_load_lds(i32x4 rsrc, lds_u32* lds, int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

template <class T>
__device__ constexpr int kb_slot(T) {
  return T::value;
}

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 256;  // query rows per workgroup with one wave group (G = 1)
// G = 2 (small grids, d = 64): the two groups of 4 waves share 128 query
// rows and take alternate key tiles, merging (m, l, O) at the end.
template <int G>
constexpr int block_q() {
  return kBQ / G;
}
constexpr int kLead = 3;
constexpr int kRingK = 4;  // K ring: tile being read, one landing, one being written, one spare
constexpr int kRingV = 4;  // V ring: as K (equal rings make the buffers of an interval depend on j mod 4 only)

// K and V tiles sit unpadded in LDS (rows of D bf16) because the LDS-DMA
// writes 1 KiB per wave instruction contiguously.  Bank conflicts of the
// MFMA operand reads are removed by XOR-swizzling the 16-byte chunks of
// each row.  d = 128 (256-byte rows, one row per bank line):
//   K: chunk c of row r is stored at c ^ (r mod 16) -- the 16 lanes reading
//      one logical chunk of 16 consecutive rows hit 16 distinct chunks;
//   V: chunk c of row r is stored at c ^ 4(r mod 4) -- the LDS serves a
//      transposing 8-byte read 32 lanes (256 bytes over its 64 banks) at a
//      time, and those lanes touch 4 consecutive rows x 4 chunks, which land
//      on 16 distinct chunks (a factor of 2 instead of 4 spreads them over
//      only half the banks: a two-way conflict on every V read).
// d = 64 (128-byte rows, two rows per bank line, so the bank quad of chunk
// p of row r is 8 (r mod 2) + p):
//   K: chunk c of row r is stored at c ^ ((r >> 1) mod 8) -- among 16
//      consecutive rows the 8 of one parity get 8 distinct masks;
//   V: chunk c of row r is stored at c ^ 4 ((r >> 1) mod 2) -- of 4
//      consecutive rows x an aligned group of 4 chunks, rows r0 + 2 and
//      r0 + 3 move the group to the other half of the row and the parities
//      split each pair: 16 distinct quads.  The mask repeats every 4 rows,
//      so the 8- and 16-row steps of the reads stay immediate offsets.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128)
    return r & 15;
  else
    return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128)
    return 4 * (r & 3);
  else
    return 4 * ((r >> 1) & 1);
}

// A ring slot holds one key tile per wave group (G tiles of kBK rows, the
// keys of one interval, contiguous in HBM and copied as one G kBK-row tile).
// F8 (e4m3 inputs, d = 64 or 128): the K slots hold the tile's bytes in
// 128-byte rows (the bf16 d = 64 geometry and swizzle; at d = 64 the last
// four chunks of a row are never read and their copies fetch nothing); V
// is copied as bytes into a staging ring of 128-byte rows (unswizzled) and
// widened to bf16 into the V ring (the bf16 geometry of d) by the
// workgroup in the interval before its P.V.  Sizes in elements of the
// 16-bit type.
template <int D, int G, bool F8 = false>
struct Layout {
  static constexpr int CPR = F8 ? 8 : D / 8;  // 16-byte chunks of a copied row
  static constexpr int TILE = kBK * D;  // one group's tile
  static constexpr int SLOT = G * TILE;
  static constexpr int KSLOT = F8 ? kBK * 64 : SLOT;
  static constexpr int STSLOT = F8 ? kBK * 64 : 0;
  static constexpr int K0 = 0;
  static constexpr int V0 = kRingK * KSLOT;
  static constexpr int ST0 = V0 + kRingV * SLOT;
  static constexpr int TOTAL = ST0 + kRingV * STSLOT;
  static constexpr int ROWS_PER_INSTR = 64 / CPR;
  static constexpr int INSTR_PER_TILE = G * kBK / ROWS_PER_INSTR;  // per slot
  static constexpr int INSTR_PER_WAVE = INSTR_PER_TILE / kWaves;
  static_assert(INSTR_PER_TILE % kWaves == 0, "DMA instructions split evenly over waves");
  static_assert(D == 64 || D == 128, "row swizzles exist for 128- and 256-byte rows");
  static_assert(!F8 || ((D == 64 || D == 128) && G == 1), "e4m3 inputs: d = 64 or 128, one wave group");
  static_assert(TOTAL * 2 <= 160 * 1024, "fits the 160 KiB LDS");
};

// PERSIST: a grid of W workgroups per XCD (one per CU) walks the XCD's
// items -- its heads one after the other, each head's query blocks heaviest
// first -- dealt to the W workgroups in snake order (W items forward, the
// next W backward), so the XCD's CUs stream the K and V of one or two heads
// at a time (shared in its L2) and every workgroup's total pairs heavy
// blocks with light ones.  The copies
// that, on an item's last intervals, would re-read its last tile fetch the
// next item's first K and V tiles instead (each item is a whole number of
// ring periods), and the next Q block is loaded while the item's last P.V
// and its stores run: no workgroup launch and no cold prologue per item.
// Only for fixed length with N a multiple of the 256-row block and every
// XCD holding whole heads.
// LDS row length of head dim D: d = 96 keeps the 256-byte rows (and
// swizzles) of d = 128, d = 32 the 128-byte rows of d = 64; the last
// 16-byte chunks of each K and V row (four of them) are never read, and
// their copies are given an out-of-range source, so they fetch nothing.
template <int D>
constexpr int lds_dim() {
  return D == 96 ? 128 : D == 32 ? 64 : D;
}

// F8: q, k, v hold e4m3 bytes (In = uint8_t), T = bf16 is the type of P,
// of the widened V and of O; o_scale (the V factor) multiplies O.
template <class T, int D, bool CAUSAL, int G = 1, bool PERSIST = false, bool F8 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const std::conditional_t<F8, uint8_t, T>* __restrict__ Qg,
                const std::conditional_t<F8, uint8_t, T>* __restrict__ Kg,
                const std::conditional_t<F8, uint8_t, T>* __restrict__ Vg, T* __restrict__ Og,
                float* __restrict__ Lg, int BH, int N, int nqb, float c, int negate, int group,
                const int* __restrict__ cu_seqlens, int H, int total, float o_scale) {
  using In = std::conditional_t<F8, uint8_t, T>;
  constexpr int LD = lds_dim<D>();
  using Ly = Layout<LD, G, F8>;
  // Copied rows: bytes per row in HBM, and the row length (in elements of
  // T) of the K tile in LDS, whose swizzle it takes.
  constexpr int HROWB = F8 ? D : D * 2;
  constexpr int KLD = F8 ? 64 : LD;
  constexpr int BQ = block_q<G>();
  static_assert(!PERSIST || G == 1, "persistent launches run one wave group");
  constexpr int DT = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = Ly::CPR;
  constexpr int NV = (kBK / 16) * DB;
  // Q.K MFMAs per interval: 16-wide d steps, or 64-wide with e4m3 inputs
  constexpr int NK = F8 ? 2 * (D / 64) : 2 * DT;
  constexpr int IPW = Ly::INSTR_PER_WAVE;
  // 32 softmax slots per interval over its NK + NV MFMAs, 16 per product:
  // MFMA F of a product of NM MFMAs carries slots 16F/NM .. 16(F+1)/NM - 1
  // (one per MFMA at d = 128, two at d = 64, one or two at d = 96, four at
  // d = 32; with e4m3 inputs one per P.V and four per Q.K MFMA, each of
  // which takes twice the time of a 16-bit one).
  static_assert(NV <= 16 && NK <= 16, "32 softmax slots per interval");
  static_assert(NK % IPW == 0 && NK / IPW >= 2, "DMA instructions spread over the MFMAs");
  __shared__ __attribute__((aligned(1024))) T smem[Ly::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  // The k-th item (head, query block) of this workgroup.
  auto item = [&](int k, int* bh, int* qb) -> bool {
    if constexpr (!PERSIST) {
      if (k > 0) return false;
      map_block(blockIdx.x, BH * nqb, nqb, CAUSAL ? Order::HeavyLast : Order::Plain, bh, qb);
      return true;
    } else {
      const int per = BH * nqb / kNumXcd;  // items of this XCD
      const int W = (int)gridDim.x / kNumXcd;
      const int xcd = (int)blockIdx.x % kNumXcd, wg = (int)blockIdx.x / kNumXcd;
      const int p = k * W + ((k & 1) ? W - 1 - wg : wg);
      if (p >= per) return false;
      const int hd = p / nqb;          // head of this XCD
      const int rank = p - hd * nqb;   // 0 = heaviest
      *bh = xcd * (per / nqb) + hd;
      *qb = CAUSAL ? nqb - 1 - rank : rank;
      return true;
    }
  };

  // A zero scale becomes 1e-30: every P stays exactly 1 in fp32 while
  // -inf * c stays -inf for hidden keys.
  c = fmaxf(c, 1e-30f);
  // Waves w and w + 4 share a SIMD.  G = 1: they get rows 64(w%4) + 32(w/4),
  // so the two waves of a SIMD meet the causal diagonal at the same tile
  // (their numbers of visible tiles differ by at most one).  G = 2: they
  // get the same rows 32(w%4), wave w the even key tiles (group 0), wave
  // w + 4 the odd ones (group 1).
  const int grp = G == 2 ? (wave >> 2) : 0;
  const int q_rel = G == 2 ? (wave & 3) * 32 : (wave & 3) * 64 + (wave >> 2) * 32;
  vec8<T> qf[F8 ? 1 : DT];
  // e4m3: lane (query, half) holds bytes 64 t + 32 half .. + 31 of its row
  // (and K fragments the same bytes of a key row).
  i32x8 qf8[F8 ? D / 64 : 1];
  auto load_q = [&](const In* Qh, int qi, int n) {
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < D / 64; ++t) {
        if (qi < n) {
          const u32x4* src = (const u32x4*)(Qh + (size_t)qi * D + 64 * t + 32 * half);
          const u32x4 lo = src[0], hi = src[1];
          qf8[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                         (int)hi[3]};
        } else {
          qf8[t] = i32x8{};
        }
      }
    } else if (qi < n) {
      const vec8<T>* src = (const vec8<T>*)(Qh + (size_t)qi * D + half * 8);
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[t] = src[2 * t];
    } else {
#pragma unroll
      for (int t = 0; t < DT; ++t) qf[t] = vec8<T>{};
    }
  };

  int bh, qb;
  bool have = item(0, &bh, &qb);
  for (int k_item = 0; have; ++k_item) {
  int nbh = 0, nqbi = 0;
  const bool more = PERSIST && item(k_item + 1, &nbh, &nqbi);
  const int q0 = qb * BQ;
  HeadRows hr = head_rows(bh, BH, group, N, D, cu_seqlens, H, total);
  if (cu_seqlens) {
    N = hr.n;
    if (q0 >= N) return;  // past the end of this sequence (the whole workgroup)
  }
  const size_t head = hr.q;
  const In* Qh = Qg + head;
  const In* Kh = Kg + hr.kv;
  const In* Vh = Vg + hr.kv;
  // the next item's K and V heads (persistent launches)
  const HeadRows hn = head_rows(nbh, BH, group, N, D, cu_seqlens, H, total);
  const In* Kn = Kg + hn.kv;
  const In* Vn = Vg + hn.kv;
  const int qw = q0 + q_rel;
  const int qi = qw + col;
  if (k_item == 0) load_q(Qh, qi, N);  // later items' Q blocks come with the previous item
  if (negate) {  // scale < 0: use -Q and |scale| (negation is exact)
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < D / 64; ++t) qf8[t] ^= (int)0x80808080u;
    } else {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        u32x4 u = __builtin_bit_cast(u32x4, qf[t]) ^ 0x80008000u;
        qf[t] = __builtin_bit_cast(vec8<T>, u);
      }
    }
  }

  // Key tiles of kBK rows (global index t); the workgroup runs nkt
  // intervals, interval j holding tiles G j .. G j + G - 1, and a wave
  // handles tile G j + grp of interval j: below, wave_nt and nfull count
  // the wave's own tiles (its local index j).
  int nkt_all = (N + kBK - 1) / kBK;
  if (CAUSAL) nkt_all = min(nkt_all, (q0 + BQ - 1) / kBK + 1);
  const int nkt = (nkt_all + G - 1) / G;
  // the number of the wave's tiles among tiles 0 .. x - 1
  auto local = [&](int x) { return G == 1 ? x : max(0, (x - grp + 1) / 2); };
  int wave_nt = nkt_all;
  if (CAUSAL) wave_nt = min(nkt_all, (qw + 31) / kBK + 1);
  if (qw >= N) wave_nt = 0;
  // Tiles every row of this wave sees in full (the wave's own count: under
  // the causal mask a wave's rows meet the diagonal at tile qw / kBK, so
  // the waves of a workgroup leave the steady schedule at different tiles).
  int nfull = N / kBK;
  if (CAUSAL) nfull = min(nfull, qw / kBK);
  if (wave_nt == 0) nfull = 0;
  wave_nt = local(wave_nt);
  nfull = min(local(nfull), wave_nt - 1);

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  f32x16 sacc[2];
  sacc[0] = sacc[1] = f32x16{};
  vec8<T> pfrag[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pfrag[u] = vec8<T>{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  const int dma_row = lane / CPR;
  const int dma_chunk = lane % CPR;
  // Source byte offsets of the lane within a copied tile (the descriptor's
  // range cuts rows past the end of the sequence).
  unsigned dk_lane[IPW], dv_lane[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (wave * IPW + i) * Ly::ROWS_PER_INSTR + dma_row;
    const int ck = dma_chunk ^ swz_k<KLD>(row), cv = F8 ? dma_chunk : dma_chunk ^ swz_v<LD>(row);
    dk_lane[i] = ck < HROWB / 16 ? (unsigned)(row * HROWB + ck * 16) : kPadOffset;
    dv_lane[i] = cv < HROWB / 16 ? (unsigned)(row * HROWB + cv * 16) : kPadOffset;
  }
  auto dma_one = [&](const In* Xh, int buf, int t, int i, auto is_v) {
    if (PERSIST && more && t >= nkt) {  // the next item's tile t - nkt (same ring slot: nkt is a multiple of 4)
      Xh = decltype(is_v)::value ? Vn : Kn;
      t -= nkt;
    } else {
      t = min(t, nkt - 1);  // tiles past the last one re-read it (never used)
    }
    const int kt0 = t * G * kBK;
    const int rows = min(N - kt0, G * kBK);
    const uint64_t base = (uint64_t)(uintptr_t)(Xh + (size_t)kt0 * D);
    const i32x4 rs = {(int)(uint32_t)base, (int)(uint32_t)(base >> 32), rows * HROWB, kBufferWord3};
    const int r0 = (wave * IPW + i) * Ly::ROWS_PER_INSTR;
    raw_buffer_load_lds(rs, (lds_u32*)(smem + buf + r0 * KLD), 16, (int)(decltype(is_v)::value ? dv_lane[i] : dk_lane[i]),
                        0, 0, 0);
  };
  // DMA of tile t into a ring slot given as an element offset (general
  // path) or as integral_constant<int, slot> of the K (is_v false) or V
  // ring.
  auto dma_any = [&](const In* Xh, auto buf, int t, int i, auto is_v) {
    if constexpr (std::is_integral_v<decltype(buf)>) {
      dma_one(Xh, buf, t, i, is_v);
    } else {
      constexpr int eoff = decltype(is_v)::value ? (F8 ? Ly::ST0 + kb_slot(buf) * Ly::STSLOT
                                                       : Ly::V0 + kb_slot(buf) * Ly::SLOT)
                                                 : Ly::K0 + kb_slot(buf) * Ly::KSLOT;
      dma_one(Xh, eoff, t, i, is_v);
    }
  };
  auto kbuf = [](int t) { return Ly::K0 + (t % kRingK) * Ly::KSLOT; };
  auto vbuf = [](int t) { return Ly::V0 + (t % kRingV) * Ly::SLOT; };
  // copy target of V tile t: the V ring, or the staging ring (F8)
  auto vdst = [](int t) { return F8 ? Ly::ST0 + (t % kRingV) * Ly::STSLOT : Ly::V0 + (t % kRingV) * Ly::SLOT; };
  // V tiles are copied kVLead intervals ahead (one more with the widening
  // step in between).
  constexpr int kVLead = F8 ? 2 : 1;
  auto iteration_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(2 * IPW) : "memory");
  };

  // K fragment reads of row col: 16-bit, chunk 2t + half (16-wide d step
  // t) at k_off[t]; e4m3, chunks 4t + 2 half and 4t + 2 half + 1 of the
  // 128-byte row (64-wide d step t) at k_off[2t] and k_off[2t + 1].
  constexpr int NKA = F8 ? 2 * (D / 64) : DT;
  unsigned k_off[NKA];
#pragma unroll
  for (int t = 0; t < NKA; ++t) {
    if constexpr (F8)
      k_off[t] = (unsigned)(col * KLD * 2 + (((4 * (t >> 1) + 2 * half + (t & 1)) ^ swz_k<KLD>(col)) * 16));
    else
      k_off[t] = (unsigned)(col * LD + (((2 * t + half) ^ swz_k<LD>(col)) * 8)) * 2u;
  }
  const int tr_e = (lane & 15) >> 2;
  const int tr_t = lane & 3;
  const int tr_cg = (lane >> 4) & 1;
  unsigned v_off[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
    v_off[b] = (unsigned)((half * 4 + tr_e) * LD + (((4 * b + 2 * tr_cg + (tr_t >> 1)) ^ swz_v<LD>(half * 4 + tr_e)) * 8) +
                          (tr_t & 1) * 4) * 2u;
  // (plus the byte offset of the wave's tile within a slot)
  const unsigned smem_base = lds_addr(smem) + (unsigned)(grp * Ly::TILE * 2);
  // Absolute LDS addresses of buffer 0 of each ring; the buffer, the
  // 32-key half and the 16-key step then enter as instruction immediates.
  unsigned k_abs[NKA], v_abs[DB];
#pragma unroll
  for (int t = 0; t < NKA; ++t) k_abs[t] = smem_base + Ly::K0 * 2 + k_off[t];
#pragma unroll
  for (int b = 0; b < DB; ++b) v_abs[b] = smem_base + Ly::V0 * 2 + v_off[b];
  auto buf_rel = [&](int elem_off) {
    unsigned a = (unsigned)(elem_off * 2);
    asm volatile("" : "+s"(a));
    return a;
  };

  FastSoftmax fs;
  f32x16 sb[2];  // scores of the tile being normalised (Q.K overwrites sacc)

  // S^T = K Q^T from K buffer kb.  With SM, slots S0..S0+15 of the fast
  // update of the scores sc ride along; with DMA, the V DMA of tile dma_t
  // into buffer dma_b.
  auto qk = [&](auto kb, auto with_sm, auto with_dma, int dma_t, auto dma_b, auto slot0, const f32x16(&sc)[2],
                f32x16(&dst)[2]) {
    constexpr bool SM = decltype(with_sm)::value;
    constexpr bool DMA = decltype(with_dma)::value;
    constexpr int S0 = decltype(slot0)::value;
    // kb: an element offset, or integral_constant<int, ring slot> (then the
    // slot is an immediate of every read)
    constexpr bool CT = !std::is_integral_v<decltype(kb)>;
    unsigned base = 0;  // byte offset of the slot from slot 0
    if constexpr (!CT) base = buf_rel(kb - Ly::K0);
    if constexpr (F8) {
      // MFMA F: key half F % 2, 64-wide d step F / 2; two 16-byte reads
      vec8<T> fl[kLead], fh[kLead];
      auto issue = [&](auto fc) {
        constexpr int F = decltype(fc)::value;
        constexpr int o = (F % 2) * 32 * KLD * 2;
        if constexpr (CT) {
          constexpr int os = kb_slot(kb) * Ly::KSLOT * 2 + o;
          read_k<os>(fl[F % kLead], k_abs[2 * (F / 2)]);
          read_k<os>(fh[F % kLead], k_abs[2 * (F / 2) + 1]);
        } else {
          read_k<o>(fl[F % kLead], base + k_abs[2 * (F / 2)]);
          read_k<o>(fh[F % kLead], base + k_abs[2 * (F / 2) + 1]);
        }
      };
      static_for<(kLead < NK ? kLead : NK)>(issue);
      static_for<NK>([&](auto fc) {
        constexpr int F = decltype(fc)::value;
        constexpr int last = (F + kLead - 1 < NK - 1) ? F + kLead - 1 : NK - 1;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(fl[F % kLead]), "+v"(fh[F % kLead]) : "i"(2 * (last - F)));
        const u32x4 lo = __builtin_bit_cast(u32x4, fl[F % kLead]), hi = __builtin_bit_cast(u32x4, fh[F % kLead]);
        const i32x8 kf{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        __builtin_amdgcn_s_setprio(2);
        if constexpr (F < 2)
          dst[F % 2] = mfma_f8(kf, qf8[F / 2], f32x16{});
        else
          dst[F % 2] = mfma_f8(kf, qf8[F / 2], dst[F % 2]);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (F + kLead < NK) issue(std::integral_constant<int, F + kLead>{});
        if constexpr (SM)
          static_for<16 * (F + 1) / NK - 16 * F / NK>(
              [&](auto sc_i) { fast_slot<T, S0 + 16 * F / NK + decltype(sc_i)::value>(fs, sc, c, m_run); });
        if constexpr (DMA && F % (NK / IPW) == (NK / IPW) - 1)
          dma_any(Vh, dma_b, dma_t, F / (NK / IPW), std::true_type{});
        __builtin_amdgcn_sched_barrier(0);
      });
      return;
    }
    vec8<T> fr[kLead];
    auto issue = [&](auto fc) {
      constexpr int F = decltype(fc)::value;
      if constexpr (CT)
        read_k<kb_slot(kb) * Ly::KSLOT * 2 + (F % 2) * 32 * LD * 2>(fr[F % kLead], k_abs[F / 2]);
      else
        read_k<(F % 2) * 32 * LD * 2>(fr[F % kLead], base + k_abs[F / 2]);
    };
    static_for<(kLead < NK ? kLead : NK)>(issue);
    static_for<NK>([&](auto fc) {
      constexpr int F = decltype(fc)::value;
      constexpr int last = (F + kLead - 1 < NK - 1) ? F + kLead - 1 : NK - 1;
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(fr[F % kLead]) : "i"(last - F));
      __builtin_amdgcn_s_setprio(2);
      if constexpr (F < 2)
        dst[F % 2] = mfma32(fr[F % kLead], qf[F / 2], f32x16{});
      else
        dst[F % 2] = mfma32(fr[F % kLead], qf[F / 2], dst[F % 2]);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (F + kLead < NK) issue(std::integral_constant<int, F + kLead>{});
      if constexpr (SM)
        static_for<16 * (F + 1) / NK - 16 * F / NK>(
            [&](auto sc_i) { fast_slot<T, S0 + 16 * F / NK + decltype(sc_i)::value>(fs, sc, c, m_run); });
      if constexpr (DMA && F % (NK / IPW) == (NK / IPW) - 1) dma_any(Vh, dma_b, dma_t, F / (NK / IPW), std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Widening of V tile t (F8): each thread takes 16 bytes, row tid / 8,
  // d = 16 (tid % 8) .. + 15, from staging slot t % 4 and writes them as
  // two 16-byte bf16 chunks into V slot t % 4 (exact: every e4m3 value is
  // a bf16 value).  Read and write are split so that the read's latency
  // can ride on MFMAs.
  // (At d = 64 a tile is 4 KiB: threads 0..255, waves 0-3, do it.)
  char* const sm = (char*)smem;
  constexpr int WCPR = D / 16;  // 16-byte chunks of an e4m3 row
  constexpr bool kWideAll = kBK * WCPR == kThreads;
  const bool w_on = kWideAll || tid < kBK * WCPR;
  const int w_row = tid / WCPR, w_c = tid % WCPR;
  const unsigned w_src = Ly::ST0 * 2 + w_row * 128 + w_c * 16;
  const unsigned w_dst0 = Ly::V0 * 2 + w_row * LD * 2 + (((2 * w_c) ^ swz_v<LD>(w_row)) * 16);
  const unsigned w_dst1 = Ly::V0 * 2 + w_row * LD * 2 + (((2 * w_c + 1) ^ swz_v<LD>(w_row)) * 16);
  u32x4 w_in{};
  auto widen_read = [&](int slot) {
    if (w_on) w_in = *(const u32x4*)(sm + w_src + slot * (Ly::STSLOT * 2));
  };
  auto widen_write = [&](int slot) {
    if (!w_on) return;
    unsigned w[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      w[2 * x] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w_in[x], 1.f, false));
      w[2 * x + 1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w_in[x], 1.f, true));
    }
    *(u32x4*)(sm + w_dst0 + slot * (Ly::SLOT * 2)) = u32x4{w[0], w[1], w[2], w[3]};
    *(u32x4*)(sm + w_dst1 + slot * (Ly::SLOT * 2)) = u32x4{w[4], w[5], w[6], w[7]};
  };

  // O^T += V^T P^T from V buffer vb.  With SM, slots S0..S0+15 of the fast
  // update of the scores sc ride along; with DMA, the K DMA of tile dma_t
  // into buffer dma_b; with widen = integral_constant<int, slot> (F8), the
  // widening of the V tile of that ring slot.
  auto pv = [&](auto vb, auto with_sm, auto with_dma, int dma_t, auto dma_b, auto slot0, const f32x16(&sc)[2],
                auto widen) {
    constexpr bool SM = decltype(with_sm)::value;
    constexpr bool DMA = decltype(with_dma)::value;
    constexpr int S0 = decltype(slot0)::value;
    constexpr bool WIDEN = !std::is_same_v<decltype(widen), std::false_type>;
    constexpr bool CT = !std::is_integral_v<decltype(vb)>;
    unsigned base = 0;
    if constexpr (!CT) base = buf_rel(vb - Ly::V0);
    s16x4 lo[kLead], hi[kLead];
    auto issue = [&](auto fc) {
      constexpr int F = decltype(fc)::value;
      constexpr int u = F / DB, b = F % DB;
      if constexpr (CT) {
        constexpr int o = kb_slot(vb) * Ly::SLOT * 2;
        read_v<o + u * 16 * LD * 2, o + (u * 16 + 8) * LD * 2>(lo[F % kLead], hi[F % kLead], v_abs[b]);
      } else {
        read_v<u * 16 * LD * 2, (u * 16 + 8) * LD * 2>(lo[F % kLead], hi[F % kLead], base + v_abs[b]);
      }
    };
    static_for<(kLead < NV ? kLead : NV)>(issue);
    static_for<NV>([&](auto fc) {
      constexpr int F = decltype(fc)::value;
      constexpr int u = F / DB, b = F % DB;
      constexpr int last = (F + kLead - 1 < NV - 1) ? F + kLead - 1 : NV - 1;
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo[F % kLead]), "+v"(hi[F % kLead]) : "i"(2 * (last - F)));
      const vec8<T> vf =
          __builtin_bit_cast(vec8<T>, __builtin_shufflevector(lo[F % kLead], hi[F % kLead], 0, 1, 2, 3, 4, 5, 6, 7));
      __builtin_amdgcn_s_setprio(2);
      oacc[b] = mfma32(vf, pfrag[u], oacc[b]);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (F + kLead < NV) issue(std::integral_constant<int, F + kLead>{});
      if constexpr (SM)
        static_for<16 * (F + 1) / NV - 16 * F / NV>(
            [&](auto sc_i) { fast_slot<T, S0 + 16 * F / NV + decltype(sc_i)::value>(fs, sc, c, m_run); });
      if constexpr (WIDEN && F == 1) widen_read(decltype(widen)::value);
      if constexpr (WIDEN && F == NV / 2) widen_write(decltype(widen)::value);
      if constexpr (DMA && F % (NV / IPW) == (NV / IPW) - 1) dma_any(Kh, dma_b, dma_t, F / (NV / IPW), std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto rescale = [&](float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
    }
  };

  // Interval j (between two workgroup barriers) loads K_{j+3} into the
  // buffer K_{j-1} left and V_{j+1} into the buffer V_{j-2} left, and every
  // wave runs
  //   P_{j-1} V_{j-1}       || slots 0-15 of the fast update of tile j,
  //   S_{j+1} = Q K_{j+1}^T || slots 16-31 of tile j.
  // (K_{j-1} was last read in interval j-2, V_{j-2} in interval j-1.)
  // Slots 0-15 read the scores where Q.K left them; slots 16-31 a copy,
  // since the next Q.K overwrites them.
  using S_lo = std::integral_constant<int, 0>;
  using S_hi = std::integral_constant<int, 16>;
  using On = std::true_type;
  using Off = std::false_type;
  auto masked_softmax = [&](int j) {
    const int kt0 = (G * j + grp) * kBK;
    int lim = N - kt0 - half * 4;
    if (CAUSAL) lim = min(lim, qi - kt0 - half * 4 + 1);
    const float m_before = m_run;
    const float alpha = softmax_masked_inplace(sacc, c, lim, m_run, l_part, pfrag);
    rescale(m_before == -INFINITY ? 1.f : alpha);
  };
  // End of a fast tile whose scores are in sb: P fragments, and the tile's
  // row sum joins l -- unless a lane's partial sum exceeds the budget (or is
  // not finite); then fast_check returns true and the caller runs fast_redo
  // before the tile's P.V.  The redo sits outside the steady loops (they
  // only exit on it), which keeps their register allocation unchanged.
  auto fast_check = [&]() -> bool {
    const float part = fast_finish(fs, pfrag);
    const bool ovf = __builtin_amdgcn_ballot_w64(!(part <= kFastBudget)) != 0;
    if (!ovf) l_part += part;
    return ovf;
  };
  // Exact update of the tile with scores sv: m raised to the row max, P recomputed,
  // O and l rescaled.
  auto fast_redo = [&](const f32x16(&sv)[2]) {
    float mx = sv[0][0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sv[i >> 4][i & 15]);
    const float m_new = fmaxf(m_run, swap_halves(mx, true) * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ps[2] = {0.f, 0.f};
  #pragma unroll
    for (int u = 0; u < 4; ++u) {
      unsigned w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i = u * 8 + e;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[i >> 4][i & 15], c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[(i + 1) >> 4][(i + 1) & 15], c, -m_run));
        const vec2<T> pr = cvt2<T>(p0, p1);
        ps[e >> 2] += sum2(pr);
        w[e >> 1] = __builtin_bit_cast(unsigned, pr);
      }
      pfrag[u] = __builtin_bit_cast(vec8<T>, (u32x4){w[0], w[1], w[2], w[3]});
    }
    l_part = l_part * alpha + (ps[0] + ps[1]);
    rescale(alpha);
  };
  // Steady interval: tile j unmasked for every row of the wave, 1 <= j,
  // j + 1 < nkt.
  // Returns true when tile j's probabilities overflowed the budget (P_j
  // then needs fast_redo before the next interval's P.V).
  // R = j mod 4 fixes every ring slot of the interval, and the scores of
  // tile j sit in sacc for even j, in sb for odd j (Q.K of tile j + 1
  // writes the other set, so no copy is needed).
  auto steady = [&](int j, auto r_c) -> bool {
    constexpr int R = decltype(r_c)::value;
    f32x16(&cur)[2] = (R & 1) ? sb : sacc;
    f32x16(&nxt)[2] = (R & 1) ? sacc : sb;
    using Widen = std::conditional_t<F8, std::integral_constant<int, R>, std::false_type>;
    pv(std::integral_constant<int, (R + 3) % 4>{}, On{}, On{}, j + 3, std::integral_constant<int, (R + 3) % 4>{},
       S_lo{}, cur, Widen{});
    qk(std::integral_constant<int, (R + 1) % 4>{}, On{}, On{}, j + kVLead,
       std::integral_constant<int, (R + kVLead) % 4>{}, S_hi{}, cur, nxt);
    const bool ovf = fast_check();
    iteration_barrier();
    return ovf;
  };

  auto dma_all = [&](int j) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      dma_one(Kh, kbuf(j + 3), j + 3, i, Off{});
      dma_one(Vh, vdst(j + kVLead), j + kVLead, i, On{});
    }
  };
  // Any interval (first, masked or last tiles; per-wave tile counts).
  auto general = [&](int j) {
    dma_all(j);
    if constexpr (F8) {
      widen_read(j % kRingV);
      widen_write(j % kRingV);
    }
    if (j >= 1 && j - 1 < wave_nt) pv(vbuf(j - 1), Off{}, Off{}, 0, 0, S_lo{}, sacc, Off{});
    if (j < wave_nt) masked_softmax(j);
    if (j + 1 < wave_nt) qk(kbuf(j + 1), Off{}, Off{}, 0, 0, S_lo{}, sacc, sacc);
    iteration_barrier();
  };

  if (k_item == 0) {  // later items' first tiles were copied during the previous item
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      dma_one(Kh, kbuf(0), 0, i, Off{});
      dma_one(Kh, kbuf(1), 1, i, Off{});
      dma_one(Kh, kbuf(2), 2, i, Off{});
      dma_one(Vh, vdst(0), 0, i, On{});
      if constexpr (F8) dma_one(Vh, vdst(1), 1, i, On{});
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
  const int jend = min(nfull, nkt - 1);
  if (wave_nt > 0) qk(kbuf(0), Off{}, Off{}, 0, 0, S_lo{}, sacc, sacc);
  general(0);
  // Steady tiles, the loop unrolled by the ring period (ring slots and the
  // score set are compile-time in each copy).  A tile that overflowed the
  // budget is redone after the loop; the remaining tiles then take the
  // general path (correct for any tile, rarely needed).
  int j = 1;
  if (j < jend) {
    sb[0] = sacc[0];  // tile 1 (odd) in sb
    sb[1] = sacc[1];
    bool ovf = false;
    for (;;) {
      if (j >= jend) break;
      ovf = steady(j, std::integral_constant<int, 1>{});
      ++j;
      if (ovf || j >= jend) break;
      ovf = steady(j, std::integral_constant<int, 2>{});
      ++j;
      if (ovf || j >= jend) break;
      ovf = steady(j, std::integral_constant<int, 3>{});
      ++j;
      if (ovf || j >= jend) break;
      ovf = steady(j, std::integral_constant<int, 0>{});
      ++j;
      if (ovf) break;
    }
    if (ovf) {
      if (j & 1)  // tile j - 1 (even) is in sacc
        fast_redo(sacc);
      else
        fast_redo(sb);
    }
    if (j & 1) {  // the general path expects the scores of tile j in sacc
      sacc[0] = sb[0];
      sacc[1] = sb[1];
    }
  }
  for (; j < nkt; ++j) general(j);
  // every Q.K of the item is done: load the next item's Q block
  if (more) load_q(Qg + hn.q, nqbi * BQ + q_rel + col, N);
  if (nkt - 1 < wave_nt) pv(vbuf(nkt - 1), Off{}, Off{}, 0, 0, S_lo{}, sacc, Off{});
  if (!more) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (G == 2) {
    // Merge the two groups' (m, l, O~) of the same rows through LDS (the
    // rings are free once every wave has passed this barrier: its last
    // reads are done and its copies have landed).  Both sides are exact
    // for any reference m: O~ and l are rescaled by 2^(m_g - m_max).
    constexpr int NX = DB * 16 + 2;
    float* xs = (float*)smem + (wave & 3) * NX * 64 + lane;
    __syncthreads();
    if (grp == 1) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) xs[(b * 16 + e) * 64] = oacc[b][e];
      xs[DB * 16 * 64] = m_run;
      xs[(DB * 16 + 1) * 64] = l_part;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[DB * 16 * 64];
    const float m_new = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[b][e] = oacc[b][e] * a0 + xs[(b * 16 + e) * 64] * a1;
    l_part = l_part * a0 + xs[(DB * 16 + 1) * 64] * a1;
    m_run = m_new;
  }

  const float l_tot = swap_halves(l_part, false);
  if (qi < N) {
    const float inv = F8 ? o_scale / l_tot : 1.f / l_tot;
    T* orow = Og + head + (size_t)qi * D + half * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        vec4<T> out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (T)(oacc[b][g * 4 + e] * inv);
        *(vec4<T>*)(orow + b * 32 + g * 8) = out;
      }
    if (half == 0) Lg[hr.l + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
  bh = nbh;
  qb = nqbi;
  have = more;
  }
}

}  // namespace duo

// Kernel per head dim: the two-waves-per-SIMD kernel for d = 128, 96, 64
// and 32 (one softmax slot per MFMA at d = 128, one or two at d = 96, two
// at d = 64, four at d = 32), the 4-wave kernel for d = 256 (two waves per
// SIMD do not fit the registers) and for d = 96 on grids of fewer 256-row
// blocks than CUs.
// Grids of at most this many workgroups of 128 rows run with two wave
// groups over the keys of each row block (G = 2; the duo kernel at d = 64
// and 32, the 4-wave one at d = 96): with few workgroups per CU there is no
// later workgroup to balance the causal row blocks, and the run takes as
// long as the longest block's chain of key tiles.  Measured with the 4-wave
// kernel (causal bf16, same box): +22 % at B1 H16 N2048 d64 (256
// workgroups), +47 % at B1 H16 N4096 d64, +6 % at B2 H16 N4096 d64 (1024),
// -5 % at B4 H16 N2048 d64 (1024), -12 % at B2 H32 N8192 d64 (4096).  The
// duo kernel with two groups, against the 4-wave one with two: B1 H16
// N2048 d64 300 -> 412 TFLOP/s, B2 H16 N4096 d64 593 -> 768; d32 B1 H16
// N2048 190 -> 246, B2 H16 N4096 500 -> 505.
constexpr int kSplitMaxBlocks = 1024;

// Compute units of the current device (cached per device; 0 if unknown).
inline int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

template <class T, int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  constexpr bool kCanDuo = D == 128 || D == 96 || D == 64 || D == 32;
  constexpr bool kCanSplit = D <= 96;
  const bool split = kCanSplit && (int64_t)p.BH * ((p.N + kBQ - 1) / kBQ) <= kSplitMaxBlocks;
  // d = 64 and 32 run the duo kernel on every grid: one wave group per 256
  // rows on large grids, two groups over the key tiles of 128 rows on small
  // ones.
  // d = 96 (whose two groups' rings would not fit the LDS) runs one group
  // of 256 rows unless that leaves CUs without a workgroup; then the 4-wave
  // kernel's two-group form.  Causal bf16, same box: B2 H16 N4096 710 ->
  // 1039 TFLOP/s, B1 H16 N4096 679 -> 707, but B1 H16 N2048 (128 blocks
  // of 256 rows) 356 -> 334.
  const bool duo_k =
      kCanDuo && !(D == 96 && split && (int64_t)p.BH * ((p.N + duo::kBQ - 1) / duo::kBQ) < device_cus());
  const int duo_g = (D == 64 || D == 32) && split ? 2 : 1;
  const int bq = duo_k ? (duo_g == 2 ? duo::block_q<2>() : duo::block_q<1>()) : kBQ;
  const int nqb = (p.N + bq - 1) / bq;
  const float c_signed = p.scale * 1.44269504088896340736f;
  const int negate = p.scale < 0.f ? 1 : 0;
  const float c = negate ? -c_signed : c_signed;
  constexpr int kOS = D == 256 ? 2 : 1;  // d = 256: two waves per query block, each half of O
  dim3 grid(p.BH * nqb), block(duo_k ? duo::kThreads : split ? 2 * kThreads : kOS * kThreads);
  // Persistent duo launch: fixed length, whole 256-row blocks, every XCD
  // holding whole heads; one workgroup per CU.
  const int64_t items = (int64_t)p.BH * nqb;
  const int cus = device_cus();
  const bool persist = duo_k && duo_g == 1 && !p.cu_seqlens && p.N % duo::kBQ == 0 && items % kNumXcd == 0 &&
                       (items / kNumXcd) % nqb == 0 && cus >= kNumXcd;
  if (persist) grid = dim3((unsigned)(kNumXcd * std::min<int64_t>(cus / kNumXcd, items / kNumXcd)));
  const T* q = (const T*)p.q;
  const T* k = (const T*)p.k;
  const T* v = (const T*)p.v;
  T* o = (T*)p.o;
  float* lse = p.lse;
  int bh = p.BH, n = p.N;
  int group = p.group;
  const int* cu = p.cu_seqlens;
  int H = p.H, total = p.total;
  float o_scale = 1.f;
  void* args[] = {&q,     &k,          &v,     &o,     &lse, &bh, &n, (void*)&nqb, (void*)&c, (void*)&negate,
                  &group, &cu,         &H,     &total, &o_scale};
  const void* fn;
  if constexpr (D == 96) {
    if (duo_k)
      fn = persist ? (const void*)duo::fwd_kernel<T, D, CAUSAL, 1, true> : (const void*)duo::fwd_kernel<T, D, CAUSAL>;
    else
      fn = (const void*)fwd_mfma_kernel<T, D, CAUSAL, 2>;
  } else if constexpr (kCanDuo) {
    fn = persist ? (const void*)duo::fwd_kernel<T, D, CAUSAL, 1, true> : (const void*)duo::fwd_kernel<T, D, CAUSAL>;
    if constexpr (D == 64 || D == 32) {
      if (duo_g == 2) fn = (const void*)duo::fwd_kernel<T, D, CAUSAL, 2>;
    }
  } else {  // d = 256
    fn = (const void*)fwd_mfma_kernel<T, D, CAUSAL, 1, kOS>;
  }
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <class T>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 32: return p.causal ? launch<T, 32, true>(p, stream) : launch<T, 32, false>(p, stream);
    case 64: return p.causal ? launch<T, 64, true>(p, stream) : launch<T, 64, false>(p, stream);
    case 96: return p.causal ? launch<T, 96, true>(p, stream) : launch<T, 96, false>(p, stream);
    case 128: return p.causal ? launch<T, 128, true>(p, stream) : launch<T, 128, false>(p, stream);
    case 256: return p.causal ? launch<T, 256, true>(p, stream) : launch<T, 256, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool CAUSAL>
hipError_t launch_f8(const FwdParams& p, hipStream_t stream) {
  const int nqb = (p.N + kBQ - 1) / kBQ;
  const bool split = (int64_t)p.BH * nqb <= kSplitMaxBlocks;
  // the Q and K factors join the softmax scale; a negative product runs
  // as -Q with |c|
  const float c_signed = p.scale * p.q_descale * p.k_descale * 1.44269504088896340736f;
  const int negate = c_signed < 0.f ? 1 : 0;
  const float c = negate ? -c_signed : c_signed;
  if constexpr (D == 128 || D == 64) {
    // The two-waves-per-SIMD kernel (e4m3 Q.K, V widened in LDS) unless
    // its 256-row blocks would leave CUs idle; persistent as in launch().
    const int nqb2 = (p.N + duo::kBQ - 1) / duo::kBQ;
    const int64_t items = (int64_t)p.BH * nqb2;
    const int cus = device_cus();
    if (!(split && items < cus)) {
      const bool persist = p.N % duo::kBQ == 0 && items % kNumXcd == 0 && (items / kNumXcd) % nqb2 == 0 &&
                           cus >= kNumXcd;
      dim3 grid(p.BH * nqb2), block(duo::kThreads);
      if (persist) grid = dim3((unsigned)(kNumXcd * std::min<int64_t>(cus / kNumXcd, items / kNumXcd)));
      const uint8_t* q = (const uint8_t*)p.q;
      const uint8_t* k = (const uint8_t*)p.k;
      const uint8_t* v = (const uint8_t*)p.v;
      __bf16* o = (__bf16*)p.o;
      float* lse = p.lse;
      int bh = p.BH, n = p.N, group = p.group, H = p.H, total = p.total;
      const int* cu = nullptr;
      float o_scale = p.v_descale;
      void* args[] = {&q,     &k,  &v, &o,     &lse,     &bh, &n, (void*)&nqb2, (void*)&c, (void*)&negate,
                      &group, &cu, &H, &total, &o_scale};
      const void* fn = persist ? (const void*)duo::fwd_kernel<__bf16, D, CAUSAL, 1, true, true>
                               : (const void*)duo::fwd_kernel<__bf16, D, CAUSAL, 1, false, true>;
      return hipLaunchKernel(fn, grid, block, args, 0, stream);
    }
  }
  dim3 grid(p.BH * nqb), block(split ? 2 * kThreads : kThreads);
  const uint8_t* q = (const uint8_t*)p.q;
  const uint8_t* k = (const uint8_t*)p.k;
  const uint8_t* v = (const uint8_t*)p.v;
  __bf16* o = (__bf16*)p.o;
  float* lse = p.lse;
  int bh = p.BH, n = p.N, group = p.group;
  float vd = p.v_descale;
  void* args[] = {&q, &k, &v, &o, &lse, &bh, &n, (void*)&nqb, (void*)&c, (void*)&negate, &vd, &group};
  const void* fn = split ? (const void*)fwd_fp8_kernel<D, CAUSAL, 2> : (const void*)fwd_fp8_kernel<D, CAUSAL, 1>;
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return p.causal ? launch_f8<64, true>(p, stream) : launch_f8<64, false>(p, stream);
    case 128: return p.causal ? launch_f8<128, true>(p, stream) : launch_f8<128, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

// Waves per workgroup as launched on large grids (d <= 96 runs 8 waves, in
// two key groups, only on grids of at most kSplitMaxBlocks workgroups).
TileConfig mfma_tile(int d) {
  if (d == 128 || d == 96 || d == 64 || d == 32) return TileConfig{duo::kBQ, kBK, duo::kWaves};
  if (d == 256) return TileConfig{kBQ, kBK, 2 * kWaves};  // two waves per 32 query rows
  return TileConfig{kBQ, kBK, kWaves};
}

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) { return launch_t<__bf16>(p, stream); }
hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t stream) { return launch_t<_Float16>(p, stream); }

}  // namespace fa
