// FlashAttention-2 forward, bfloat16 in/out, fp32 softmax state, gfx950 MFMA.
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
// MI355X mapping:
//   * scores are computed transposed (keys x queries) with
//     v_mfma_f32_32x32x16_bf16, so each lane holds 32 scores of ONE query:
//     row max and row sum are in-lane plus one permlane32 swap;
//   * the fp32 score accumulator, exponentiated and packed to bf16, is
//     directly the B operand of the P.V MFMA (the key order inside a 16-key
//     step is permuted consistently on both operands);
//   * V^T operands come from the row-major V tile through ds_read_b64_tr_b16
//     (the gfx950 transposing LDS read), so V is stored in LDS as it sits in
//     HBM;
//   * K/V tiles are double-buffered in LDS, next tile's global loads are in
//     flight while the current tile computes; LDS rows are padded so the
//     MFMA operand reads are bank-conflict free;
//   * exp is the hardware exp2 with scale*log2(e) folded into one FMA.
#include <math.h>

#include "fa_internal.h"
#include "fa_schedule.h"
#include <stdint.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBQ = 128;  // query rows per workgroup
constexpr int kBK = 64;   // keys per streamed tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kBQ / kWaves;  // 32 = one MFMA column block
static_assert(kRowsPerWave == 32, "one 32-wide MFMA block of queries per wave");

template <int D>
struct Layout {
  static constexpr int KS = D + 8;   // K tile row stride in elements (+16 B)
  static constexpr int VS = D + 16;  // V tile row stride in elements (+32 B)
  static constexpr int K_ELEMS = kBK * KS;
  static constexpr int V_ELEMS = kBK * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS_PER_ROW = D / 8;                    // 16-byte chunks
  static constexpr int CHUNKS_PER_THREAD = kBK * D / 8 / kThreads;
  static_assert(kBK * D / 8 % kThreads == 0, "tile splits evenly over threads");
};

__device__ inline float swap_halves(float x, bool want_max) {
  // Lane l receives x from lane l ^ 32; returns max or sum of the two.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]);
  const float b = __uint_as_float(r[1]);
  return want_max ? fmaxf(a, b) : a + b;
}

__device__ inline bf16x8 read_vt(const __bf16* p0, const __bf16* p1) {
  // Two transposing 8-byte LDS reads -> the 8 bf16 of one MFMA A operand.
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Raw LDS addressing: 32-bit byte addresses kept in VGPRs, so each operand
// read is one ds_read with a compile-time immediate offset.
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ inline bf16x8 lds_read_b128(unsigned addr) { return *(const lds_bf16x8*)(uintptr_t)addr; }
__device__ inline bf16x8 lds_read_vt(unsigned addr, unsigned addr8) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr8);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Offset, within a 64-key tile, of score i of a lane (i = 16*kb + r for the
// two 32-key MFMA halves kb and accumulator register r), without the
// lane's 4*half: kb*32 + (r/4)*8 + r%4.
__device__ constexpr int score_key_offset(int i) { return (i >> 4) * 32 + ((i >> 2) & 3) * 8 + (i & 3); }

// Online-softmax update of one 64-key tile for the lane's query row
// ("FlashAttention-2: ...", "FA2 change #1"; "FlashAttention: Move Less,
// Not Compute Less", "Tiling Is Easy"): sv holds the lane's 32 raw scores
// q.k (the other 32 of the row sit in lane ^ 32).  m_run is the running
// max in log2 units (scores times c = scale*log2 e), l_part the lane's
// partial row sum.  Writes P = 2^(s*c - m') as bf16 MFMA B-operand
// fragments and returns alpha = 2^(m - m') for rescaling O.
//   MASK: the tile crosses the causal diagonal or the end of the sequence;
//   scores with key offset > lim_causal (causal) or >= lim_n are excluded.
//   Unmasked tiles run no per-score compare or select at all.
template <bool MASK, bool CAUSAL>
__device__ inline float tile_softmax(float (&sv)[32], float c, int lim_causal, int lim_n, float& m_run,
                                     float& l_part, bf16x8 (&pfrag)[4]) {
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
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    unsigned w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float x0 = sv[u * 8 + e], x1 = sv[u * 8 + e + 1];
      float p0 = __builtin_amdgcn_exp2f(fmaf(x0, c, -m_use));
      float p1 = __builtin_amdgcn_exp2f(fmaf(x1, c, -m_use));
      if (MASK) {  // keeps masked P exactly 0 also when scale = 0 (-inf * 0)
        p0 = (x0 == -INFINITY) ? 0.f : p0;
        p1 = (x1 == -INFINITY) ? 0.f : p1;
      }
      const bf16x2 pr = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
      // Row sum of exactly the bf16 probabilities the P.V product uses.
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lsum, false);
      w[e >> 1] = __builtin_bit_cast(unsigned, pr);
    }
    pfrag[u] = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
  }
  l_part = lsum;
  return alpha;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    __bf16* __restrict__ Og, float* __restrict__ Lg, int BH, int N, int nqb, float c, int negate) {
  using Ly = Layout<D>;
  constexpr int DT = D / 16;  // 16-wide d steps of the QK^T contraction
  constexpr int DB = D / 32;  // 32-wide d blocks of the output
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * Ly::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column of the transposed tiles
  const int half = lane >> 5;  // which 4-key group of each 8 (MFMA layout)

  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL, &bh, &qb);
  const int q0 = qb * kBQ;
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = Qg + head;
  const __bf16* Kh = Kg + head;
  const __bf16* Vh = Vg + head;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop
  const int qw = q0 + wave * kRowsPerWave;  // first query row of this wave
  const int qi = qw + col;                  // this lane's query row
  bf16x8 qf[DT];
  if (qi < N) {
    const bf16x8* src = (const bf16x8*)(Qh + (size_t)qi * D + half * 8);
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = src[2 * t];
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = bf16x8{};
  }
  if (negate) {  // scale < 0: use -Q and |scale| (negation is exact)
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 u = __builtin_bit_cast(u32x4, qf[t]) ^ 0x80008000u;
      qf[t] = __builtin_bit_cast(bf16x8, u);
    }
  }

  int nkt = (N + kBK - 1) / kBK;
  if (CAUSAL) nkt = min(nkt, (q0 + kBQ - 1) / kBK + 1);

  // ---- running state: O^T blocks (d x queries), m in log2 units, partial l
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // ---- global -> register prefetch, register -> LDS store
  bf16x8 kreg[Ly::CHUNKS_PER_THREAD], vreg[Ly::CHUNKS_PER_THREAD];
  auto gload = [&](int j) {
    const int kt0 = j * kBK;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS_PER_THREAD; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / Ly::CHUNKS_PER_ROW;
      const int c8 = ci % Ly::CHUNKS_PER_ROW;
      const int key = kt0 + row;
      if (key < N) {
        const size_t off = (size_t)key * D + c8 * 8;
        kreg[i] = *(const bf16x8*)(Kh + off);
        vreg[i] = *(const bf16x8*)(Vh + off);
      } else {
        kreg[i] = bf16x8{};
        vreg[i] = bf16x8{};
      }
    }
  };
  auto lstore = [&](int buf) {
    __bf16* Kl = smem + buf * Ly::STAGE;
    __bf16* Vl = Kl + Ly::K_ELEMS;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS_PER_THREAD; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / Ly::CHUNKS_PER_ROW;
      const int c8 = ci % Ly::CHUNKS_PER_ROW;
      *(bf16x8*)(Kl + row * Ly::KS + c8 * 8) = kreg[i];
      *(bf16x8*)(Vl + row * Ly::VS + c8 * 8) = vreg[i];
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
    const int kt0 = j * kBK;
    const bool skip = CAUSAL && kt0 > qw + kRowsPerWave - 1;
    if (!skip) {
      const __bf16* Kl = smem + buf * Ly::STAGE;
      const __bf16* Vl = Kl + Ly::K_ELEMS;

      // S^T[key][query] for two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const __bf16* krow = Kl + (kb * 32 + col) * Ly::KS + half * 8;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const bf16x8 kf = *(const bf16x8*)(krow + t * 16);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kb], 0, 0, 0);
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
      bf16x8 pfrag[4];
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
        const bf16x8 pf = pfrag[u];
        const __bf16* vrow = Vl + (u * 16 + half * 4 + tr_e) * Ly::VS + tr_cg * 16 + 4 * tr_t;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16x8 vf = read_vt(vrow + b * 32, vrow + b * 32 + 8 * Ly::VS);
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[b], 0, 0, 0);
        }
      }
    }
    if (j + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: one reciprocal per row, bf16 store, L = ln2 (m + log2 l)
  const float l_tot = swap_halves(l_part, false);
  if (qi < N) {
    const float inv = 1.f / l_tot;
    __bf16* orow = Og + head + (size_t)qi * D + half * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (__bf16)(oacc[b][g * 4 + e] * inv);
        *(bf16x4*)(orow + b * 32 + g * 8) = out;
      }
    if (half == 0) Lg[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong variant: 8 waves per workgroup (two per SIMD), 256 query rows.
//
// Each wave alternates an MFMA phase M_j = {O^T += V_{j-1}^T P_{j-1}^T;
// S_j^T = K_j Q^T} and a softmax phase S_j (mask, max, alpha, exp, row sum,
// O rescale, pack P_j to bf16).  The two waves that share a SIMD run one
// phase apart (workgroup barriers separate the phases), so while one issues
// MFMAs the other runs the exp/max/sum VALU work: the matrix unit is kept
// busy while softmax runs ("FlashAttention-3" pipelining principle in
// "FlashAttention: Move Less, Not Compute Less", "FA1 to FA3", rebuilt for
// CDNA4 wave scheduling instead of Hopper warpgroups).  K/V tiles rotate
// through three LDS stages; a tile is fetched into registers two phases
// before it is stored to LDS.
// Compile-time scheduling pattern for a run of N MFMAs whose operand
// fragment f needs 2 LDS reads if f < NV, else 1: the first LEAD fragments
// are read up front, then each MFMA is followed by the reads of the
// fragment LEAD steps later (instruction-group masks: 0x008 MFMA, 0x100 DS
// read).
template <int F, int LEAD, int NV, int N>
struct SchedPrologue {
  static __device__ __forceinline__ void run() {
    if constexpr (F < LEAD && F < N) {
      __builtin_amdgcn_sched_group_barrier(0x100, F < NV ? 2 : 1, 0);
      SchedPrologue<F + 1, LEAD, NV, N>::run();
    }
  }
};
template <int I, int LEAD, int NV, int N>
struct SchedSteady {
  static __device__ __forceinline__ void run() {
    if constexpr (I < N) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (I + LEAD < N) __builtin_amdgcn_sched_group_barrier(0x100, I + LEAD < NV ? 2 : 1, 0);
      SchedSteady<I + 1, LEAD, NV, N>::run();
    }
  }
};
template <int LEAD, int NV, int N>
__device__ __forceinline__ void sched_mfma_run() {
  SchedPrologue<0, LEAD, NV, N>::run();
  SchedSteady<0, LEAD, NV, N>::run();
}

namespace pp {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 256;
constexpr int kBK = 64;
constexpr int kStages = 3;

// K and V tiles sit unpadded in LDS (rows of D bf16) because the
// HBM->LDS DMA writes 1 KiB per wave instruction contiguously.  Bank
// conflicts are removed by XOR-swizzling the 16-byte chunks of each row:
//   K: chunk c of row r is stored at c ^ (r mod CPR)  -- the MFMA A-operand
//      reads (16 consecutive rows, same chunk) hit 16 distinct chunks;
//   V: chunk c of row r is stored at c ^ 2(r mod 4)   -- each 16-lane group
//      of a transposing read touches 4 consecutive rows x 2 chunks, which
//      land on 8 distinct chunks.
template <int D>
struct Layout {
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int TILE = kBK * D;                 // elements per K (or V) tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int ROWS_PER_INSTR = 64 / CPR;      // rows one DMA instruction fills
  static constexpr int INSTR_PER_TILE = kBK / ROWS_PER_INSTR;
  static constexpr int INSTR_PER_WAVE = INSTR_PER_TILE / kWaves;
  static_assert(INSTR_PER_TILE % kWaves == 0, "DMA instructions split evenly over waves");
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
                __bf16* __restrict__ Og, float* __restrict__ Lg, int BH, int N, int nqb, float c, int negate) {
  using Ly = Layout<D>;
  constexpr int DT = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = Ly::CPR;
  __shared__ __attribute__((aligned(1024))) __bf16 smem[kStages * Ly::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  // Waves w and w + 4 share a SIMD; they form the two phase groups.  Rows
  // are interleaved so both groups meet the causal diagonal equally.
  const int group = wave >> 2;
  const int rowbase = ((wave & 3) * 2 + group) * 32;

  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL, &bh, &qb);
  const int q0 = qb * kBQ;
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = Qg + head;
  const __bf16* Kh = Kg + head;
  const __bf16* Vh = Vg + head;

  const int qw = q0 + rowbase;
  const int qi = qw + col;
  bf16x8 qf[DT];
  if (qi < N) {
    const bf16x8* src = (const bf16x8*)(Qh + (size_t)qi * D + half * 8);
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = src[2 * t];
  } else {
#pragma unroll
    for (int t = 0; t < DT; ++t) qf[t] = bf16x8{};
  }
  if (negate) {
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 u = __builtin_bit_cast(u32x4, qf[t]) ^ 0x80008000u;
      qf[t] = __builtin_bit_cast(bf16x8, u);
    }
  }

  int nkt = (N + kBK - 1) / kBK;
  if (CAUSAL) nkt = min(nkt, (q0 + kBQ - 1) / kBK + 1);
  int wave_nt = nkt;  // tiles this wave computes
  if (CAUSAL) wave_nt = min(nkt, (qw + 31) / kBK + 1);
  if (qw >= N) wave_nt = 0;

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
  f32x16 sacc[2];
  sacc[0] = f32x16{};
  sacc[1] = f32x16{};
  bf16x8 pfrag[kBK / 16];
#pragma unroll
  for (int u = 0; u < kBK / 16; ++u) pfrag[u] = bf16x8{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // ---- HBM -> LDS DMA of key/value tile t into stage t % kStages.  Each wave
  // fills INSTR_PER_WAVE 1 KiB row groups of K and of V; lane l lands at
  // chunk l % CPR of row l / CPR and fetches the chunk the swizzle puts there.
  // Rows past N re-read row N - 1 (finite data; those keys are masked).
  const int dma_row = lane / CPR;
  const int dma_chunk = lane % CPR;
  auto issue_tile = [&](int t) {
    __bf16* Kl = smem + (t % kStages) * Ly::STAGE;
    __bf16* Vl = Kl + Ly::TILE;
    const int kt0 = t * kBK;
#pragma unroll
    for (int i = 0; i < Ly::INSTR_PER_WAVE; ++i) {
      const int r0 = (wave * Ly::INSTR_PER_WAVE + i) * Ly::ROWS_PER_INSTR;
      const int row = r0 + dma_row;
      const size_t key = (size_t)min(kt0 + row, N - 1);
      const int ck = dma_chunk ^ (row % CPR);
      const int cv = dma_chunk ^ (2 * (row & 3));
      __builtin_amdgcn_global_load_lds((const void*)(Kh + key * D + ck * 8),
                                       (__attribute__((address_space(3))) void*)(Kl + r0 * D), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Vh + key * D + cv * 8),
                                       (__attribute__((address_space(3))) void*)(Vl + r0 * D), 16, 0, 0);
    }
  };

  // ---- per-lane LDS byte offsets of the MFMA operands within a stage
  // K: row kb*32 + col, logical chunk 2t + half (kb adds 32 rows).
  unsigned k_off[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) k_off[t] = (unsigned)(col * D + (((2 * t + half) ^ (col % CPR)) * 8)) * 2u;
  // V (transposing reads): 16-lane group g = (half, tr_cg); lane (tr_e, tr_t)
  // reads 8 bytes of key row u*16 + half*4 + tr_e (and +8), logical chunk
  // 4b + 2*tr_cg + tr_t/2, 8-byte half tr_t & 1.
  const int tr_e = (lane & 15) >> 2;
  const int tr_t = lane & 3;
  const int tr_cg = (lane >> 4) & 1;
  unsigned v_off[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
    v_off[b] = (unsigned)(Ly::TILE + (half * 4 + tr_e) * D +
                          (((4 * b + 2 * tr_cg + (tr_t >> 1)) ^ (2 * tr_e)) * 8) + (tr_t & 1) * 4) * 2u;
  const unsigned smem_base = lds_addr(smem);

  // The scheduling hints below keep LDS operand reads a few MFMAs ahead of
  // their use instead of hoisting a whole phase's reads (which would need
  // ~128 more VGPRs): kLead fragments are in flight, then each MFMA is
  // followed by the read of the fragment kLead steps later.
  constexpr int kLead = 3;
  auto stage_base = [&](int j) {
    unsigned base = smem_base + (unsigned)((j % kStages) * Ly::STAGE * 2);
    asm volatile("" : "+s"(base));  // one add per operand per phase, not per read
    return base;
  };
  auto pv_body = [&](int j) {  // O^T += V_j^T P_j^T
    const unsigned base = stage_base(j);
    unsigned va[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) va[b] = base + v_off[b];
#pragma unroll
    for (int u = 0; u < kBK / 16; ++u) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 vf = lds_read_vt(va[b] + u * 16 * D * 2, va[b] + (u * 16 + 8) * D * 2);
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfrag[u], oacc[b], 0, 0, 0);
      }
    }
  };
  auto qk_body = [&](int j) {  // S_j^T = K_j Q^T
    const unsigned base = stage_base(j);
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const unsigned ka = base + k_off[t];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = lds_read_b128(ka + kb * 32 * D * 2);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sacc[kb], 0, 0, 0);
      }
    }
  };
  constexpr int kPvMfma = (kBK / 16) * DB;
  constexpr int kQkMfma = 2 * DT;
  // MFMA phase M_j: P_{j-1} V_{j-1} (if active) then Q K_j (if active).
  auto mphase = [&](bool do_pv, bool do_qk, int j) {
    if (do_pv) {
      pv_body(j - 1);
      sched_mfma_run<kLead, kPvMfma, kPvMfma>();
    }
    if (do_qk) {
      qk_body(j);
      sched_mfma_run<kLead, 0, kQkMfma>();
    }
  };
  // Softmax phase: online update for tile j; P_j packed for the next MFMA phase.
  auto softmax = [&](int j) {
    float sv[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = sacc[0][r];
      sv[16 + r] = sacc[1][r];
    }
    const int kt0 = j * kBK;
    const bool need_mask = (CAUSAL && kt0 + kBK - 1 > qw) || (kt0 + kBK > N);
    const int lim_causal = qi - kt0 - half * 4;
    const int lim_n = N - kt0 - half * 4;
    const float alpha = need_mask
                            ? tile_softmax<true, CAUSAL>(sv, c, lim_causal, lim_n, m_run, l_part, pfrag)
                            : tile_softmax<false, CAUSAL>(sv, c, lim_causal, lim_n, m_run, l_part, pfrag);
    // Rescale only when some row's max moved (alpha is exactly 1 otherwise).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
    }
  };

  issue_tile(0);
  if (nkt > 1) issue_tile(1);
  __syncthreads();

  // Global slot s: group 0 runs M_j in slot 2j and S_j in slot 2j + 1;
  // group 1 runs them one slot later.  Every slot ends with one s_barrier
  // for all 8 waves.  Tile t is DMA'd in slot 2t - 2 (into the stage that
  // tile t - 3 used, last read in slot 2t - 3); the barrier ending each odd
  // slot waits for the wave's DMA and LDS traffic (vmcnt/lgkmcnt = 0), so
  // tile t is complete and visible from slot 2t on.  Even-slot barriers
  // only keep the two groups in step.
  auto end_slot = [&](int slot) {
    if (slot & 1) {
      __syncthreads();
    } else {
      __builtin_amdgcn_s_barrier();
    }
  };
  if (group == 1) end_slot(0);
  for (int j = 0; j <= nkt; ++j) {
    const int slot_m = 2 * j + group;
    mphase(j >= 1 && j - 1 < wave_nt, j < wave_nt, j);
    // DMA of tile slot/2 + 1 in even slots 2, 4, ..., issued after this
    // phase's LDS reads so they need not wait for it.
    if ((slot_m & 1) == 0 && slot_m >= 2 && slot_m / 2 + 1 < nkt) issue_tile(slot_m / 2 + 1);
    end_slot(slot_m);
    if (j < nkt) {
      const int slot_s = slot_m + 1;
      if ((slot_s & 1) == 0 && slot_s / 2 + 1 < nkt) issue_tile(slot_s / 2 + 1);
      if (j < wave_nt) softmax(j);
      end_slot(slot_s);
    }
  }
  if (group == 0) end_slot(2 * nkt + 1);

  const float l_tot = swap_halves(l_part, false);
  if (qi < N) {
    const float inv = 1.f / l_tot;
    __bf16* orow = Og + head + (size_t)qi * D + half * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (__bf16)(oacc[b][g * 4 + e] * inv);
        *(bf16x4*)(orow + b * 32 + g * 8) = out;
      }
    if (half == 0) Lg[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

}  // namespace pp

// Kernel choice per head dim: the ping-pong kernel for d = 128 (MFMA phase
// long enough to cover a softmax phase), the 4-wave kernel for d = 64.
bool use_pp(int d) { return d == 128; }

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const bool pingpong = use_pp(D);
  const int bq = pingpong ? pp::kBQ : kBQ;
  const int nqb = (p.N + bq - 1) / bq;
  const float c_signed = p.scale * 1.44269504088896340736f;
  const int negate = p.scale < 0.f ? 1 : 0;
  const float c = negate ? -c_signed : c_signed;
  dim3 grid(p.BH * nqb), block(pingpong ? pp::kThreads : kThreads);
  const __bf16* q = (const __bf16*)p.q;
  const __bf16* k = (const __bf16*)p.k;
  const __bf16* v = (const __bf16*)p.v;
  __bf16* o = (__bf16*)p.o;
  float* lse = p.lse;
  int bh = p.BH, n = p.N;
  void* args[] = {&q, &k, &v, &o, &lse, &bh, &n, (void*)&nqb, (void*)&c, (void*)&negate};
  const void* fn = pingpong ? (const void*)pp::fwd_kernel<D, CAUSAL> : (const void*)fwd_bf16_kernel<D, CAUSAL>;
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace

TileConfig bf16_tile(int d) {
  return use_pp(d) ? TileConfig{pp::kBQ, pp::kBK, pp::kWaves} : TileConfig{kBQ, kBK, kWaves};
}

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
