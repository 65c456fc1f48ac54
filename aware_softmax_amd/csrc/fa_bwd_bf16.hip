// FlashAttention-2 backward, bfloat16 in/out, fp32 accumulation, gfx950 MFMA.
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
// How ("FA2 change #2", last paragraph): the backward is parallel over key
// columns.  Each workgroup owns one block of 128 keys and keeps dK and dV of
// those keys in registers for the whole sweep over query tiles, so dK and dV
// need no atomics; the dQ rows, which every key block touches, are
// accumulated in an fp32 buffer with atomic adds.
//
// Three kernels:
//   bwd_pre   D_i = dO_i . O_i (fp32), L in log2 units, dQ accumulator = 0;
//   bwd_main  one workgroup per (head, 128-key block), 4 wave64s with 32
//             keys each; 64-query tiles of Q and dO (plus L, D) streamed
//             through double-buffered LDS;
//   bwd_post  dQ = scale * accumulator, rounded to bf16.
//
// MI355X mapping of bwd_main (v_mfma_f32_32x32x16_bf16 throughout):
//   * S = Q K^T and dP = dO V^T are computed with queries as MFMA rows and
//     the wave's 32 keys as columns, K and V fragments resident in VGPRs:
//     each lane owns one key and 16 query rows of each 32-query block;
//   * that accumulator layout, packed to bf16, is directly the B operand of
//     dV^T += dO^T P and dK^T += Q^T dS (the query order inside a 16-query
//     step is permuted identically on both operands); the dO^T and Q^T
//     fragments come from the row-major tiles through ds_read_b64_tr_b16;
//   * dS^T (keys x queries) is written to LDS and dQ = dS K is formed per
//     workgroup over all 128 keys (both operands through transposing reads),
//     one tile behind, so a single barrier per tile suffices;
//   * LDS tiles are XOR-swizzled per 16-byte chunk so that both the
//     row-fragment reads (ds_read_b128) and the transposing reads are free
//     of bank conflicts.
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"
#include "fa_schedule.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBQ = 64;    // queries per streamed tile
constexpr float kLog2e = 1.44269504088896340736f;

// Physical 16-byte chunk of logical chunk c in row r of an LDS tile whose
// rows are ROWB bytes.  Conflict-free for
//   * 16 lanes reading one chunk of 16 consecutive rows (ds_read_b128), and
//   * 32 lanes reading 4 chunks of 4 consecutive rows (transposing reads).
template <int ROWB>
__device__ __forceinline__ int swz_mask(int r) {
  static_assert(ROWB == 256 || ROWB == 128, "rows of 64 or 128 bf16");
  if constexpr (ROWB == 256)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ bf16x8 tr_frag(const char* p_lo, const char* p_hi) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p_lo));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// ---------------------------------------------------------------------------
// bwd_pre: one row per LPR lanes (one 16-byte chunk of dO and O each).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ Og, const __bf16* __restrict__ dOg,
                                                      const float* __restrict__ Lg, float* __restrict__ dqacc,
                                                      float* __restrict__ L2g, float* __restrict__ Dg, int N,
                                                      int Npad) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int c = tid % LPR;
  const size_t row = (size_t)blockIdx.x * RPB + tid / LPR;  // in [0, BH * Npad)
  const int bh = (int)(row / Npad);
  const int i = (int)(row % Npad);
  float acc = 0.f;
  if (i < N) {
    const size_t off = ((size_t)bh * N + i) * D + c * 8;
    const bf16x8 a = *(const bf16x8*)(Og + off);
    const bf16x8 b = *(const bf16x8*)(dOg + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, 64);
  f32x4* z = (f32x4*)(dqacc + row * D + c * 8);
  z[0] = f32x4{};
  z[1] = f32x4{};
  if (c == 0) {
    Dg[row] = acc;
    L2g[row] = i < N ? Lg[(size_t)bh * N + i] * kLog2e : 0.f;
  }
}

// bwd_post: dQ = scale * accumulator -> bf16, 8 elements per thread.
template <int D>
__global__ __launch_bounds__(256) void bwd_post_kernel(const float* __restrict__ dqacc, __bf16* __restrict__ dQg,
                                                       int N, int Npad, size_t total8, float scale) {
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= total8) return;
  const size_t e = g * 8;  // element index in [B][H][N][D]
  const size_t row = e / D;
  const int cd = (int)(e % D);
  const size_t bh = row / N;
  const int i = (int)(row % N);
  const f32x4* src = (const f32x4*)(dqacc + (bh * Npad + i) * D + cd);
  const f32x4 a = src[0], b = src[1];
  bf16x8 out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[k] = (__bf16)(a[k] * scale);
    out[4 + k] = (__bf16)(b[k] * scale);
  }
  *(bf16x8*)(dQg + e) = out;
}

// ---------------------------------------------------------------------------
// bwd_main.
template <int D>
struct BwdLayout {
  static constexpr int ROWB = 2 * D;            // bytes per Q / dO / K row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int QTILE = kBQ * ROWB;      // one Q or dO tile
  static constexpr int KTILE = kBKV * ROWB;     // the workgroup's K block
  static constexpr int DSROWB = 2 * kBQ;        // dS^T row: 64 queries
  static constexpr int DSTILE = kBKV * DSROWB;  // dS^T tile
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = OFF_K + KTILE;
  static constexpr int OFF_DO = OFF_Q + 2 * QTILE;
  static constexpr int OFF_DS = OFF_DO + 2 * QTILE;
  static constexpr int OFF_LD = OFF_DS + 2 * DSTILE;  // per buffer: L2[64], D[64]
  static constexpr int LDTILE = 2 * kBQ * 4;
  static constexpr int TOTAL = OFF_LD + 2 * LDTILE;
  static constexpr int CH = QTILE / 16 / kThreads;  // staged chunks per thread per tile
  static_assert(QTILE % (16 * kThreads) == 0 && KTILE % (16 * kThreads) == 0, "tiles split over threads");
  static_assert(TOTAL <= 160 * 1024, "fits the 160 KiB LDS");
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
                     const __bf16* __restrict__ dOg, const float* __restrict__ L2g, const float* __restrict__ Dg,
                     float* __restrict__ dqacc, __bf16* __restrict__ dKg, __bf16* __restrict__ dVg, int BH, int N,
                     int Npad, int nkb, float c, float scale) {
  using Ly = BwdLayout<D>;
  constexpr int DT = D / 16;  // 16-wide d steps (S and dP contractions)
  constexpr int DB = D / 32;  // 32-wide d blocks (dK, dV, dQ outputs)
  constexpr int ROWB = Ly::ROWB;
  constexpr int CPR = Ly::CPR;
  constexpr int DQB = DB / 2;  // dQ blocks per wave: 2 query blocks x DB d blocks over 4 waves
  __shared__ __attribute__((aligned(1024))) char smem[Ly::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  int bh, jb;
  map_block(blockIdx.x, BH * nkb, nkb, false, &bh, &jb);  // key block 0 (the most query tiles) first
  const int kb0 = jb * kBKV;
  const int kw0 = kb0 + 32 * wave;  // first key of this wave
  const int key = kw0 + col;        // this lane's key (MFMA column)
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = Qg + head;
  const __bf16* Kh = Kg + head;
  const __bf16* Vh = Vg + head;
  const __bf16* dOh = dOg + head;
  const float* L2h = L2g + (size_t)bh * Npad;
  const float* Dh = Dg + (size_t)bh * Npad;
  float* dqh = dqacc + (size_t)bh * Npad * D;

  // K and V fragments of the wave's keys: B operands of S = Q K^T and
  // dP = dO V^T (lane: key `col`, d = 16t + 8 half .. + 7).  Rows past the
  // end are clamped (finite values; their scores are masked).
  bf16x8 kf[DT], vf[DT];
  {
    const size_t r = (size_t)min(key, N - 1) * D + half * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      kf[t] = *(const bf16x8*)(Kh + r + 16 * t);
      vf[t] = *(const bf16x8*)(Vh + r + 16 * t);
    }
  }
  // The workgroup's K block into LDS (B operand of dQ = dS K).
#pragma unroll
  for (int i = 0; i < Ly::KTILE / 16 / kThreads; ++i) {
    const int ci = tid + kThreads * i;
    const int row = ci / CPR, ch = ci % CPR;
    const bf16x8 x = *(const bf16x8*)(Kh + (size_t)min(kb0 + row, N - 1) * D + ch * 8);
    *(bf16x8*)(smem + Ly::OFF_K + row * ROWB + ((ch ^ swz_mask<ROWB>(row)) << 4)) = x;
  }

  const int nqt = Npad / kBQ;
  const int it0 = CAUSAL ? kb0 / kBQ : 0;

  // ---- Q / dO / L2 / D tiles: global -> registers -> swizzled LDS rows.
  bf16x8 qreg[Ly::CH], doreg[Ly::CH];
  float ldreg = 0.f;
  auto gload = [&](int it) {
    const int q0 = it * kBQ;
#pragma unroll
    for (int i = 0; i < Ly::CH; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / CPR, ch = ci % CPR;
      const size_t off = (size_t)min(q0 + row, N - 1) * D + ch * 8;
      qreg[i] = *(const bf16x8*)(Qh + off);
      doreg[i] = *(const bf16x8*)(dOh + off);
    }
    if (tid < 2 * kBQ) ldreg = tid < kBQ ? L2h[q0 + tid] : Dh[q0 + tid - kBQ];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Ly::CH; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / CPR, ch = ci % CPR;
      const int off = row * ROWB + ((ch ^ swz_mask<ROWB>(row)) << 4);
      *(bf16x8*)(smem + Ly::OFF_Q + buf * Ly::QTILE + off) = qreg[i];
      *(bf16x8*)(smem + Ly::OFF_DO + buf * Ly::QTILE + off) = doreg[i];
    }
    if (tid < 2 * kBQ) *(float*)(smem + Ly::OFF_LD + buf * Ly::LDTILE + tid * 4) = ldreg;
  };

  // ---- lane-constant LDS offsets
  // Row fragments (A operand of S and dP): row 32 qb + col, chunk 2t + half.
  int rf_off[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = 32 * qb + col;
    rf_off[qb] = r * ROWB + ((half ^ swz_mask<ROWB>(r)) << 4);  // chunk 2t + half = 2t ^ (half)
  }
  // Transposing reads of a row-major tile X (rows = contraction index):
  // lane gets column 32b + col of rows 16u + 4 half + {0..3} (lo) and
  // 16u + 8 + 4 half + {0..3} (hi).  The swizzle does not depend on u.
  const int tr_e = (lane & 15) >> 2;
  const int tr_t = lane & 3;
  const int tr_cg = (lane >> 4) & 1;
  auto tr_off = [&](int rowb_is_256, int hi, int chunk) {
    const int r = 4 * half + tr_e + 8 * hi;
    const int m = rowb_is_256 ? swz_mask<256>(r) : swz_mask<128>(r);
    return r * (rowb_is_256 ? 256 : 128) + ((chunk ^ m) << 4) + (tr_t & 1) * 8;
  };
  int trq_off[DB][2];  // Q / dO / K tiles
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) trq_off[b][hi] = tr_off(ROWB == 256, hi, 4 * b + 2 * tr_cg + (tr_t >> 1));
  int trs_off[2][2];  // dS^T tile (rows of 64 queries), query block qb
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) trs_off[qb][hi] = tr_off(0, hi, 4 * qb + 2 * tr_cg + (tr_t >> 1));
  // dS^T writes: row = local key 32 wave + col, queries 32 qb + 8 g + 4 half.
  const int ds_row = 32 * wave + col;
  const int ds_mask = swz_mask<128>(ds_row);

  const int dq_qb = wave >> 1;
  const int dq_db0 = (wave & 1) * DQB;

  // dQ(tile) += dS K over the workgroup's 128 keys, from dS^T buffer `buf`.
  auto dq_step = [&](int it, int buf) {
    const char* dst = smem + Ly::OFF_DS + buf * Ly::DSTILE;
    const char* kt = smem + Ly::OFF_K;
    f32x16 acc[DQB];
#pragma unroll
    for (int j = 0; j < DQB; ++j) acc[j] = f32x16{};
    int usteps = kBKV / 16;
    if (CAUSAL) usteps = min(usteps, max(0, (it * kBQ + kBQ - 1 - kb0) / 16 + 1));
    for (int u = 0; u < usteps; ++u) {
      const bf16x8 a = tr_frag(dst + u * 16 * Ly::DSROWB + trs_off[dq_qb][0],
                               dst + u * 16 * Ly::DSROWB + trs_off[dq_qb][1]);
#pragma unroll
      for (int j = 0; j < DQB; ++j) {
        const bf16x8 b = tr_frag(kt + u * 16 * ROWB + trq_off[dq_db0 + j][0], kt + u * 16 * ROWB + trq_off[dq_db0 + j][1]);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    // rows of the padded accumulator past N receive zeros (dS = 0 there)
    float* base = dqh + (size_t)(it * kBQ + 32 * dq_qb + 4 * half) * D + col;
#pragma unroll
    for (int j = 0; j < DQB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float* p = base + (size_t)(8 * (r >> 2) + (r & 3)) * D + 32 * (dq_db0 + j);
        unsafeAtomicAdd(p, acc[j][r]);
      }
  };

  f32x16 dkT[DB], dvT[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    dkT[b] = f32x16{};
    dvT[b] = f32x16{};
  }

  gload(it0);
  lstore(0);
  __syncthreads();

  for (int it = it0; it < nqt; ++it) {
    const int buf = (it - it0) & 1;
    if (it + 1 < nqt) gload(it + 1);
    const int q0 = it * kBQ;
    const char* qt = smem + Ly::OFF_Q + buf * Ly::QTILE;
    const char* dot = smem + Ly::OFF_DO + buf * Ly::QTILE;

    // S = Q K^T and dP = dO V^T for the two 32-query blocks.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 a = *(const bf16x8*)(qt + (rf_off[qb] ^ (t << 5)));
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[t], s[qb], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 a = *(const bf16x8*)(dot + (rf_off[qb] ^ (t << 5)));
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[t], dp[qb], 0, 0, 0);
      }
    }

    // dQ of the previous tile (its dS^T was completed before the barrier).
    if (it > it0) dq_step(it - 1, buf ^ 1);

    // P = 2^(s c - L2), dS = P (dP - D); lane: key `key`, queries
    // q0 + 32 qb + 8 g + 4 half + e for accumulator register 4 g + e.
    const float* l2t = (const float*)(smem + Ly::OFF_LD + buf * Ly::LDTILE);
    const float* dt = l2t + kBQ;
    const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (q0 + kBQ > N) || (kw0 + 32 > N);
    bf16x8 pf[4], dsf[4];
    char* dsw = smem + Ly::OFF_DS + buf * Ly::DSTILE + ds_row * Ly::DSROWB + half * 8;  // + chunk * 16
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      unsigned pw[8], dw[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(l2t + 32 * qb + 8 * g + 4 * half);
        const f32x4 d4 = *(const f32x4*)(dt + 32 * qb + 8 * g + 4 * half);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pe = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -l4[e]));
          if (need_mask) {
            const int qi = q0 + 32 * qb + 8 * g + 4 * half + e;
            const bool vis = qi < N && key < N && (!CAUSAL || key <= qi);
            pe = vis ? pe : 0.f;
          }
          p[e] = pe;
          ds[e] = pe * (dp[qb][r] - d4[e]);
        }
        pw[2 * g] = pack_bf16(p[0], p[1]);
        pw[2 * g + 1] = pack_bf16(p[2], p[3]);
        dw[2 * g] = pack_bf16(ds[0], ds[1]);
        dw[2 * g + 1] = pack_bf16(ds[2], ds[3]);
        // dS^T row `ds_row`, queries 32 qb + 8 g + 4 half + {0..3}: chunk 4 qb + g
        *(uint2*)(dsw + (((4 * qb + g) ^ ds_mask) << 4)) = make_uint2(dw[2 * g], dw[2 * g + 1]);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        pf[2 * qb + h2] = __builtin_bit_cast(bf16x8, (u32x4){pw[4 * h2], pw[4 * h2 + 1], pw[4 * h2 + 2], pw[4 * h2 + 3]});
        dsf[2 * qb + h2] = __builtin_bit_cast(bf16x8, (u32x4){dw[4 * h2], dw[4 * h2 + 1], dw[4 * h2 + 2], dw[4 * h2 + 3]});
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS over four 16-query steps.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 a = tr_frag(dot + u * 16 * ROWB + trq_off[b][0], dot + u * 16 * ROWB + trq_off[b][1]);
        dvT[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], dvT[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 a = tr_frag(qt + u * 16 * ROWB + trq_off[b][0], qt + u * 16 * ROWB + trq_off[b][1]);
        dkT[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[u], dkT[b], 0, 0, 0);
      }
    }

    if (it + 1 < nqt) lstore(buf ^ 1);
    __syncthreads();
  }
  dq_step(nqt - 1, (nqt - 1 - it0) & 1);

  // ---- dK = scale * dK^T^T, dV: lane writes key `key`, d = 32 b + 8 g + 4 half + {0..3}.
  if (key < N) {
    __bf16* dkrow = dKg + head + (size_t)key * D + 4 * half;
    __bf16* dvrow = dVg + head + (size_t)key * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ok, ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[e] = (__bf16)(dkT[b][4 * g + e] * scale);
          ov[e] = (__bf16)dvT[b][4 * g + e];
        }
        *(bf16x4*)(dkrow + 32 * b + 8 * g) = ok;
        *(bf16x4*)(dvrow + 32 * b + 8 * g) = ov;
      }
  }
}

template <int D>
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  const int npad = (p.N + kBQ - 1) / kBQ * kBQ;
  float* dqacc = (float*)p.workspace;
  float* l2 = dqacc + (size_t)p.BH * npad * D;
  float* dv = l2 + (size_t)p.BH * npad;
  {
    constexpr int RPB = 256 / (D / 8);
    const size_t rows = (size_t)p.BH * npad;  // a multiple of RPB
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)(rows / RPB)), dim3(256), 0, stream,
                       (const __bf16*)p.o, (const __bf16*)p.dout, p.lse, dqacc, l2, dv, p.N, npad);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (p.N + kBKV - 1) / kBKV;
    const float c = p.scale * kLog2e;
    const dim3 grid((unsigned)(p.BH * nkb)), block(kThreads);
    if (p.causal)
      hipLaunchKernelGGL((bwd_main_kernel<D, true>), grid, block, 0, stream, (const __bf16*)p.q, (const __bf16*)p.k,
                         (const __bf16*)p.v, (const __bf16*)p.dout, l2, dv, dqacc, (__bf16*)p.dk, (__bf16*)p.dv,
                         p.BH, p.N, npad, nkb, c, p.scale);
    else
      hipLaunchKernelGGL((bwd_main_kernel<D, false>), grid, block, 0, stream, (const __bf16*)p.q, (const __bf16*)p.k,
                         (const __bf16*)p.v, (const __bf16*)p.dout, l2, dv, dqacc, (__bf16*)p.dk, (__bf16*)p.dv,
                         p.BH, p.N, npad, nkb, c, p.scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const size_t total8 = (size_t)p.BH * p.N * D / 8;
    hipLaunchKernelGGL(bwd_post_kernel<D>, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, stream, dqacc,
                       (__bf16*)p.dq, p.N, npad, total8, p.scale);
    return hipGetLastError();
  }
}

}  // namespace

size_t bwd_workspace_bytes(int BH, int N, int d) {
  const size_t npad = ((size_t)N + kBQ - 1) / kBQ * kBQ;
  return (size_t)BH * npad * ((size_t)d + 2) * sizeof(float);
}

int bwd_block_k() { return kBKV; }
int bwd_block_q() { return kBQ; }

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_bwd<64>(p, stream) : launch_bwd<128>(p, stream);
}

}  // namespace fa
