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

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

      // Mask: only tiles crossing this wave's diagonal or the ragged end.
      const bool need_mask = (CAUSAL && kt0 + kBK - 1 > qw) || (kt0 + kBK > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            if ((CAUSAL && key > qi) || key >= N) s[kb][r] = -INFINITY;
          }
      }

      // Row max (in-lane over 32 keys, then across the lane pair).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = swap_halves(mx, true);
      const float mc = (mx == -INFINITY) ? -INFINITY : mx * c;
      const float m_new = fmaxf(m_run, mc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      // P = 2^(S*c - m'), partial row sum, rescale O.
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_use));
          if (need_mask && s[kb][r] == -INFINITY) p = 0.f;
          psum += p;
          s[kb][r] = p;
        }
      l_part = alpha * l_part + psum;
#pragma unroll
      for (int b = 0; b < DB; ++b) oacc[b] *= alpha;

      // O^T += V^T P^T, four 16-key steps.
#pragma unroll
      for (int u = 0; u < kBK / 16; ++u) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (__bf16)s[u >> 1][(u & 1) * 8 + e];
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

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int nqb = (p.N + kBQ - 1) / kBQ;
  const float c_signed = p.scale * 1.44269504088896340736f;
  const int negate = p.scale < 0.f ? 1 : 0;
  const float c = negate ? -c_signed : c_signed;
  dim3 grid(p.BH * nqb), block(kThreads);
  const __bf16* q = (const __bf16*)p.q;
  const __bf16* k = (const __bf16*)p.k;
  const __bf16* v = (const __bf16*)p.v;
  __bf16* o = (__bf16*)p.o;
  float* lse = p.lse;
  int bh = p.BH, n = p.N;
  void* args[] = {&q, &k, &v, &o, &lse, &bh, &n, (void*)&nqb, (void*)&c, (void*)&negate};
  return hipLaunchKernel((const void*)fwd_bf16_kernel<D, CAUSAL>, grid, block, args, 0, stream);
}

}  // namespace

TileConfig bf16_tile(int) { return TileConfig{kBQ, kBK, kWaves}; }

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
