// FlashAttention-2 forward in float32 (float32 in/out, fp32 arithmetic).
//
// Same method as the bf16 path ("FlashAttention-2: Why the Attention
// Bottleneck Wasn't Where Everyone Was Looking", "FA2 change #1"/"#2";
// "FlashAttention: Move Less, Not Compute Less", "Tiling Is Easy"): one
// workgroup per (head, 64-query block), 64-key K/V tiles in LDS, running
// (m, l, unnormalised O) per row, one division by l at the end.  It exists
// for full-precision callers: every product and sum is an fp32 VALU FMA
// (no reduced-precision matrix path), so results stay within a few fp32
// ulps of the exact attention.  LPR lanes share a query row: each scores
// 64 / LPR of the tile's 64 keys and owns 1 / LPR of the output columns;
// the probabilities of a row are exchanged through LDS; a workgroup is 256
// threads, 256 / LPR query rows.  LPR = 4 (64-row blocks) on large grids;
// on grids too small to fill the chip the time is one workgroup's chain of
// dependent FMAs and LDS reads, and LPR = 16 (16-row blocks; 8 and 32 rows
// at d = 32 and 96) cuts it by four.
#include <math.h>

#include "fa_internal.h"
#include "fa_schedule.h"

namespace fa {
namespace {

constexpr int kBQ = 64;  // query rows per workgroup on large grids (LPR = 4)
constexpr int kBK = 64;
constexpr int kThreads = 256;
// Grids of at most this many 64-row blocks run more lanes per row.
constexpr int kSmallGrid = 256;

template <int D, bool CAUSAL, int LPR>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ Qg,
                                                          const float* __restrict__ Kg,
                                                          const float* __restrict__ Vg,
                                                          float* __restrict__ Og,
                                                          float* __restrict__ Lg, int BH, int N,
                                                          int nqb, float c, int group) {
  constexpr int THREADS = kThreads;
  constexpr int BQ = kThreads / LPR;  // query rows per workgroup
  constexpr int KPL = kBK / LPR;  // keys per lane
  constexpr int KP = D + 4;       // padded K row (floats)
  constexpr int PP = kBK + 1;     // padded P row
  constexpr int DQ = D / LPR;     // output columns per lane
  static_assert(DQ % 4 == 0, "whole float4 column groups per lane");
  __shared__ __attribute__((aligned(16))) float Kl[kBK * KP];
  __shared__ __attribute__((aligned(16))) float Vl[kBK * D];
  __shared__ float Pl[BQ * PP];

  const int tid = threadIdx.x;
  const int row = tid / LPR;
  const int sub = tid % LPR;
  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL ? Order::HeavyLast : Order::Plain, &bh, &qb);
  const int q0 = qb * BQ;
  const int qi = q0 + row;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float* Qh = Qg + head;
  // Query heads of a group are consecutive, so head bh reads key/value
  // head bh / group.
  const size_t kvhead = (size_t)(bh / group) * (size_t)N * D;
  const float* Kh = Kg + kvhead;
  const float* Vh = Vg + kvhead;

  float qv[D];
#pragma unroll
  for (int x = 0; x < D; x += 4) {
    float4 t = (qi < N) ? *(const float4*)(Qh + (size_t)qi * D + x) : make_float4(0.f, 0.f, 0.f, 0.f);
    qv[x] = t.x;
    qv[x + 1] = t.y;
    qv[x + 2] = t.z;
    qv[x + 3] = t.w;
  }
  float oacc[DQ];
#pragma unroll
  for (int x = 0; x < DQ; ++x) oacc[x] = 0.f;
  float m_run = -INFINITY;  // log2 units (scores times c)
  float l_part = 0.f;

  int nkt = (N + kBK - 1) / kBK;
  if (CAUSAL) nkt = min(nkt, (q0 + BQ - 1) / kBK + 1);

  for (int j = 0; j < nkt; ++j) {
    const int kt0 = j * kBK;
    __syncthreads();  // previous tile fully consumed
    for (int ci = tid; ci < kBK * D / 4; ci += THREADS) {
      const int r = ci / (D / 4);
      const int x = (ci % (D / 4)) * 4;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (kt0 + r < N) {
        kk = *(const float4*)(Kh + (size_t)(kt0 + r) * D + x);
        vv = *(const float4*)(Vh + (size_t)(kt0 + r) * D + x);
      }
      *(float4*)(Kl + r * KP + x) = kk;
      *(float4*)(Vl + r * D + x) = vv;
    }
    __syncthreads();

    float s[KPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int key = sub + LPR * i;
      const float* kr = Kl + key * KP;
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < D; x += 4) {
        const float4 kk = *(const float4*)(kr + x);
        acc = fmaf(qv[x], kk.x, acc);
        acc = fmaf(qv[x + 1], kk.y, acc);
        acc = fmaf(qv[x + 2], kk.z, acc);
        acc = fmaf(qv[x + 3], kk.w, acc);
      }
      const int kg = kt0 + key;
      // score in log2 units: scale * log2(e) * q.k  (any sign of scale)
      const float t = ((CAUSAL && kg > qi) || kg >= N) ? -INFINITY : acc * c;
      s[i] = t;
      mx = fmaxf(mx, t);
    }
#pragma unroll
    for (int x = 1; x < LPR; x <<= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const float p = exp2f(s[i] - m_use);  // masked: 2^-inf = 0
      psum += p;
      Pl[row * PP + sub + LPR * i] = p;
    }
    l_part = alpha * l_part + psum;
#pragma unroll
    for (int x = 0; x < DQ; ++x) oacc[x] *= alpha;
    __syncthreads();  // P row visible to the 4 lanes of the row
    const float* vcol = Vl + sub * DQ;
    for (int key = 0; key < kBK; ++key) {
      const float p = Pl[row * PP + key];
#pragma unroll
      for (int x = 0; x < DQ; x += 4) {
        const float4 vv = *(const float4*)(vcol + key * D + x);
        oacc[x] = fmaf(p, vv.x, oacc[x]);
        oacc[x + 1] = fmaf(p, vv.y, oacc[x + 1]);
        oacc[x + 2] = fmaf(p, vv.z, oacc[x + 2]);
        oacc[x + 3] = fmaf(p, vv.w, oacc[x + 3]);
      }
    }
  }

  float l_tot = l_part;
#pragma unroll
  for (int x = 1; x < LPR; x <<= 1) l_tot += __shfl_xor(l_tot, x);
  if (qi < N) {
    float* orow = Og + head + (size_t)qi * D + sub * DQ;
#pragma unroll
    for (int x = 0; x < DQ; x += 4)
      *(float4*)(orow + x) = make_float4(oacc[x] / l_tot, oacc[x + 1] / l_tot, oacc[x + 2] / l_tot,
                                         oacc[x + 3] / l_tot);
    if (sub == 0) Lg[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const float c = p.scale * 1.44269504088896340736f;
  // small grids: 16 lanes per row (8 at d = 32 and 96, whose columns
  // split into float4 groups only eight ways)
  constexpr int kSmallLpr = D % 64 == 0 ? 16 : 8;
  const bool small = (int64_t)p.BH * ((p.N + kBQ - 1) / kBQ) <= kSmallGrid;
  const int bq = small ? kThreads / kSmallLpr : kBQ;
  const int nqb = (p.N + bq - 1) / bq;
  dim3 grid(p.BH * nqb), block(kThreads);
  const float* q = (const float*)p.q;
  const float* k = (const float*)p.k;
  const float* v = (const float*)p.v;
  float* o = (float*)p.o;
  float* lse = p.lse;
  int bh = p.BH, n = p.N;
  int group = p.group;
  void* args[] = {&q, &k, &v, &o, &lse, &bh, &n, (void*)&nqb, (void*)&c, &group};
  const void* fn = small ? (const void*)fwd_f32_kernel<D, CAUSAL, kSmallLpr> : (const void*)fwd_f32_kernel<D, CAUSAL, 4>;
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace

TileConfig f32_tile(int) { return TileConfig{kBQ, kBK, kThreads / 64}; }

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 32: return p.causal ? launch<32, true>(p, stream) : launch<32, false>(p, stream);
    case 64: return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
    case 96: return p.causal ? launch<96, true>(p, stream) : launch<96, false>(p, stream);
    case 128: return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
