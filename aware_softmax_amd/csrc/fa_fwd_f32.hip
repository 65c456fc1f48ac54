// FlashAttention-2 forward in float32 (float32 in/out, fp32 arithmetic).
//
// Same method as the bf16 path ("FlashAttention-2: Why the Attention
// Bottleneck Wasn't Where Everyone Was Looking", "FA2 change #1"/"#2";
// "FlashAttention: Move Less, Not Compute Less", "Tiling Is Easy"): one
// workgroup per (head, query block), 64-key K/V tiles in LDS, running
// (m, l, unnormalised O) per row, one division by l at the end.  It exists
// for full-precision callers: every product and sum is an fp32 FMA (no
// reduced-precision path), so results stay within a few fp32 ulps of the
// exact attention.  Two kernels:
//   * grids that fill the chip: fwd_f32_mfma_kernel, the products on the
//     fp32 matrix cores (v_mfma_f32_32x32x2_f32), 128-row blocks;
//   * grids of at most kSmallGrid 64-row blocks: fwd_f32_kernel on the
//     VALU.  LPR lanes share a query row: each scores 64 / LPR of the
//     tile's 64 keys and owns 1 / LPR of the output columns; the
//     probabilities of a row are exchanged through LDS; a workgroup is 256
//     threads, 256 / LPR query rows.  The time there is one workgroup's
//     chain of dependent FMAs and LDS reads, which LPR = 16 (16-row blocks;
//     8 lanes and 32 rows at d = 32 and 96) keeps short.
#include <math.h>

#include "fa_internal.h"
#include "fa_schedule.h"

namespace fa {
namespace {

constexpr int kBQ = 64;  // the block size that decides "small grid"
constexpr int kBK = 64;
constexpr int kThreads = 256;
// Grids of at most this many 64-row blocks run the VALU kernel.
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

// ---------------------------------------------------------------------------
// The same method on the fp32 matrix cores (d = 32 to 128), for grids large
// enough to fill the chip: v_mfma_f32_32x32x2_f32 computes every product
// in fp32 with fp32 sums, like the VALU kernel, while the VALU is left to
// the softmax and the matrix unit reuses each operand 32 times (the VALU
// kernel reads one LDS value per FMA and is bound by that).
//   * 4 waves, 128 query rows (32 per wave), 64-key tiles of K and V in
//     one LDS buffer, loaded into registers one tile ahead and stored
//     between two barriers; the small LDS footprint lets two workgroups
//     share a CU (two waves per SIMD);
//   * S^T = K Q^T (keys x the wave's queries) in two 32-key halves: MFMA
//     step s takes, in lane half h, dimension (D/2) h + s of the key row
//     (A) and of the lane's query row (B), so a lane reads four steps of
//     its key row with one 16-byte LDS read and keeps its Q row in
//     registers;
//   * O^T += V^T P^T: step s of key half kb takes in lane half h the key
//     that register s of the score accumulator holds there (8 (s/4) + 4 h
//     + s%4), so P is the accumulator itself, and each lane reads one fp32
//     V value (row of that key, its output dimension) per step;
//   * K rows are padded by 16 bytes and V rows by 32 bytes in LDS, so the
//     16-byte K reads of 16 lanes and the 4-byte V reads of 64 lanes fall
//     on distinct banks.
typedef float f32x16m __attribute__((ext_vector_type(16)));

// Waves per SIMD: two (four at d = 32, whose registers allow it: +6 % on B2
// H16 N4096; three at d = 64 lost 5 %).
template <int D>
constexpr int f32_mfma_waves() {
  return D <= 32 ? 4 : 2;
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(f32_mfma_waves<D>(), f32_mfma_waves<D>()))) void fwd_f32_mfma_kernel(const float* __restrict__ Qg,
                                                          const float* __restrict__ Kg,
                                                          const float* __restrict__ Vg, float* __restrict__ Og,
                                                          float* __restrict__ Lg, int BH, int N, int nqb, float c,
                                                          int group) {
  constexpr int BQ = 128;
  constexpr int KS = D + 4;  // K row stride (floats)
  constexpr int VS = D + 8;  // V row stride (floats)
  constexpr int HALF = D / 2;
  constexpr int DB = D / 32;
  constexpr int LPT = kBK * D / 4 / 256;  // float4 loads per thread and tensor
  __shared__ __attribute__((aligned(16))) float Ks[1][kBK * KS];  // one buffer: 2 workgroups per CU
  __shared__ __attribute__((aligned(16))) float Vs[1][kBK * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int h = lane >> 5;
  int bh, qb;
  map_block(blockIdx.x, BH * nqb, nqb, CAUSAL ? Order::HeavyLast : Order::Plain, &bh, &qb);
  const int q0 = qb * BQ;
  const int qw = q0 + 32 * wave;
  const int qi = qw + col;
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t kvhead = (size_t)(bh / group) * (size_t)N * D;
  const float* Kh = Kg + kvhead;
  const float* Vh = Vg + kvhead;

  // Q row of the lane's query, dimensions HALF h .. HALF h + HALF - 1
  float qv[HALF];
#pragma unroll
  for (int x = 0; x < HALF; x += 4) {
    const float4 t = qi < N ? *(const float4*)(Qg + head + (size_t)qi * D + HALF * h + x)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    qv[x] = t.x;
    qv[x + 1] = t.y;
    qv[x + 2] = t.z;
    qv[x + 3] = t.w;
  }

  int nkt = (N + kBK - 1) / kBK;
  if (CAUSAL) nkt = min(nkt, (q0 + BQ - 1) / kBK + 1);
  // this wave's tiles: none past its last row's diagonal
  int wave_nt = nkt;
  if (CAUSAL) wave_nt = min(nkt, (qw + 31) / kBK + 1);
  if (qw >= N) wave_nt = 0;

  float4 kst[LPT], vst[LPT];
  auto gload = [&](int j) {
    const int kt0 = j * kBK;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ci = tid + 256 * i;
      const int r = ci / (D / 4), x = (ci % (D / 4)) * 4;
      if (kt0 + r < N) {
        kst[i] = *(const float4*)(Kh + (size_t)(kt0 + r) * D + x);
        vst[i] = *(const float4*)(Vh + (size_t)(kt0 + r) * D + x);
      } else {
        kst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        vst[i] = kst[i];
      }
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ci = tid + 256 * i;
      const int r = ci / (D / 4), x = (ci % (D / 4)) * 4;
      *(float4*)(&Ks[b][r * KS + x]) = kst[i];
      *(float4*)(&Vs[b][r * VS + x]) = vst[i];
    }
  };

  f32x16m oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = f32x16m{};
  float m_run = -INFINITY;  // log2 units
  float l_part = 0.f;

  if (nkt > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int j = 0; j < nkt; ++j) {
    const int buf = 0;
    if (j + 1 < nkt) gload(j + 1);
    if (j < wave_nt) {
      const int kt0 = j * kBK;
      const float* kb_ = &Ks[buf][0];
      const float* vb_ = &Vs[buf][0];
      f32x16m sacc[2];
      sacc[0] = sacc[1] = f32x16m{};
      // the two key halves' accumulation chains alternate MFMA by MFMA
#pragma unroll
      for (int x = 0; x < HALF; x += 4) {
        const float4 k0 = *(const float4*)(kb_ + col * KS + HALF * h + x);
        const float4 k1 = *(const float4*)(kb_ + (32 + col) * KS + HALF * h + x);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0.x, qv[x], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1.x, qv[x], sacc[1], 0, 0, 0);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0.y, qv[x + 1], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1.y, qv[x + 1], sacc[1], 0, 0, 0);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0.z, qv[x + 2], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1.z, qv[x + 2], sacc[1], 0, 0, 0);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0.w, qv[x + 3], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1.w, qv[x + 3], sacc[1], 0, 0, 0);
      }
      // scale, mask, running max (log2 units)
      const bool need_mask = (CAUSAL && kt0 + kBK - 1 > qw) || kt0 + kBK > N;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = sacc[kb][r] * c;
          if (need_mask) {
            const int key = kt0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            if ((CAUSAL && key > qi) || key >= N) t = -INFINITY;
          }
          sacc[kb][r] = t;
          mx = fmaxf(mx, t);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // hardware exp2 (a result below 2^-126 flushes to zero, far below
          // the fp32 resolution of l >= 1); masked: 2^-inf = 0
          const float pr = __builtin_amdgcn_exp2f(sacc[kb][r] - m_use);
          sacc[kb][r] = pr;
          psum += pr;
        }
      l_part = alpha * l_part + psum;
      // the running max rarely moves after the first tiles: rescale O only
      // when some lane's did
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b) oacc[b] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 16; ++st) {
          const int key = 32 * kb + 8 * (st >> 2) + 4 * h + (st & 3);
#pragma unroll
          for (int b = 0; b < DB; ++b)
            oacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(vb_[key * VS + 32 * b + col], sacc[kb][st], oacc[b], 0,
                                                          0, 0);
        }
    }
    if (j + 1 < nkt) {
      __syncthreads();  // every wave is done with tile j
      lstore(0);
    }
    __syncthreads();
  }

  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (qi < N) {
    const float inv = 1.f / l_tot;
    float* orow = Og + head + (size_t)qi * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(orow + 32 * b + 8 * g + 4 * h) =
            make_float4(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv, oacc[b][4 * g + 2] * inv,
                        oacc[b][4 * g + 3] * inv);
    if (h == 0) Lg[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const float c = p.scale * 1.44269504088896340736f;
  const float* q = (const float*)p.q;
  const float* k = (const float*)p.k;
  const float* v = (const float*)p.v;
  float* o = (float*)p.o;
  float* lse = p.lse;
  int bh = p.BH, n = p.N, group = p.group;
  if ((int64_t)p.BH * ((p.N + kBQ - 1) / kBQ) > kSmallGrid) {  // the matrix-core kernel, 128-row blocks
    int nqb = (p.N + 127) / 128;
    void* args[] = {&q, &k, &v, &o, &lse, &bh, &n, (void*)&nqb, (void*)&c, &group};
    return hipLaunchKernel((const void*)fwd_f32_mfma_kernel<D, CAUSAL>, dim3(p.BH * nqb), dim3(256), args, 0,
                           stream);
  }
  // small grids: the VALU kernel with 16 lanes per row (8 at d = 32 and
  // 96, whose columns split into float4 groups only eight ways)
  constexpr int kLpr = D % 64 == 0 ? 16 : 8;
  int nqb = (p.N + kThreads / kLpr - 1) / (kThreads / kLpr);
  void* args[] = {&q, &k, &v, &o, &lse, &bh, &n, (void*)&nqb, (void*)&c, &group};
  return hipLaunchKernel((const void*)fwd_f32_kernel<D, CAUSAL, kLpr>, dim3(p.BH * nqb), dim3(kThreads), args, 0,
                         stream);
}

}  // namespace

TileConfig f32_tile(int) { return TileConfig{128, kBK, 4}; }  // the matrix-core kernel

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
