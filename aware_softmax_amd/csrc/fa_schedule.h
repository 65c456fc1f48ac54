// Workgroup-id -> (head, query block) schedule, shared by host self-checks
// and device code.
//
// "FlashAttention-2: Why the Attention Bottleneck Wasn't Where Everyone Was
// Looking", "FA2 change #2": every query row block is an independent worker,
// so the grid is (batch * heads) x (query blocks).  On MI355X the hardware
// hands consecutive workgroup ids to the 8 XCDs round-robin, and each XCD
// has its own L2.  The remap below gives every XCD a contiguous range of
// heads, so the workgroups that stream one head's K/V tiles share an L2.
// With a causal mask, block i streams i + 1 key tiles ("The causal masking
// freebie"); within a head the heaviest blocks are issued first so the light
// ones fill the tail of the launch.
#pragma once

#ifndef FA_HD
#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif
#endif

namespace fa {

constexpr int kNumXcd = 8;

// id in [0, total) -> (bh, qb) with bh in [0, total / nqb), qb in [0, nqb).
// A bijection for any total = heads * nqb >= 1.
FA_HD inline void map_block(int id, int total, int nqb, bool heavy_first, int* bh, int* qb) {
  const int per = total / kNumXcd;
  const int rem = total % kNumXcd;
  const int xcd = id % kNumXcd;
  const int slot = id / kNumXcd;
  const int ord = (xcd < rem) ? xcd * (per + 1) + slot
                              : rem * (per + 1) + (xcd - rem) * per + slot;
  *bh = ord / nqb;
  const int r = ord - *bh * nqb;
  *qb = heavy_first ? (nqb - 1 - r) : r;
}

}  // namespace fa
