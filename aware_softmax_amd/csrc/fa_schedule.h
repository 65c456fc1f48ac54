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
// freebie"); the heaviest blocks are issued first (within a head, or across
// all of an XCD's heads when the launch is only a few rounds deep) so the
// light ones fill the tail of the launch.
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

// Up to this many workgroups per XCD (a few rounds of its 32 CUs) the
// launch ends with a ragged tail unless the heaviest blocks of ALL the
// XCD's heads start first: then a CU that finishes a light block picks up
// the next-heaviest one, and the per-CU sums even out (longest-first list
// scheduling).  Beyond it the head-by-head order keeps one head's K/V in the
// XCD's L2 and the tail is a small part of many rounds.
constexpr int kLptMaxPerXcd = 128;

// Which block of a head carries the most work.
enum class Order {
  Plain,       // all blocks alike (no causal mask): head by head, block 0 first
  HeavyLast,   // causal query blocks: block nqb - 1 streams the most key tiles
  HeavyFirst,  // causal key blocks: block 0 streams the most query tiles
};

// id in [0, total) -> (bh, qb) with bh in [0, total / nqb), qb in [0, nqb).
// A bijection for any total = heads * nqb >= 1.
FA_HD inline void map_block(int id, int total, int nqb, Order order, int* bh, int* qb) {
  const int per = total / kNumXcd;
  const int rem = total % kNumXcd;
  const int xcd = id % kNumXcd;
  const int slot = id / kNumXcd;
  int ord;
  if (order != Order::Plain && rem == 0 && per % nqb == 0 && per <= kLptMaxPerXcd) {
    // the XCD holds whole heads: rank r of every head before rank r + 1
    const int nh = per / nqb;
    const int r = slot / nh;
    ord = xcd * per + (slot - r * nh) * nqb + r;
  } else {
    ord = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  }
  *bh = ord / nqb;
  const int r = ord - *bh * nqb;  // rank within the head, heaviest first
  *qb = order == Order::HeavyLast ? (nqb - 1 - r) : r;
}

}  // namespace fa
