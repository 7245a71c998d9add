// Host-side planning of the decode FFN's K split (no device code: the
// kernels in ffn.hip and ffn_split.hip take its results as arguments).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

namespace moe {

constexpr int kMaxParts = 8;   // K parts per item at most

// K split for small batches.  The dispatcher places the first blocks of a
// launch round-robin, block b on CU b % kCus, as many per CU as fit (3 for
// the decode FFN kernels, 4 for the 256-row down tiles), and each CU streams ~18-22
// GB/s however many of its slots are busy, so a launch takes about as long
// as its busiest CU needs for its bytes.  One token on the 288-expert layer
// gives 288 gate/up items of ~260 KB: 32 CUs stream two of them while the
// rest idle after one.  For up to kSplitMaxT tokens, when the unsplit live
// items fit one round of slots, the parts (routed, shared) that minimise the
// busiest CU's bytes, counting kSplitCostBytes for the block starts and the
// partial-sum round trip of a split, are chosen among those whose blocks
// still fit one round and hold at least kSplitMinBytes.  Measured at one
// token (interleaved A/B): the 42-layer step 2.21 -> 1.92 ms (gate/up 3
// routed x 2 shared parts, its launch 26.4 -> 21-22 us), the coarse layer
// 0.885 -> 0.847 ms (down in 2 parts).  Left whole by the rule, and slower
// when split: the balanced down launch of the 288-expert layer and the
// 512-expert layer's launches (fewer items than CUs); the gate/up launch
// with the 8-bit shared expert (2-5% slower in 2 routed parts, which set
// kSplitCostBytes) is never split.
constexpr int kCus = 256;
constexpr int kSplitMaxT = 4;
constexpr int64_t kSplitMinBytes = 48 << 10;
constexpr int64_t kSplitCostBytes = 160 << 10;

// Bytes of the busiest CU when ns blocks of sb bytes and then nr blocks of rb
// bytes (at most slots * kCus in all) are placed on CU b % kCus.  A CU's load
// only changes where c + j * kCus crosses ns or ns + nr, so those points (and
// 0) are the only ones to evaluate.
inline int64_t busiest_cu(int64_t ns, int64_t sb, int64_t nr, int64_t rb, int slots) {
  const int64_t n = ns + nr;
  auto load = [&](int64_t c) {
    int64_t v = 0;
    for (int j = 0; j < slots; ++j) {
      const int64_t b = c + (int64_t)j * kCus;
      v += b < ns ? sb : (b < n ? rb : 0);
    }
    return v;
  };
  int64_t m = load(0);
  for (int j = 0; j < slots; ++j)
    for (int64_t edge : {ns, n})
      for (int64_t c : {edge - (int64_t)j * kCus - 1, edge - (int64_t)j * kCus})
        if (c >= 0 && c < kCus) {
          const int64_t v = load(c);
          m = v > m ? v : m;
        }
  return m;
}

// nr live routed items of rb bytes (at most max_rp parts) and ns shared items
// of sb bytes (at most max_sp parts) -> parts per item.
inline void split_parts(int64_t nr, int64_t rb, int max_rp, int64_t ns, int64_t sb, int max_sp,
                        int slots, int *rp, int *sp) {
  *rp = *sp = 1;
  const int64_t round = (int64_t)slots * kCus;
  if (nr + ns > round) return;
  int64_t best = busiest_cu(ns, sb, nr, rb, slots);
  for (int r = 1; r <= max_rp && r <= kMaxParts; ++r)
    for (int q = 1; q <= (ns ? max_sp : 1) && q <= kMaxParts; ++q) {
      if ((r == 1 && q == 1) || nr * r + ns * q > round) continue;
      if ((r > 1 && rb / r < kSplitMinBytes) || (q > 1 && sb / q < kSplitMinBytes)) continue;
      const int64_t c = busiest_cu(ns * q, ns ? sb / q : 0, nr * r, rb / r, slots) + kSplitCostBytes;
      if (c < best) {
        best = c;
        *rp = r;
        *sp = q;
      }
    }
}

// Partial-sum floats of a split launch: one round of slots * kCus blocks, each
// 4 waves x `tiles` 16-row tiles x tm token rows x 16 weight rows.
inline size_t split_floats(int slots, int tiles, int tm) {
  return (size_t)slots * kCus * 4 * tiles * tm * 16;
}

}  // namespace moe
