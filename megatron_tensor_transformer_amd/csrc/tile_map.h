// Workgroup -> (problem, tile) order of the GEMM launches, host- and
// device-callable so that the CPU tests can check it is a bijection.
//
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2),
// in increasing index: workgroup w runs on XCD w % 8 as its (w / 8)-th.  A
// launch has a long group of tiles (problem 0's T0, then problem 1's T1; the
// long-K problems) and a short one (problem 2's T2).  Its tiles form one
// logical sequence in which the two groups are interleaved in proportion
// (position j is preceded by floor(j·G/T) long-group tiles, G = T0 + T1,
// T = G + T2).  XCD x takes a contiguous range of that sequence, exactly as
// many positions as the round-robin deal gives it, and works first through
// the long-group tiles of its range, then the short-group ones: every XCD gets
// its proportional share of both, the long tiles first so the short ones fill
// in behind them.  ("Long group" names the problems' role in the launch, not
// their K: when the short problem's tiles take more K steps than the long
// group's, e.g. dgrad-2 with K = m_i against weight gradients with K = n at
// few tokens, the launch sets short_first and each XCD runs its range's
// short-problem tiles first.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

// Positions [begin, begin + count) of the logical sequence of `total` that the
// round-robin deal gives XCD `xcd`.
__host__ __device__ inline void xcd_range(int total, int xcd, int& begin, int& count) {
  const int q = total >> 3, r = total & 7;
  begin = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  count = xcd < r ? q + 1 : q;
}

// Per XCD: where its range starts in the short problem (short0), where it
// starts in the long group (long0) and how many long-group tiles it has
// (nlong).  Computed once per launch on the host (it needs 64-bit divisions).
struct XcdSplit {
  int long0[8], nlong[8], short0[8], nshort[8];
  int short_first;  // 1: each XCD runs its short-problem tiles before its long-group ones
};

__host__ __device__ inline XcdSplit make_split(int t0, int t1, int t2, bool short_first = false) {
  const int64_t glong = static_cast<int64_t>(t0) + t1, total = glong + t2;
  XcdSplit s;
  s.short_first = short_first ? 1 : 0;
  for (int x = 0; x < 8; ++x) {
    int begin, count;
    xcd_range(static_cast<int>(total), x, begin, count);
    // long-group tiles before position j: floor(j·glong/total)
    const int a = total > 0 ? static_cast<int>(begin * glong / total) : 0;
    const int b = total > 0 ? static_cast<int>((static_cast<int64_t>(begin) + count) * glong / total) : 0;
    s.long0[x] = a;
    s.nlong[x] = b - a;
    s.short0[x] = begin - a;
    s.nshort[x] = count - (b - a);
  }
  return s;
}

// prob: 0, 1 (the long group: problem 0's t0 tiles, then problem 1's) or 2
// (the short problem); tile: index within that problem.
__host__ __device__ inline void map_workgroup(const XcdSplit& s, int t0, int wg, int& prob, int& tile) {
  const int xcd = wg & 7, local = wg >> 3;
  int lk;  // position among the XCD's long-group tiles, or -1 for a short one
  if (!s.short_first) {
    lk = local < s.nlong[xcd] ? local : -1;
    if (lk < 0) {
      prob = 2;
      tile = s.short0[xcd] + (local - s.nlong[xcd]);
      return;
    }
  } else {
    const int nshort = s.nshort[xcd];
    if (local < nshort) {
      prob = 2;
      tile = s.short0[xcd] + local;
      return;
    }
    lk = local - nshort;
  }
  const int k = s.long0[xcd] + lk;
  prob = k < t0 ? 0 : 1;
  tile = k < t0 ? k : k - t0;
}

// Attention launches: `heads` independent sequences of `nblk` blocks each, in
// the logical order head by head; block position p (0 = the most work, e.g.
// the last causal query block) of head h is logical index h·nblk + p.  XCD x
// keeps its contiguous range of that order (a head's blocks read the same
// K/V or Q/dO panel, so they share its L2), but runs it position-major: all
// its heads' position-0 blocks first, then position 1, ...  so the longest
// blocks start first and the short ones fill in behind them.  wg -> (head, p).
__host__ __device__ inline void heavy_first_block(int heads, int nblk, int wg, int& head, int& p) {
  const int total = heads * nblk;
  int begin, count;
  xcd_range(total, wg & 7, begin, count);
  const int local = wg >> 3;
  const int last = begin + count - 1;
  const int h_first = begin / nblk, p_first = begin - h_first * nblk;
  const int h_last = last / nblk, p_last = last - h_last * nblk;
  const int H = h_last - h_first + 1;
  // Blocks at positions < P in the range: every head of the run has one at
  // each position, except the first head before p_first and the last head
  // after p_last.  Monotone in P: the position of `local` by bisection.
  auto before = [&](int P) {
    return P * H - (P < p_first ? P : p_first) - (P - p_last - 1 > 0 ? P - p_last - 1 : 0);
  };
  int lo = 0, hi = nblk - 1;  // largest P with before(P) <= local
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (before(mid) <= local) lo = mid;
    else hi = mid - 1;
  }
  p = lo;
  head = (p >= p_first ? h_first : h_first + 1) + (local - before(p));
}

}  // namespace tpmlp
