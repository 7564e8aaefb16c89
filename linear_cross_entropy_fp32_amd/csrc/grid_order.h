// Workgroup-to-tile orders of the logit-tile and contraction launches.
//
// Plain integer arithmetic with no HIP types, so that the same functions the
// kernels call can be compiled into a host program and checked there
// (tests/native/grid_order_check.cpp).  A file that includes this header from
// device code defines FLCE_HD as "__host__ __device__" first.
#pragma once

#ifndef FLCE_HD
#define FLCE_HD
#endif

namespace flce {

// Order over a (token tile, vocabulary group) grid in windows of up to
// G groups x T token tiles, G = W / T (W workgroups: what one XCD holds at
// once, 32 x the workgroups per CU; W and T powers of two, T <= W).  Inside
// a window, consecutive workgroups share the operand that benefits most from
// being read by workgroups that run in step: the vocabulary group (token tile fastest) when all token
// tiles fit in L2 anyway, else the token tile (group fastest).  Windows run
// over the token tiles of a band of G groups, then the next band; edge
// windows are narrower.  The map is a bijection onto the n_tt x n_grp grid.
struct GridPos {
  int tt, grp;
};
FLCE_HD inline GridPos grouped_order(int id, int n_tt, int n_grp, int T, bool tt_fastest, int W) {
  const int G = W / T;
  const int b = id / (n_tt * G), r = id - b * (n_tt * G);
  const int gh = n_grp - b * G < G ? n_grp - b * G : G;    // groups in this band
  const int tb = r / (T * gh), j = r - tb * (T * gh);
  const int tw = n_tt - tb * T < T ? n_tt - tb * T : T;    // token tiles in this window
  return tt_fastest ? GridPos{tb * T + j % tw, b * G + j / tw}
                    : GridPos{tb * T + j / gh, b * G + j % gh};
}

// Map a linear workgroup id so that ids adjacent in the logical order land on
// the same XCD (workgroups are dealt to the 8 XCDs round robin), keeping tiles
// that share an operand in one L2.  A bijection on [0, nblocks).
FLCE_HD inline int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int full = nblocks - nblocks % kXcd;
  if (bid >= full) return bid;
  const int per = full / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace flce
