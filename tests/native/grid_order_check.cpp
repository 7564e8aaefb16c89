// Host check of the workgroup orders the kernels use (grid_order.h, the same
// functions, compiled for the host): for every window size the planner picks
// (windows of W = 32 or 64 workgroups, T = 1, 2, 4, 8 token tiles x W/T
// vocabulary groups), both inner orders and
// a spread of grid shapes, grouped_order maps the workgroup ids one to one
// onto the token-tile x group grid, and xcd_remap is a permutation of the ids.
// A map that missed or repeated a cell would leave logits unreduced or make a
// workgroup write its partial states past the split count.
// Prints "ok <cases>" and exits 0, or names the first failing case and exits 1.
#include <cstdio>
#include <vector>

#include "grid_order.h"

int main() {
  const int tts[] = {1, 2, 3, 7, 8, 9, 17, 64};
  const int grps[] = {1, 5, 31, 32, 33, 63, 64, 65, 250};
  std::vector<std::pair<int, int>> shapes;
  for (int a : tts)
    for (int b : grps) shapes.push_back({a, b});
  shapes.push_back({8, 256});
  shapes.push_back({32, 63});
  shapes.push_back({64, 32});
  shapes.push_back({64, 63});
  shapes.push_back({3, 71});
  shapes.push_back({128, 1187});   // 16384 tokens, 151936 / 128 vocabulary tiles
  long cases = 0;
  for (int W = 32; W <= 64; W *= 2)
    for (int T = 1; T <= 8; T *= 2)
      for (int fast = 0; fast < 2; ++fast)
        for (auto [n_tt, n_grp] : shapes) {
          std::vector<char> seen((size_t)n_tt * n_grp, 0);
          for (int id = 0; id < n_tt * n_grp; ++id) {
            const flce::GridPos p = flce::grouped_order(id, n_tt, n_grp, T, fast != 0, W);
            if (p.tt < 0 || p.tt >= n_tt || p.grp < 0 || p.grp >= n_grp ||
                seen[(size_t)p.tt * n_grp + p.grp]) {
              std::printf("grouped_order fails: W=%d T=%d fast=%d n_tt=%d n_grp=%d id=%d\n", W,
                          T, fast, n_tt, n_grp, id);
              return 1;
            }
            seen[(size_t)p.tt * n_grp + p.grp] = 1;
          }
          ++cases;
        }
  for (int nb = 1; nb <= 5000; nb += (nb < 300 ? 1 : 97)) {
    std::vector<char> seen(nb, 0);
    for (int b = 0; b < nb; ++b) {
      const int r = flce::xcd_remap(b, nb);
      if (r < 0 || r >= nb || seen[r]) {
        std::printf("xcd_remap fails: nblocks=%d bid=%d\n", nb, b);
        return 1;
      }
      seen[r] = 1;
    }
    ++cases;
  }
  std::printf("ok %ld\n", cases);
  return 0;
}
