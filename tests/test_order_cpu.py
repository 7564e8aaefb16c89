"""The logit-tile workgroup order (grouped_order in
linear_cross_entropy_fp32_amd/csrc/tile_engine.h), restated step for step:
for every window size the plan picks (T = 1, 2, 4 or 8 token tiles x 64/T
vocabulary groups) and both inner orders, workgroup ids map one to one onto
the token-tile x group grid.  A map that missed or repeated a cell would
leave logits unreduced or make a forward workgroup write its partial states
past the split count."""
import pytest


def grouped_order(i, n_tt, n_grp, T, tt_fastest):
    G = 64 // T
    b, r = divmod(i, n_tt * G)
    gh = min(G, n_grp - b * G)
    tb, j = divmod(r, T * gh)
    tw = min(T, n_tt - tb * T)
    if tt_fastest:
        return tb * T + j % tw, b * G + j // tw
    return tb * T + j // gh, b * G + j % gh


@pytest.mark.parametrize("T", [1, 2, 4, 8])
@pytest.mark.parametrize("tt_fastest", [False, True])
def test_window_order_is_a_bijection(T, tt_fastest):
    shapes = [(a, b) for a in (1, 2, 3, 7, 8, 9, 17, 64) for b in (1, 5, 31, 32, 33, 63, 64, 65, 250)]
    shapes += [(8, 256), (32, 63), (64, 32), (64, 63), (3, 71)]
    for n_tt, n_grp in shapes:
        cells = [grouped_order(i, n_tt, n_grp, T, tt_fastest) for i in range(n_tt * n_grp)]
        assert all(0 <= t < n_tt and 0 <= g < n_grp for t, g in cells), (n_tt, n_grp)
        assert len(set(cells)) == n_tt * n_grp, (n_tt, n_grp)
