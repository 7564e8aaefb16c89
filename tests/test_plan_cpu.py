"""The planner of the C library (flce_plan_info, no GPU needed), swept over
the validated extremes of N, H and V: every 32-bit buffer offset the kernels
form stays inside its range, and the workspace holds no (tokens x vocab)
buffer beyond one backward chunk.

Offsets the kernels form in 32 bits (the operand's descriptor base is the
tile's first row, so a tile adds at most its own rows):
  * dz stores of the recompute kernel: token row (up to 127 past a wave's
    base, phantom rows past N included) x 2 Vc bytes + the column offset;
  * K-major operand rows of a tile (up to 255 rows: 256 tokens, or the 128
    or 256 vocabulary rows of a logit tile): row x 2 ld, with ld = H
    (lm_head, hidden) or Vc (a dz chunk);
  * MN-major operands: K row x 2 ld bytes, K rows running up to the K bound
    plus one 32-deep slice (phantom rows read zero only if the offset does not
    wrap past 2^32): dz and hidden along the N tokens, the lm_head chunk along
    its Vc rows;
  * result stores: (row x H + column) x 4 bytes, rows up to 255 past the base.
"""
import itertools

import pytest

import linear_cross_entropy_fp32_amd as flce

U31, U32 = 1 << 31, 1 << 32

NS = [0, 1, 2, 3, 31, 100, 255, 256, 257, 2048, 8192, 16384, 65535, (1 << 20) - 1, (1 << 23) - 1]
HS = [8, 16, 24, 64, 640, 1024, 4096, 1 << 14, 1 << 20]
VS = [1, 2, 127, 128, 129, 32000, 151936, 262144, (1 << 20) + 3, 1 << 26, (1 << 30)]


def _valid_problems():
    for n, h, v in itertools.product(NS, HS, VS):
        for hd, wd, comp in ((0, 0, False), (1, 0, False), (0, 1, True), (1, 1, True)):
            p = flce.make_problem(n, h, v, hidden_dtype=hd, weight_dtype=wd, compact_valid=comp)
            if flce.flce_validate(p) == 0:
                yield n, h, v, p


def test_sweep_has_extremes():
    shapes = {(n, h, v) for n, h, v, _ in _valid_problems()}
    assert (1, 8, 1 << 26) in shapes            # tiny N with a huge vocabulary
    assert ((1 << 23) - 1, 8, 1) in shapes       # the largest N
    assert (1, 1 << 20, 1) in shapes             # the largest H
    assert len(shapes) > 200


@pytest.mark.parametrize("chunk", range(4))
def test_offsets_stay_in_32_bits(chunk):
    probs = list(_valid_problems())
    for n, h, v, p in probs[chunk::4]:
        pl = flce.flce_plan_info(p)
        vc = pl["chunk_rows"]
        label = (n, h, v, p.hidden_dtype, p.weight_dtype, p.compact_valid, vc)
        # 256-row dz tiles, except where one 256-row dz column would pass the
        # descriptor extent, or where a chunk holds fewer 256-row tiles than
        # the 256 CUs
        dt = pl["dz_tile_rows"]
        ntt = -(-n // 256)
        if n * 2 * 256 >= U31:
            assert dt == 128, label
        elif dt == 256:
            assert ntt * -(-min(vc, v) // 256) >= 256, label
        else:
            assert dt == 128 and ntt * -(-min(vc, v) // 256) < 256, label
        assert pl["fwd_tile_rows"] == (256 if h >= 1024 else 128), label
        assert pl["contract_tile_cols"] == (256 if h >= 1024 and h % 256 == 0 else 128), label
        assert vc % dt == 0 and vc >= dt, label
        assert pl["n_chunks"] == -(-v // vc), label
        width = min(vc, v)
        # dz stores: 128 token rows of a wave, 2 Vc bytes each
        assert 128 * 2 * vc + 2 * vc < U31, label
        # K-major rows of a 256-row tile: lm_head / hidden (ld H), dz (ld Vc)
        assert 256 * 2 * max(h, vc) < U31, label
        # MN-major K rows: real rows inside the descriptor, phantom rows of the
        # last slice do not wrap
        assert n * 2 * vc < U31 and (n + 32) * 2 * vc < U32, label
        assert n * 2 * h < U31 and (n + 32) * 2 * h < U32, label
        assert width * 2 * h < U31 and (width + 32) * 2 * h < U32, label
        # result stores of 256 x 128 tiles (grad_hidden slots, grad_weight rows)
        assert (256 * h + h) * 4 < U31, label
        # split-K slots cover the chunk
        assert pl["gh_rows_per_split"] % 32 == 0, label
        assert pl["gh_splits"] * pl["gh_rows_per_split"] >= width, label
        assert (pl["gh_splits"] - 1) * pl["gh_rows_per_split"] < width, label
        # forward splits cover the vocabulary tiles
        tiles = -(-v // pl["fwd_tile_rows"])
        assert pl["fwd_splits"] * pl["fwd_tiles_per_split"] >= tiles, label
        assert (pl["fwd_splits"] - 1) * pl["fwd_tiles_per_split"] < tiles, label


def test_chunk_cap_reached_by_tiny_batches():
    """N = 1, H = 8, V = 2^26: before the cap the chunk was 2^26 rows wide and
    token row 32 of a wave wrapped to byte 0 of the dz chunk."""
    pl = flce.flce_plan_info(flce.make_problem(1, 8, 1 << 26))
    assert pl["chunk_rows"] == 1 << 21
    assert pl["n_chunks"] == 32


@pytest.mark.parametrize("n,h,v,hd", [(256, 256, 32000, 0), (2048, 640, 262144, 0),
                                      (8192, 2048, 128256, 0), (16384, 1024, 151936, 0),
                                      (16384, 4096, 151936, 1)])
def test_workspace_holds_one_chunk_only(n, h, v, hd):
    """The workspace is the larger of the forward's (per-(split, token) states,
    block sums, the fp32 hidden split) and the backward's (one dz chunk,
    split-K slots, the split); its only (tokens x vocab) buffer is one chunk of
    at most 2^28 bytes, or N rows wide when N is large, and for every
    workload past the first that is at most a quarter of N x V x 2 bytes."""
    p = flce.make_problem(n, h, v, hidden_dtype=hd)
    pl = flce.flce_plan_info(p)
    assert pl["workspace_bytes"] == max(pl["fwd_workspace_bytes"], pl["bwd_workspace_bytes"])
    assert pl["workspace_bytes"] == flce.flce_workspace_bytes(p)
    chunk = pl["dz_chunk_bytes"]
    assert chunk == n * pl["chunk_rows"] * 2
    assert chunk <= max(1 << 28, n * (-(-n // 128) * 128) * 2)
    split = 2 * n * h * 2 if hd == 1 else 0
    slots = pl["gh_splits"] * n * h * 4 if pl["gh_splits"] > 1 else 0
    states = pl["fwd_splits"] * n * 24
    slack = 16 * 256 + (-(-n // 8)) * 32 + 4 * (1 << 22)
    assert pl["bwd_workspace_bytes"] <= split + chunk + slots + slack
    assert pl["fwd_workspace_bytes"] <= split + states + slack
    if v * n > 256 * 32000:
        assert chunk <= n * v * 2 // 4, (chunk, n * v * 2)


def test_plan_info_errors():
    import ctypes
    p = flce.make_problem(4, 12, 10)            # H % 8 != 0
    with pytest.raises(flce.FlceError):
        flce.flce_plan_info(p)
    lib = flce.lib()
    assert lib.flce_plan_info(ctypes.byref(flce.make_problem(4, 64, 10)), None, 3) == -1
    out = (ctypes.c_int64 * 2)()
    assert lib.flce_plan_info(ctypes.byref(flce.make_problem(4, 64, 10)), out, 2) == 2


def _golden_names():
    import glob
    import os
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    return sorted(os.path.basename(p)[len("fullsize_"):-len(".npz")]
                  for p in glob.glob(os.path.join(root, "fullsize_*.npz")))


@pytest.mark.parametrize("name", _golden_names())
def test_golden_sampling_matches_the_plan(name):
    """The stored full-size goldens sampled the chunks and split-K slots the
    library actually plans: the recorded chunk plan equals flce_plan_info's,
    every backward chunk holds at least two sampled grad_weight rows with both
    of its edge rows among them, every split-K slot edge has a sampled row on
    each side, and every 256-token tile has a sampled grad_hidden row."""
    import os

    import numpy as np

    from linear_cross_entropy_fp32_amd import synth
    w = synth.WORKLOADS[name]
    gold = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                f"fullsize_{name}.npz"), allow_pickle=False)
    if "chunk_rows" not in gold.files:
        pytest.skip("golden written before the chunk plan was recorded")
    p = flce.make_problem(w.n_tokens, w.hidden, w.vocab,
                          hidden_dtype=1 if w.hidden_dtype == "f32" else 0,
                          weight_dtype=1 if w.weight_dtype == "f32" else 0)
    pl = flce.flce_plan_info(p)
    vc, kps = pl["chunk_rows"], pl["gh_rows_per_split"]
    assert vc == int(gold["chunk_rows"]) and kps == int(gold["gh_rows_per_split"])
    vrows = set(int(x) for x in gold["vocab_rows"])
    for c0 in range(0, w.vocab, vc):
        c1 = min(w.vocab, c0 + vc)
        assert {c0, c1 - 1} <= vrows, (c0, c1)
        assert len([x for x in vrows if c0 <= x < c1]) >= 2
        for e in range(c0 + kps, c1, kps):
            assert {e - 1, e} <= vrows, e
    rows = set(int(x) for x in gold["rows"])
    for t0 in range(0, w.n_tokens, 256):
        assert any(t0 <= r < t0 + 256 for r in rows), t0
    for k in ("sketch_grad_hidden", "sketch_grad_weight", "sketch_grad_bias"):
        assert k in gold.files
