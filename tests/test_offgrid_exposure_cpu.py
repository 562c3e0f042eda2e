"""Rows off the 16-byte grid: which shapes put the row's last (window) vector
in another wave than the vector before it.

Off the grid, a row's last vector, when only partly inside the row, is read
and written as a window over the row's last 16 bytes.  Its leading columns
are also the previous vector's.  When the two vectors sit in different waves
of the row, nothing but the row barrier orders one wave's stores against the
other wave's loads of those columns.  An output that is the very same buffer
as an input (the ABI allows it) is then safe only because every aligned-away
store is made after every load of the row has returned: the kernels store
residual_out (forward, LayerNorm) and dh (residual backward) after the row's
reductions, and the residual backward waits for its dres loads before the
row barrier.

This test needs no GPU: it asks the library for the tile each call takes
(rmsnorm_tuning_tile) and lists the exposed shapes, H <= 8192 in every
format.  The in-place GPU tests run the listed worked case, bf16 H = 4097.

A backward whose row streams share one offset within their 16-byte chunks
sets its vectors on memory's 16-byte grid instead (the frame): the row's
first vector then sits at the row start and overlaps the next chunk (lanes 0
and 1, always one wave), and its last is the same window over the row's last
16 bytes, after up to one more vector than at the row's offset.  The same row
barrier orders those overlaps.

Backward rows longer than one tile take two passes; there the window is read
in pass 1 only, and in pass 2 (dx stores, workspace updates) the lane of the
last partial vector takes its own columns one by one, so no shape of that
form is exposed.
"""

from __future__ import annotations

import os

import pytest

import transformer_normalization_amd as tn
from transformer_normalization_amd import build as hipbuild

OPS = ("fwd", "fwd_residual", "adaln", "layernorm", "bwd", "bwd_residual")
ES = {"f32": 4, "f16": 2, "bf16": 2}


def _lib():
    if not os.path.exists(tn.LIB_PATH):
        hipbuild.build()
    return tn.load_library()


def _exposed(H: int, vec: int, wpr: int) -> bool:
    """Whether the window vector and the vector before it are in different
    waves: thread t of a row group of 64*wpr threads holds vectors t, t +
    64*wpr, ...; its wave is t // 64."""
    nvec = -(-H // vec)
    if H % vec == 0 or nvec < 2:
        return False  # no partial vector, or no neighbour
    row_threads = 64 * wpr
    wave = lambda v: (v % row_threads) // 64
    return wave(nvec - 1) != wave(nvec - 2)


def exposure_table(hmax: int = 8192):
    _lib()
    rows = []
    for dt, es in ES.items():
        vec = 16 // es
        for op in OPS:
            for H in range(2, hmax + 1):
                if H % vec == 0:
                    continue
                t = tn.tile(op, H, dt, off_grid=True)
                if t["mis"] and _exposed(H, t["vec"], t["wpr"]):
                    rows.append((op, dt, H, t["vpt"], t["wpr"]))
    return rows


def test_exposure_rule_matches_mapping():
    # the closed form: exposed iff wpr > 1 and the window vector is lane 0 of
    # a wave, i.e. (nvec - 1) % 64 == 0
    for vec in (4, 8):
        for wpr in (1, 2, 3, 4, 8):
            for H in range(2, 4 * 64 * vec * wpr):
                nvec = -(-H // vec)
                want = H % vec != 0 and nvec >= 2 and wpr > 1 and (nvec - 1) % 64 == 0
                assert _exposed(H, vec, wpr) == want, (vec, wpr, H)


def test_worked_case_is_exposed():
    # bf16 H = 4097 fused residual: 513 vectors on a 2-wave row of 128
    # threads, 6 vectors per thread; vector 511 is thread 127 (wave 1) and
    # vector 512 (the window) thread 0 (wave 0)
    t = tn.tile("fwd_residual", 4097, "bf16", off_grid=True)
    assert t["mis"] and (t["vpt"], t["wpr"]) == (6, 2)
    assert _exposed(4097, 8, 2)


def test_exposure_table(capsys):
    rows = exposure_table()
    by_op = {}
    for op, dt, H, vpt, wpr in rows:
        by_op.setdefault((op, dt), []).append(H)
    with capsys.disabled():
        print("\noff-grid shapes (H <= 8192) whose window vector is in another wave than its neighbour:")
        for (op, dt), hs in sorted(by_op.items()):
            print(f"  {op:13s} {dt:5s} {len(hs):3d} H: {hs}")
    # the exposure only arises for rows of several waves whose last vector
    # starts a wave; every row whose length leaves H % vec != 0 and nvec - 1
    # a multiple of 64 and that takes a multi-wave tile is listed
    assert ("fwd_residual", "bf16", 4097, 6, 2) in rows
    for op, dt, H, vpt, wpr in rows:
        vec = 16 // ES[dt]
        assert wpr > 1 and (-(-H // vec) - 1) % 64 == 0


@pytest.mark.parametrize("args", [(-1, 64, 2, 0), (7, 64, 2, 0), (0, 64, 2, 3), (0, 64, 2, -1), (0, 0, 2, 0),
                                  (0, 64, 9, 0)])
def test_tile_query_rejects_bad_arguments(args):
    import ctypes
    lib = _lib()
    out = (ctypes.c_int32 * 6)()
    op, H, dt, layout = args
    assert lib.rmsnorm_tuning_tile(op, H, dt, layout, out) != 0


def test_tile_query_aligned_rows():
    # the headline forward: bf16 rows of 4096 on the grid take 2 vectors per
    # thread over 4 waves, one row per workgroup
    t = tn.tile("fwd", 4096, "bf16", off_grid=False)
    assert (t["vec"], t["vpt"], t["wpr"], t["mis"], t["multi_pass"]) == (8, 2, 4, False, False)
    t = tn.tile("bwd", 6144, "bf16", off_grid=False)
    assert t["vec"] == 8 and not t["mis"] and not t["multi_pass"]
    assert 64 * t["wpr"] * t["vpt"] >= 768


@pytest.mark.parametrize("op,dt,H", [("bwd", "bf16", 16385), ("bwd", "f32", 16385), ("bwd", "bf16", 70001),
                                     ("bwd_residual", "bf16", 16385), ("bwd_residual", "f16", 20001),
                                     ("bwd_residual", "f32", 8193), ("fwd", "bf16", 70001),
                                     ("fwd_residual", "bf16", 32769), ("fwd_residual", "f32", 30001),
                                     ("adaln", "bf16", 32769), ("layernorm", "bf16", 24577),
                                     ("layernorm", "f32", 70001)])
def test_long_rows_off_the_grid_take_vectors(op, dt, H):
    # rows longer than one tile: passes over the row in 16-byte vectors at
    # each row's byte offset, not single elements
    t = tn.tile(op, H, dt, off_grid=True)
    assert t["multi_pass"] and t["mis"] and t["vec"] == 16 // ES[dt]


# the forward family's longest rows held in registers: 16-bit rows whose
# parameters are 16-bit too take twice the elements per thread of float32 rows
# at the same workgroup size
@pytest.mark.parametrize("op,limit16,limit32", [("fwd", 65536, 32768), ("fwd_residual", 32768, 16384),
                                                ("adaln", 32768, 16384), ("layernorm", 24576, 16384)])
def test_longest_one_pass_forward_rows(op, limit16, limit32):
    for dt, limit in (("bf16", limit16), ("f16", limit16), ("f32", limit32)):
        assert not tn.tile(op, limit, dt, off_grid=False)["multi_pass"], (dt, limit)
        assert not tn.tile(op, limit - 1, dt, off_grid=True)["multi_pass"], (dt, limit - 1)
        assert tn.tile(op, limit + 16 // ES[dt], dt, off_grid=False)["multi_pass"], (dt, limit)
        assert tn.tile(op, limit + 1, dt, off_grid=True)["multi_pass"], (dt, limit + 1)


@pytest.mark.parametrize("op,dt,H", [("bwd", "bf16", 16383), ("bwd", "f32", 16383), ("bwd_residual", "bf16", 16383),
                                     ("bwd_residual", "f16", 12289), ("bwd_residual", "f32", 8191)])
def test_longest_one_pass_backward_rows_off_the_grid(op, dt, H):
    t = tn.tile(op, H, dt, off_grid=True)
    assert t["mis"] and not t["multi_pass"]


@pytest.mark.parametrize("op", ["fwd", "fwd_residual", "adaln", "layernorm"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_two_waves_per_row_for_16bit_rows_of_193_to_768_vectors(op, dt):
    # from 193 vectors (H = 1537) to 768 (H = 6144) a 16-bit row off the grid
    # takes two waves, with the fewest idle slots over 1-6 vectors per thread
    for H, vpt in ((1537, 2), (2049, 3), (3073, 4), (4097, 6), (6143, 6), (6144, 6)):
        t = tn.tile(op, H, dt, off_grid=True)
        assert t["mis"] and (t["vpt"], t["wpr"], t["rpw"]) == (vpt, 2, 2), (H, t)
    # 192 vectors and fewer, and 769 and more, keep the other rules
    assert tn.tile(op, 1535, dt, off_grid=True)["wpr"] == 1
    assert tn.tile(op, 6145, dt, off_grid=True)["wpr"] > 2


def test_float32_rows_keep_their_rules():
    assert tn.tile("fwd", 2049, "f32", off_grid=True)["wpr"] == 3
    assert tn.tile("fwd", 4097, "f32", off_grid=True)["wpr"] == 3


def test_adaln_keeps_two_workgroups_per_cu_on_its_large_tiles():
    # AdaLN tiles of more than 16 elements per thread hold a CU at four waves
    # per SIMD, so past 8 waves a workgroup would run alone on its CU: rows
    # that a tile of at most 8 waves covers take it, where the fused residual
    # takes the tile with the preferred element count
    for H, tile in ((12296, (4, 7)), (16384, (4, 8))):
        t = tn.tile("adaln", H, "bf16", off_grid=False)
        assert (t["vpt"], t["wpr"]) == tile, (H, t)
    assert (lambda t: (t["vpt"], t["wpr"]))(tn.tile("fwd_residual", 16384, "bf16", off_grid=False)) == (3, 11)
    # rows no 8-wave tile covers stay resident on the best tile over the cap
    t = tn.tile("adaln", 24576, "bf16", off_grid=False)
    assert not t["multi_pass"] and t["wpr"] > 8
    # 16-bit rows take the 8-wave cap at 2 vectors per thread too (3 x 7
    # rather than 2 x 10 at H = 10240); float32 rows of 16 elements per
    # thread keep the 12-wave cap
    for H, tile in ((10240, (3, 7)), (12288, (3, 8))):
        t = tn.tile("adaln", H, "bf16", off_grid=False)
        assert (t["vpt"], t["wpr"]) == tile, (H, t)
    t = tn.tile("adaln", 12288, "f32", off_grid=False)
    assert (t["vpt"], t["wpr"]) == (4, 12), t


@pytest.mark.parametrize("op", ["bwd", "bwd_residual"])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_frame_tile_covers_the_chunks_a_row_touches(op, dt):
    # a row of H elements at offset a (a multiple of the element size, below
    # 16) within its first 16-byte chunk touches ceil((a + H*es) / 16)
    # chunks, at most ceil((H*es + 16 - es) / 16); the frame's tile holds that
    # many vectors, in one pass, wherever the row-offset tile is one pass and
    # the rule for the extra vector stays one pass
    es = ES[dt]
    _lib()
    seen = 0
    for H in list(range(16 // es, 2600)) + [4095, 4097, 6143, 8191, 12287, 12289, 16383]:
        off = tn.tile(op, H, dt, off_grid=True)
        fr = tn.tile(op, H, dt, off_grid=True, shared_offset=True)
        chunks = -(-(H * es + 16 - es) // 16)
        if fr["frame"]:
            seen += 1
            assert off["mis"] and not off["multi_pass"] and not fr["multi_pass"], (H, off, fr)
            assert fr["vec"] == 16 // es and 64 * fr["wpr"] * fr["vpt"] >= chunks, (H, fr)
        else:
            assert off["multi_pass"] or not off["mis"] or \
                tn.tile(op, H + (16 - es) // es, dt, off_grid=True)["multi_pass"], (H, off, fr)
    assert seen > 2000
    # on the grid (layout 0) there is no frame
    assert not tn.tile(op, 4096, dt, off_grid=False, shared_offset=True)["frame"]


def test_frame_worked_case():
    # bf16 H = 4097: 8194 bytes touch 513 chunks at any even offset, the same
    # 9-wave one-vector tile as at the row offset
    off = tn.tile("bwd", 4097, "bf16", off_grid=True)
    fr = tn.tile("bwd", 4097, "bf16", off_grid=True, shared_offset=True)
    assert fr["frame"] and (fr["vpt"], fr["wpr"]) == (off["vpt"], off["wpr"]) == (1, 9)
    # bf16 H = 4095: 8190 bytes touch 513 chunks at offsets 4 .. 14 (512
    # vectors at the row offset)
    assert tn.tile("bwd", 4095, "bf16", off_grid=True, shared_offset=True)["wpr"] == 9
    assert tn.tile("bwd", 4095, "bf16", off_grid=True)["wpr"] == 8


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_two_waves_per_row_for_16bit_rows_on_the_grid(dt):
    # 16-bit rows on the grid of 193 to 768 vectors take two waves per row
    # for LayerNorm and AdaLN always, for the plain forward unless the
    # general rule's tile is a whole tile of 2 or more vectors per thread
    # (3072, 4096, 5120, 6144 keep it); the fused residual keeps its rule
    tile = lambda op, H: tuple(tn.tile(op, H, dt, off_grid=False)[k] for k in ("vpt", "wpr", "rpw"))
    for H, vpt in ((2056, 3), (2560, 3), (3072, 3), (3584, 4), (4096, 4), (4104, 6), (5120, 6), (6144, 6)):
        assert tile("layernorm", H) == (vpt, 2, 2), H
        assert tile("adaln", H) == (vpt, 2, 2), H
    for H, want in ((2056, (3, 2, 2)), (2560, (3, 2, 2)), (3584, (4, 2, 2)), (4104, (6, 2, 2)),
                    (3072, (2, 3, 2)), (4096, (2, 4, 1)), (5120, (2, 5, 1)), (6144, (2, 6, 1))):
        assert tile("fwd", H) == want, H
    assert tile("fwd_residual", 2056) == (1, 5, 1)
    # outside the range, and float32 rows, the general rule
    assert tile("layernorm", 12288)[1] != 2
    assert tn.tile("layernorm", 4096, "f32", off_grid=False)["wpr"] != 2


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_layernorm_two_wave_tile_of_up_to_eight_vectors(dt):
    # plain LayerNorm of 16-bit rows on the grid of 769 to 1024 vectors:
    # two waves of 8 vectors per thread, two rows per workgroup; the
    # LayerNorm fused with the residual add keeps the general rule
    tile = lambda op, H: tuple(tn.tile(op, H, dt, off_grid=False)[k] for k in ("vpt", "wpr", "rpw"))
    for H in (6152, 7168, 7176, 8192):
        assert tile("layernorm", H) == (8, 2, 2), H
    assert tile("layernorm", 6144) == (6, 2, 2)
    assert tile("layernorm_residual", 8192) == (2, 8, 1)
    assert tile("layernorm_residual", 4096) == tile("layernorm", 4096)
    assert tile("layernorm", 8200) != (8, 2, 2)
