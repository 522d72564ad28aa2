"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by monkeypatching)
and checks that at least one pin then fails.  This is what makes the pins
evidence: a dropped term, a wrong rounding or an off-by-one would not pass.
"""

import numpy as np
import pytest

from oracle import golden, layout, mxfp8

import test_oracle_layout as tl
import test_oracle_mxfp8 as tm


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_floor_chunk_is_caught(monkeypatch):
    def floor_chunk(length, parts, index):
        size = length // parts
        start = min(index * size, length)
        return start, min((index + 1) * size, length) - start
    monkeypatch.setattr(layout, "chunk", floor_chunk)
    assert _fails(tl.test_chunk_matches_torch_chunk, 3)
    assert _fails(tl.test_chunk_examples)


def test_reversed_nesting_is_caught(monkeypatch):
    orig = layout.shard_box

    def reversed_nesting(shape, mesh, placements, coord):
        idx = list(range(len(mesh)))[::-1]
        return orig(shape, [mesh[i] for i in idx], [placements[i] for i in idx],
                    [coord[i] for i in idx])
    monkeypatch.setattr(layout, "shard_box", reversed_nesting)
    assert _fails(tl.test_nested_shard_matches_nested_torch_chunk)


def test_dropped_view_base_is_caught(monkeypatch):
    orig = golden.view_array

    def no_base(buf, esize, view, lengths, writeable=False):
        if view is not None:
            view = (0, view[1])
        return orig(buf, esize, view, lengths, writeable)
    monkeypatch.setattr(golden, "view_array", no_base)
    assert _fails(tl.test_fused_view_is_cat_of_gate_and_up)


def test_transposed_destination_is_caught(monkeypatch):
    orig = golden.reshard

    def transposed(src_desc, dst_desc, src_bufs, dst_bufs):
        d = dict(dst_desc)
        orig(src_desc, d, src_bufs, dst_bufs)
        for e in dst_bufs:
            a = e["buf"].view(np.uint32)
            if a.size == 16:
                a[:] = a.reshape(8, 2).T.reshape(-1)
    monkeypatch.setattr(golden, "reshard", transposed)
    assert _fails(tl.test_worked_example_golden)


def test_wrong_scale_offset_is_caught(monkeypatch):
    def minus7(amax):
        amax = np.asarray(amax, dtype=np.float64)
        out = np.full(amax.shape, -127, dtype=np.int64)
        nz = amax > 0
        out[nz] = np.clip(mxfp8.floor_log2(amax[nz]) - 7, -127, 127)
        return out
    monkeypatch.setattr(mxfp8, "shared_exponent", minus7)
    blk = tm.read_blocks()[0]
    assert _fails(tm.test_hand_computed_blocks, blk)
    assert _fails(tm.test_scale_rule_from_exponent_bits)


def test_round_half_away_is_caught(monkeypatch):
    monkeypatch.setattr(mxfp8.np, "rint", lambda x: np.floor(x + 0.5))
    assert _fails(tm.test_encode_exhaustive_vs_brute_force, -8)
    ties = [b for b in tm.read_blocks() if b["name"] == "ties"][0]
    assert _fails(tm.test_hand_computed_blocks, ties)


def test_lost_sign_of_zero_is_caught(monkeypatch):
    orig = mxfp8.e4m3_encode

    def unsigned_zero(q):
        c = orig(q)
        return np.where(c == 0x80, 0, c).astype(np.uint8)
    monkeypatch.setattr(mxfp8, "e4m3_encode", unsigned_zero)
    zeros = [b for b in tm.read_blocks() if b["name"] == "zeros"][0]
    assert _fails(tm.test_hand_computed_blocks, zeros)
    assert _fails(tm.test_encode_vs_torch_float8, 0)


def test_inverted_rank_grid_is_caught(monkeypatch):
    """Reading the grid the wrong way round (entry c as the coordinate of
    slot c, instead of the slot at coordinate c)."""
    def inverted(desc):
        coords = layout.mesh_coords(desc["mesh"])
        soc = desc.get("slot_of_coord")
        if soc is None:
            return coords
        return [coords[soc[s]] for s in range(len(coords))]
    monkeypatch.setattr(layout, "slot_coords", inverted)
    assert _fails(tl.test_permuted_rank_grid_boxes)
    assert _fails(tl.test_permuted_rank_grid_golden)
