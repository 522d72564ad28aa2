"""Pins of the oracle's layout and golden reshard against facts fixed outside it.

Each test compares the oracle with something it does not compute itself: the
pages' worked 8x8 example (hand-written fixture), torch.chunk / torch.cat
(PyTorch's own definition of an uneven Shard and of an all-gather), the
per-element brute force, and the identity / round-trip invariants that the
pages' same-checkpoint verification relies on (zero changed parameters after
a refit of the same weights).
"""

import os

import numpy as np
import pytest
import torch

from oracle import brute, golden, layout
from rl_weight_refit_amd import synth

import helpers

HERE = os.path.dirname(os.path.abspath(__file__))


def read_worked_fixture():
    dst, owners, cur = {}, None, None
    with open(os.path.join(HERE, "golden", "worked_8x8.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    i = 0
    while i < len(lines):
        if lines[i].startswith("dst"):
            k = int(lines[i].split()[1])
            dst[k] = np.array([[int(x) for x in lines[i + 1 + r].split()] for r in range(8)])
            i += 9
        elif lines[i] == "owners":
            owners = [int(x) for x in lines[i + 1].split()]
            i += 2
        else:
            raise ValueError(lines[i])
    return dst, owners


def test_worked_example_golden():
    wl = synth.worked_example()
    t = wl["tensors"][0]
    G, _, _, per_tensor = helpers.golden_workload(wl)
    want, _ = read_worked_fixture()
    for k in range(4):
        got = per_tensor[0][k]["buf"].view(np.uint32).reshape(8, 2)
        np.testing.assert_array_equal(got, want[k].astype(np.uint32))


def test_worked_example_ownership():
    """Each destination is assembled from one 4x2 region of each source."""
    wl = synth.worked_example()
    t = wl["tensors"][0]
    src = helpers.src_desc_for(t)
    dst = helpers.odesc(t, "dst")
    _, owners = read_worked_fixture()
    for k in range(4):
        for i in range(8):
            for j in range(2):
                s, local = golden.source_location(src, [i, 2 * k + j])
                assert s == owners[i]
                assert local == [i - 4 * s, 2 * k + j]
    boxes = layout.slot_boxes(src)
    assert boxes == [([0, 0], [4, 8]), ([4, 0], [4, 8])]
    assert layout.slot_boxes(dst) == [([0, 2 * k], [8, 2]) for k in range(4)]


@pytest.mark.parametrize("parts", range(1, 9))
def test_chunk_matches_torch_chunk(parts):
    for n in range(0, 41):
        x = torch.arange(n)
        pieces = torch.chunk(x, parts) if n > 0 else []
        want = [(int(p[0]), len(p)) for p in pieces]
        want += [(n, 0)] * (parts - len(want))
        got = [layout.chunk(n, parts, i) for i in range(parts)]
        assert [g[1] for g in got] == [w[1] for w in want], (n, parts)
        for g, w in zip(got, want):
            if w[1]:
                assert g[0] == w[0]


def test_chunk_examples():
    """Uneven splits quoted for the uneven layouts."""
    sizes = lambda n, m: [layout.chunk(n, m, i)[1] for i in range(m)]
    assert sizes(3000, 7) == [429] * 6 + [426]
    assert sizes(1000, 3) == [334, 334, 332]
    assert sizes(513, 7) == [74] * 6 + [69]
    assert sizes(257, 4) == [65, 65, 65, 62]
    assert sizes(5, 4) == [2, 2, 1, 0]


def test_nested_shard_matches_nested_torch_chunk():
    """Two mesh dims sharding one tensor dim = chunk of a chunk (lower mesh dim outer)."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(0, 30))
        mi, mj = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        G = torch.arange(n)
        for ci in range(mi):
            outer = torch.chunk(G, mi) if n else []
            piece = outer[ci] if ci < len(outer) else G[:0]
            inner = torch.chunk(piece, mj) if len(piece) else []
            for cj in range(mj):
                want = inner[cj] if cj < len(inner) else piece[:0]
                off, ln = layout.shard_box([n], [mi, mj], [0, 0], (ci, cj))
                assert ln[0] == len(want)
                if len(want):
                    assert off[0] == int(want[0])


def test_nested_even_equals_flat():
    for n, mi, mj in [(24, 2, 3), (48, 4, 2), (16, 2, 2)]:
        for ci in range(mi):
            for cj in range(mj):
                a = layout.shard_box([n, 5], [mi, mj], [0, 0], (ci, cj))
                b = layout.shard_box([n, 5], [mi * mj], [0], (ci * mj + cj,))
                assert a == b


def _local_from_image(entry, esize, lengths):
    return golden.view_array(entry["buf"], esize, entry.get("view"), lengths).copy()


@pytest.mark.parametrize("seed", range(200))
def test_golden_matches_brute_force_tiny(seed):
    wl = synth.tiny_case(seed)
    t = wl["tensors"][0]
    G, _, _, per_tensor = helpers.golden_workload(wl)
    G = G[0]
    src_locals = helpers.local_arrays(t, G, "src")
    want = brute.reshard_local(helpers.src_desc_for(t), helpers.odesc(t, "dst"), src_locals)
    dboxes = layout.slot_boxes(helpers.odesc(t, "dst"))
    for k, box in enumerate(dboxes):
        got = _local_from_image(per_tensor[0][k], 4, box[1])
        np.testing.assert_array_equal(got, want[k])


@pytest.mark.parametrize("seed", range(0, 200, 17))
def test_golden_narrow_dtypes_tiny(seed):
    """Same tiny layouts at 1- and 2-byte element granularity."""
    for dt in ("u8", "bf16"):
        wl = synth.tiny_case(seed, dtype=dt)
        t = wl["tensors"][0]
        G, _, _, per_tensor = helpers.golden_workload(wl)
        G = G[0]
        want = brute.reshard_local(helpers.src_desc_for(t), helpers.odesc(t, "dst"),
                                   helpers.local_arrays(t, G, "src"))
        es = synth.ELEM_BYTES[dt]
        for k, box in enumerate(layout.slot_boxes(helpers.odesc(t, "dst"))):
            np.testing.assert_array_equal(_local_from_image(per_tensor[0][k], es, box[1]),
                                          want[k])


def test_replicate_to_shard_is_torch_chunk():
    G = torch.arange(7 * 11, dtype=torch.int32).reshape(7, 11)
    for d in (0, 1):
        for m in (1, 2, 3, 4, 5):
            src = {"shape": [7, 11], "dtype": "i32", "mesh": [3], "placements": [-1]}
            dst = {"shape": [7, 11], "dtype": "i32", "mesh": [m], "placements": [d]}
            sb = [{"buf": G.numpy().view(np.uint8).reshape(-1).copy(), "view": None}] * 3
            boxes = layout.slot_boxes(dst)
            db = [{"buf": np.zeros(layout.box_volume(b) * 4, np.uint8), "view": None}
                  for b in boxes]
            golden.reshard(src, dst, sb, db)
            pieces = torch.chunk(G, m, d)
            for k in range(m):
                want = pieces[k] if k < len(pieces) else G.narrow(d, 0, 0)
                got = db[k]["buf"].view(np.int32)
                np.testing.assert_array_equal(got, want.contiguous().numpy().reshape(-1))


def test_shard_to_replicate_is_torch_cat():
    G = torch.arange(9 * 6, dtype=torch.int32).reshape(9, 6)
    for d in (0, 1):
        m = 4
        pieces = list(torch.chunk(G, m, d))
        while len(pieces) < m:
            pieces.append(G.narrow(d, 0, 0))
        src = {"shape": [9, 6], "dtype": "i32", "mesh": [m], "placements": [d]}
        dst = {"shape": [9, 6], "dtype": "i32", "mesh": [2], "placements": [-1]}
        sb = [{"buf": p.contiguous().numpy().view(np.uint8).reshape(-1).copy(), "view": None}
              for p in pieces]
        db = [{"buf": np.zeros(9 * 6 * 4, np.uint8), "view": None} for _ in range(2)]
        golden.reshard(src, dst, sb, db)
        want = torch.cat(pieces, d).numpy().reshape(-1)
        for k in range(2):
            np.testing.assert_array_equal(db[k]["buf"].view(np.int32), want)


def _roundtrip(seed):
    wl = synth.uneven_case(seed, shapes=[[100, 300], [7, 51, 25]])
    t = wl["tensors"][0]
    G = synth.host_values(t)
    src = helpers.source_buffers(t, G)
    fwd_dst = helpers.odesc(t, "dst")
    _, per = helpers.alloc_destinations(wl)
    golden.reshard(helpers.src_desc_for(t), fwd_dst, src, per[0])
    back = synth.reverse(wl)
    tb = back["tensors"][0]
    _, per_b = helpers.alloc_destinations(back, poison=0x3C)
    golden.reshard(helpers.src_desc_for(tb), helpers.odesc(tb, "dst"), per[0], per_b[0])
    for a, b in zip(src, per_b[0]):
        np.testing.assert_array_equal(a["buf"], b["buf"])


@pytest.mark.parametrize("seed", range(0, 500, 5))
def test_round_trip_identity(seed):
    _roundtrip(seed)


@pytest.mark.parametrize("seed", range(0, 40, 3))
def test_identity_layout(seed):
    wl = synth.uneven_case(seed, shapes=[[40, 30]])
    t = wl["tensors"][0]
    t["dst"] = t["src"]
    G = synth.host_values(t)
    src = helpers.source_buffers(t, G)
    _, per = helpers.alloc_destinations(wl)
    golden.reshard(helpers.src_desc_for(t), helpers.odesc(t, "dst"), src, per[0])
    for a, b in zip(src, per[0]):
        np.testing.assert_array_equal(a["buf"], b["buf"])


def test_fused_view_is_cat_of_gate_and_up():
    """A fused gate/up destination equals cat([gate_k, up_k]) along the
    intermediate dim (gate first)."""
    wl = synth.dense_ffn(hidden=24, inter=40, src_tp=4, dst_tp=2, dst_dp=2)
    G, _, named, per = helpers.golden_workload(wl)
    gate, up = G[0], G[1]
    for k in range(4):
        tp = k // 2
        want = np.concatenate([np.array_split(gate, 2, 0)[tp], np.array_split(up, 2, 0)[tp]], 0)
        got = named["w13/%d" % k].view(np.uint16).reshape(40, 24)
        np.testing.assert_array_equal(got, want)


def test_poison_outside_views_untouched():
    wl = synth.moe_experts(6, 16, 10, 3, 2, 3, seed=3)
    _, _, named, per = helpers.golden_workload(wl, poison=0x5A)
    # w13 capacity rows: 2*ceil(10/3)=8 per expert, valid gate/up rows per slot 4,4,2
    for k in range(6):
        tp = k % 3
        ip_valid = [4, 4, 2][tp]
        img = named["w13/%d" % k].view(np.uint16).reshape(3, 8, 16)
        assert (img[:, ip_valid:4, :] == 0x5A5A).all()
        assert (img[:, 4 + ip_valid:, :] == 0x5A5A).all()
        assert not (img[:, :ip_valid, :] == 0x5A5A).any()


def test_replica_disagreement_detected():
    src = {"shape": [4], "dtype": "i32", "mesh": [2], "placements": [-1]}
    dst = {"shape": [4], "dtype": "i32", "mesh": [1], "placements": [-1]}
    a = np.arange(4, dtype=np.int32)
    b = a.copy()
    b[2] = 99
    with pytest.raises(AssertionError):
        golden.reshard(src, dst, [{"buf": a.view(np.uint8)}, {"buf": b.view(np.uint8)}],
                       [{"buf": np.zeros(16, np.uint8)}])


def test_parts_equal_stacked_buffer():
    """A shard given as one buffer per dim-0 index reads and writes like the
    same shard in one dense buffer."""
    rng = np.random.default_rng(3)
    src = {"shape": [6, 5, 4], "dtype": "i32", "mesh": [3], "placements": [0]}
    dst = {"shape": [6, 5, 4], "dtype": "i32", "mesh": [2, 2], "placements": [0, 2]}
    G = rng.integers(0, 1 << 30, size=(6, 5, 4)).astype(np.uint32)
    stacked = [{"buf": G[2 * s:2 * s + 2].copy().view(np.uint8).reshape(-1)} for s in range(3)]
    parts = [{"parts": [G[2 * s + i].copy().view(np.uint8).reshape(-1) for i in range(2)]}
             for s in range(3)]
    outs = []
    for sb in (stacked, parts):
        db = [{"parts": [np.zeros(5 * 2 * 4, np.uint8) for _ in range(3)]} for _ in range(4)]
        golden.reshard(src, dst, sb, db)
        outs.append([np.concatenate(d["parts"]) for d in db])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    # destination k = (e, t): experts 3e..3e+2, last-dim half t
    for k in range(4):
        e, t = divmod(k, 2)
        want = G[3 * e:3 * e + 3, :, 2 * t:2 * t + 2]
        np.testing.assert_array_equal(outs[0][k].view(np.uint32).reshape(3, 5, 2), want)


def read_grid_fixture():
    """The hand-written permuted rank grid (tests/golden/permuted_grid_2x2.txt)."""
    with open(os.path.join(HERE, "golden", "permuted_grid_2x2.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    head = {l[0]: [int(x) for x in l[1:]] for l in lines[:4]}
    slots = {}
    i = 4
    while i < len(lines):
        l = lines[i]
        k = int(l[1])
        off = [int(l[3]), int(l[4])]
        ln = [int(l[6]), int(l[7])]
        block = np.array([[int(x) for x in lines[i + 1 + r]] for r in range(ln[0])])
        slots[k] = (off, ln, block)
        i += 1 + ln[0]
    return head, slots


def grid_workload(as_source=False):
    head, _ = read_grid_fixture()
    grid = synth.side(head["mesh"], head["placements"], slot_of_coord=head["grid"])
    whole = synth.side([1], [-1])
    t = {"name": "g", "shape": head["shape"], "dtype": "i32",
         "src": grid if as_source else whole, "dst": whole if as_source else grid,
         "values": {"kind": "index"}}
    return {"name": "permuted_grid_%s" % ("src" if as_source else "dst"), "buffers": {},
            "tensors": [t]}


def test_permuted_rank_grid_boxes():
    """Slot s of a layout whose mesh tensor holds rank s at coordinate c owns
    the box of coordinate c (the fixture fixes the direction of the grid)."""
    head, slots = read_grid_fixture()
    desc = {"shape": head["shape"], "mesh": head["mesh"], "placements": head["placements"],
            "slot_of_coord": head["grid"]}
    boxes = layout.slot_boxes(desc)
    for k, (off, ln, _) in slots.items():
        assert boxes[k] == (off, ln), k


def test_permuted_rank_grid_golden():
    """Replicate -> the permuted grid: each slot's buffer holds its block."""
    _, slots = read_grid_fixture()
    wl = grid_workload()
    G, _, _, per = helpers.golden_workload(wl)
    for k, (_, ln, block) in slots.items():
        got = per[0][k]["buf"].view(np.uint32).reshape(ln)
        np.testing.assert_array_equal(got, block.astype(np.uint32))
    # and back: the permuted grid as the source reassembles the index tensor
    wl = grid_workload(as_source=True)
    G, _, _, per = helpers.golden_workload(wl)
    want = np.arange(24, dtype=np.uint32)
    np.testing.assert_array_equal(per[0][0]["buf"].view(np.uint32), want)
