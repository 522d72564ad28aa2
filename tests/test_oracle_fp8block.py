"""Pins of the oracle's blockwise-FP8 helpers, and the planner's
block-alignment check against them.

* aligned() (box arithmetic) agrees with aligned_brute() (element by
  element) on random tiny layouts;
* dequantize() agrees with torch's float8_e4m3fn decoding times the
  block-expanded scales;
* after a reshard of weights and scales, every destination shard dequantizes
  to the matching slice of the dequantized global tensor;
* the library accepts exactly the layouts the oracle calls aligned.
"""

import numpy as np
import pytest
import torch

from oracle import fp8block, golden, layout
from rl_weight_refit_amd import binding, synth

import helpers
import lib_helpers as lh

MESHES = [[1], [2], [3], [4], [2, 2], [2, 3], [3, 2]]


def random_case(rng):
    ndim = int(rng.integers(1, 4))
    shape = [int(rng.integers(1, 20)) for _ in range(ndim)]
    block = [int(rng.integers(1, 6)) for _ in range(ndim)]
    mesh = MESHES[int(rng.integers(len(MESHES)))]
    pl = [int(rng.integers(-1, ndim)) for _ in mesh]
    w = {"shape": shape, "mesh": mesh, "placements": pl}
    s = {"shape": [-(-n // b) for n, b in zip(shape, block)], "mesh": mesh, "placements": pl}
    return w, s, block


@pytest.mark.parametrize("seed", range(300))
def test_aligned_matches_brute_force(seed):
    w, s, block = random_case(np.random.default_rng(seed))
    assert fp8block.aligned(w, s, block) == fp8block.aligned_brute(w, s, block)


def test_aligned_examples():
    w = {"shape": [2048, 7168], "mesh": [8], "placements": [0]}
    s = {"shape": [16, 56], "mesh": [8], "placements": [0]}
    assert fp8block.aligned(w, s, [128, 128])            # 256-row shards: 2 blocks each
    w = {"shape": [384, 256], "mesh": [4], "placements": [0]}
    s = {"shape": [3, 2], "mesh": [4], "placements": [0]}
    assert not fp8block.aligned(w, s, [128, 128])        # 96-row shards split blocks


def test_dequantize_matches_torch():
    rng = np.random.default_rng(1)
    wb = rng.integers(0, 256, size=(3, 300, 200), dtype=np.uint8)
    wb[(wb & 0x7F) == 0x7F] = 0
    sc = rng.uniform(0.01, 2.0, size=(3, 3, 2)).astype(np.float32)
    got = fp8block.dequantize(wb, sc, [1, 128, 128])
    t = torch.from_numpy(wb).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(sc).to(torch.float64)
    s = s.repeat_interleave(128, dim=1)[:, :300].repeat_interleave(128, dim=2)[:, :, :200]
    np.testing.assert_array_equal(got, (t * s).numpy())


def test_destination_shards_dequantize_to_global_slices():
    wl = synth.fp8_moe_experts(8, 256, 512, 4, 2, 2, seed=3)
    G, _, named, per = helpers.golden_workload(wl)
    deq = [fp8block.dequantize(G[i], G[i + 3].view(np.float32), [1, 128, 128]) for i in range(3)]
    for i in range(3):
        t, ts = wl["tensors"][i], wl["tensors"][i + 3]
        wboxes = layout.slot_boxes(helpers.odesc(t, "dst"))
        sboxes = layout.slot_boxes(helpers.odesc(ts, "dst"))
        for k, (wbox, sbox) in enumerate(zip(wboxes, sboxes)):
            wloc = golden.read_shard(per[i][k], 1, wbox[1])
            sloc = golden.read_shard(per[i + 3][k], 4, sbox[1]).view(np.float32)
            got = fp8block.dequantize(wloc, sloc, [1, 128, 128])
            np.testing.assert_array_equal(got, deq[i][golden.box_slices(wbox)])


@pytest.mark.parametrize("seed", range(200))
def test_library_accepts_exactly_the_aligned_layouts(seed):
    rng = np.random.default_rng(1000 + seed)
    w, s, block = random_case(rng)
    dmesh = MESHES[int(rng.integers(len(MESHES)))]
    dpl = [int(rng.integers(-1, len(w["shape"]))) for _ in dmesh]
    wd = dict(w, mesh=dmesh, placements=dpl)
    sd = dict(s, mesh=dmesh, placements=dpl)
    want = fp8block.aligned(w, s, block) and fp8block.aligned(wd, sd, block)
    mk = lambda d, dt: dict(d, dtype=dt)
    srcs = [mk(w, "u8"), dict(mk(s, "f32"), scale_of=0, scale_block=block)]
    dsts = [mk(wd, "u8"), mk(sd, "f32")]
    try:
        binding.reshard_plan(srcs, dsts)
        got = True
    except binding.ReshardError as e:
        assert e.status == 3, str(e)
        got = False
    assert got == want


def test_scale_tensor_must_match_ceil_shape():
    w = {"shape": [256, 256], "dtype": "u8", "mesh": [2], "placements": [0]}
    s = {"shape": [3, 2], "dtype": "f32", "mesh": [2], "placements": [0], "scale_of": 0,
         "scale_block": [128, 128]}
    with pytest.raises(binding.ReshardError) as e:
        binding.reshard_plan([w, s], [dict(w), dict(s, scale_of=None)])
    assert e.value.status == 2


def test_interpreted_fp8_layer():
    from test_planner import run_interpreted
    for kw in ({}, {"src_split": True}):
        run_interpreted(synth.fp8_moe_experts(8, 256, 512, 4, 2, 2, seed=3, **kw))
