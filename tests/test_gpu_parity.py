"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
byte for byte, on every workload family at sizes the oracle finishes in
seconds: the pages' worked example, 200 tiny random layouts, the 500 uneven
layouts with their A -> B -> A round trips, fused dense and MoE layers
(ragged variants included), the MXFP8 install, misaligned pointers, rank 4-6
layouts with padded views, and every kernel bucket forced on its own.  Destinations start poisoned, with guard
bytes after each buffer; sources must come back unchanged.
"""

import numpy as np
import pytest
import torch

from rl_weight_refit_amd import binding, synth

import gpu_helpers as gh
import helpers
import lib_helpers as lh

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield


@pytest.mark.parametrize("kw,bucket", [({}, "tiny"), ({"tiny_bytes": 0}, "thin"),
                                       ({"tiny_bytes": 0, "thin_bytes": 1}, "bulk")])
def test_worked_example(kw, bucket):
    """The 8x8 example through each kernel: the wave-prefix-sum tiny kernel,
    the LDS-staged thin kernel (8-byte column slabs) and the bulk kernel."""
    gh.log("worked 8x8 via %s" % bucket)
    plan = gh.check_against_oracle(synth.worked_example(), **kw)
    assert plan.info()["regions"][bucket] == 8


@pytest.mark.parametrize("seed", range(200))
def test_tiny_layouts(seed):
    gh.check_against_oracle(synth.tiny_case(seed))


@pytest.mark.parametrize("seed", range(0, 200, 3))
@pytest.mark.parametrize("dtype", ["u8", "bf16"])
def test_tiny_layouts_narrow(seed, dtype):
    gh.check_against_oracle(synth.tiny_case(seed, dtype=dtype))


@pytest.mark.parametrize("seed", range(0, 200, 5))
@pytest.mark.parametrize("shifts", [(1, 0), (0, 3), (5, 9), (8, 8)])
def test_tiny_layouts_misaligned_pointers(seed, shifts):
    gh.check_against_oracle(synth.tiny_case(seed, dtype="u8"), src_shift=shifts[0],
                            dst_shift=shifts[1])


@pytest.mark.parametrize("seed", range(0, 200, 4))
def test_tiny_layouts_no_fanout(seed):
    gh.check_against_oracle(synth.tiny_case(seed), fanout=False)


def _round_trip(wl):
    """A -> B on the GPU (checked against the oracle), then B -> A on the GPU
    from the GPU's own B buffers: A must come back bit for bit."""
    G, sources, named, per = helpers.golden_workload(wl)
    plan, src_dev, dst_dev = gh.device_run(wl, sources, per)
    for host_img, dev in dst_dev:
        assert np.array_equal(dev.host(), host_img)
        assert dev.guard_ok()
    back = synth.reverse(wl)
    bplan = lh.plan_workload(back)
    out = [gh.DevBuf(e["buf"].size, poison=0x3C) for e in sources[0]]
    binding.reshard_execute(bplan, [d.ptr for _, d in dst_dev], [o.ptr for o in out],
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for e, o in zip(sources[0], out):
        assert np.array_equal(o.host(), e["buf"])
        assert o.guard_ok()


@pytest.mark.parametrize("seed", range(500))
def test_uneven_layouts_round_trip(seed):
    _round_trip(synth.uneven_case(seed))


@pytest.mark.parametrize("kw", [{}, {"unit_bytes": 4096}, {"fanout": False},
                                {"tiny_bytes": 0, "thin_bytes": 1},
                                {"tiny_bytes": 0, "thin_bytes": 4096}])
@pytest.mark.parametrize("seed", range(0, 500, 25))
def test_uneven_layouts_bucket_variants(seed, kw):
    gh.check_against_oracle(synth.uneven_case(seed), **kw)


@pytest.mark.parametrize("fanout", [True, False])
@pytest.mark.parametrize("seed", range(0, 500, 25))
def test_uneven_layouts_through_tiny_kernel(seed, fanout):
    """Every region up to 64 KiB through the wave-scan kernel: thousands of
    granules per wave, several granules in flight per lane, replicas."""
    gh.check_against_oracle(synth.uneven_case(seed), tiny_bytes=1 << 16, fanout=fanout)


SECOND_POISON = {
    "worked_8x8": synth.worked_example,
    "moe_small": lambda: synth.moe_experts(16, 512, 192, 8, 4, 4, seed=9),
    "moe_small_mxfp8": lambda: synth.moe_experts(16, 512, 192, 8, 4, 4, seed=9, quant="mxfp8"),
    "uneven_3": lambda: synth.uneven_case(3),
    "dense_ffn_fanout": lambda: synth.dense_ffn(hidden=256, inter=1000, src_tp=4, dst_tp=2, dst_dp=2),
}


@pytest.mark.parametrize("poison", [0x00, 0xFF])
@pytest.mark.parametrize("name", sorted(SECOND_POISON))
def test_other_poison_bytes(name, poison):
    """Destinations poisoned with 0x00 and 0xFF instead of 0xA5: a byte the
    kernels fail to write, or write outside a view, cannot hide behind a
    coincidence with one poison value."""
    gh.check_against_oracle(SECOND_POISON[name](), poison=poison)


EMPTY_CASES = [
    # (shape, src mesh, src placements, dst mesh, dst placements)
    ([0, 5], [2], [0], [3], [1]),            # no elements at all
    ([3, 40], [8], [0], [4], [1]),           # 5 of 8 source shards empty
    ([2, 3, 7], [2, 4], [1, 2], [8], [0]),   # 6 of 8 destination shards empty
    ([5, 1], [3], [-1], [6], [1]),           # replicated sources, 5 of 6 destinations empty
]


@pytest.mark.parametrize("dtype", ["u8", "bf16", "f32"])
@pytest.mark.parametrize("case", range(len(EMPTY_CASES)))
def test_empty_shards(case, dtype):
    """Zero-extent tensors and meshes larger than the dim they shard (the
    torch.chunk rule leaves trailing shards empty)."""
    shape, sm, sp, dm, dp = EMPTY_CASES[case]
    t = {"name": "e", "shape": shape, "dtype": dtype, "src": synth.side(sm, sp),
         "dst": synth.side(dm, dp), "values": {"kind": "index"}}
    gh.check_against_oracle({"name": "empty_%d" % case, "buffers": {}, "tensors": [t]})


def _identity(wl):
    out = dict(wl)
    out["tensors"] = [dict(t, dst=dict(t["src"])) for t in wl["tensors"]]
    out["name"] = wl["name"] + "_identity"
    return out


@pytest.mark.parametrize("seed", range(0, 500, 50))
def test_identity_layouts(seed):
    """A -> A: the destination layout equals the source layout."""
    gh.check_against_oracle(_identity(synth.uneven_case(seed)))


def test_identity_moe_layer():
    gh.check_against_oracle(_identity(synth.moe_experts(16, 512, 192, 8, 4, 4, seed=9)))


@pytest.mark.parametrize("shifts", [(4, 0), (0, 2), (6, 10)])
@pytest.mark.parametrize("seed", range(0, 500, 50))
def test_uneven_layouts_misaligned(seed, shifts):
    gh.check_against_oracle(synth.uneven_case(seed), src_shift=shifts[0], dst_shift=shifts[1])


def test_dense_ffn_ragged():
    gh.check_against_oracle(synth.dense_ffn(hidden=256, inter=1000, src_tp=4, dst_tp=2,
                                            dst_dp=2))


def test_dense_ffn_full_size():
    """hidden 4096, intermediate 14336: TP4 -> TP2 x DP2 with fused gate/up."""
    gh.log("dense ffn 4096 x 14336")
    gh.check_against_oracle(synth.dense_ffn())


@pytest.mark.parametrize("kw", [{}, {"fanout": False}, {"unit_bytes": 4096}])
def test_dense_ffn_plan_variants(kw):
    gh.check_against_oracle(synth.dense_ffn(hidden=512, inter=1536), **kw)


MOE_SMALL = [
    (16, 512, 192, 8, 4, 4),     # several tiles per region
    (12, 200, 100, 3, 2, 4),     # ragged: 100 / 4 per TP shard, 200 hidden
    (32, 256, 64, 16, 8, 8),     # the DSV3 meshes at a small size
    (6, 96, 40, 3, 2, 3),        # uneven intermediate split
    (4, 9000, 64, 2, 2, 2),      # MXFP8 rows split into 8192 + 808 elements (short last block)
    (2, 17000, 24, 1, 2, 1),     # two full 8192-element segments and a 616-element tail
]


@pytest.mark.parametrize("shape", MOE_SMALL)
def test_moe_experts_small(shape):
    gh.check_against_oracle(synth.moe_experts(*shape, seed=9))


@pytest.mark.parametrize("quant", [None, "mxfp8"])
@pytest.mark.parametrize("shape", MOE_SMALL[:4])
def test_moe_experts_per_expert_sources(shape, quant):
    """Sources held as one buffer per expert: one region per expert, many
    pointers (several launch groups at the larger expert counts)."""
    gh.check_against_oracle(synth.moe_experts(*shape, seed=9, quant=quant, src_split=True))


@pytest.mark.parametrize("shifts", [(0, 0), (2, 6)])
def test_destination_siblings_interleaved(shifts):
    """Two pieces of every destination row (TP3 -> TP2 over a 2,049-wide bf16
    dim, meeting off the 16-byte grid), cut into interleaved chunks of 64
    units' rows by the planner: byte for byte against the oracle."""
    t = {"name": "w", "shape": [4, 2049, 2049], "dtype": "bf16", "src": synth.side([3], [2]),
         "dst": synth.side([2], [2]), "values": {"kind": "normal", "std": 0.02, "seed": 21}}
    gh.log("siblings %s" % (shifts,))
    plan = gh.check_against_oracle({"name": "dst_siblings", "buffers": {}, "tensors": [t]},
                                   src_shift=shifts[0], dst_shift=shifts[1])
    assert plan.info()["n_regions"] > 4


@pytest.mark.parametrize("quant", [None, "mxfp8"])
def test_per_expert_sources_table_form(quant):
    """256 per-expert source buffers (768 source pointers, more than one
    launch's arguments hold): reshard_execute runs the plan's table form (one
    launch per kernel kind, pointers read from a device table of the plan;
    the bf16 plan's thin regions as sibling groups loaded whole) against the
    oracle."""
    wl = synth.moe_experts(256, 256, 96, 8, 4, 2, seed=9, quant=quant, src_split=True)
    plan = gh.check_against_oracle(wl)
    info = plan.info()
    assert info["n_launches"] < info["n_launches_pooled"], info


@pytest.mark.parametrize("shape", MOE_SMALL)
def test_moe_experts_small_mxfp8(shape):
    gh.check_against_oracle(synth.moe_experts(*shape, seed=9, quant="mxfp8"))


@pytest.mark.parametrize("shifts", [(2, 0), (0, 1), (6, 3), (8, 8)])
@pytest.mark.parametrize("shape", [MOE_SMALL[0], MOE_SMALL[1], MOE_SMALL[4]])
def test_moe_experts_mxfp8_misaligned(shape, shifts):
    """Sources on 2-byte (not 16-byte) boundaries: groups are gathered into
    LDS element by element instead of the direct 16-byte loads; odd
    destination offsets take the byte stores."""
    gh.check_against_oracle(synth.moe_experts(*shape, seed=9, quant="mxfp8"), src_shift=shifts[0],
                            dst_shift=shifts[1])


@pytest.mark.parametrize("shape,inner", [([6, 40, 64], 64), ([3, 30, 200], 200), ([2, 8, 8200], 8200),
                                         ([5, 3, 33], 33), ([7, 11, 8], 8), ([4, 9, 1000], 1000),
                                         ([2, 8, 7168], 7168), ([2, 8, 4104], 4104), ([3, 5, 2050], 2050)])
@pytest.mark.parametrize("mesh,pl", [([2, 2], [0, -1]), ([4], [-1]), ([2, 3], [-1, 1])])
def test_mxfp8_fanout_and_row_lengths(shape, inner, mesh, pl):
    """Replicated MXFP8 destinations (one read, up to four replicas written)
    over row lengths that pack 1..128 rows into a work unit, rows shorter
    than a block, and a row just over one unit."""
    t = {"name": "w", "shape": shape, "dtype": "bf16", "src": synth.side([2], [0]),
         "dst": synth.side(mesh, pl, quant="mxfp8"), "values": {"kind": "normal", "std": 0.02, "seed": 21}}
    gh.check_against_oracle({"name": "mx_fan", "buffers": {}, "tensors": [t]})


@pytest.mark.parametrize("as_source", [False, True])
def test_permuted_rank_grid_fixture(as_source):
    """The hand-written permuted rank grid (tests/golden/permuted_grid_2x2.txt)
    as destination and as source."""
    import test_oracle_layout as tl
    wl = tl.grid_workload(as_source)
    gh.check_against_oracle(wl)
    if not as_source:
        _, slots = tl.read_grid_fixture()
        G, sources, named, per = helpers.golden_workload(wl)
        _, _, dst_dev = gh.device_run(wl, sources, per)
        for k, (_, ln, block) in slots.items():
            got = dst_dev[k][1].host().view(np.uint32).reshape(ln)
            np.testing.assert_array_equal(got, block.astype(np.uint32))


@pytest.mark.parametrize("dst_mesh,dst_pl", [([2], [1]), ([2, 2], [0, -1]), ([3], [2])])
def test_mxfp8_strided_scale_views(dst_mesh, dst_pl):
    """Element rows padded to a longer pitch and block scales with a last-dim
    stride of 3 bytes (every third byte of a padded scale row): the kernel's
    per-block scale addressing, with replicas and a split last dim."""
    shape = [4, 20, 200]
    t = {"name": "w", "shape": shape, "dtype": "bf16", "src": synth.side([2], [0]),
         "values": {"kind": "normal", "std": 0.02, "seed": 31}}
    nslots = 1
    for m in dst_mesh:
        nslots *= m
    # local shapes: last dim up to 200 (or 67 when split in 3), <= 10 / 20 rows
    pitch, rows, blocks = 256, 4 * 20, 7
    slots, scales, bufs = [], [], {}
    for k in range(nslots):
        bufs["e/%d" % k] = {"dtype": "u8", "elems": 5 + rows * pitch}
        bufs["s/%d" % k] = {"dtype": "u8", "elems": 2 + rows * 3 * (blocks + 1) * 2}
        slots.append({"buf": "e/%d" % k, "view": (5, [20 * pitch, pitch, 1])})
        scales.append({"buf": "s/%d" % k, "view": (2, [20 * 3 * (blocks + 1) * 2, 3 * (blocks + 1) * 2, 3])})
    t["dst"] = synth.side(dst_mesh, dst_pl, slots=slots, quant="mxfp8", scale_slots=scales)
    gh.check_against_oracle({"name": "mx_strided_scales", "buffers": bufs, "tensors": [t]})


@pytest.mark.parametrize("quant", [None, "mxfp8"])
@pytest.mark.parametrize("layout", [([2], [1], [3], [0]), ([2, 2], [0, 1], [4], [0]), ([3], [-1], [2, 2], [0, 2])])
def test_per_part_destinations(layout, quant):
    """Destinations held as one buffer per local dim-0 index (e.g. one per
    expert on the receiving side), MXFP8 scale buffers split the same way."""
    sm, sp, dm, dp = layout
    t = {"name": "w", "shape": [6, 40, 96], "dtype": "bf16", "src": synth.side(sm, sp),
         "dst": synth.side(dm, dp, quant=quant, split0=True),
         "values": {"kind": "normal", "std": 0.02, "seed": 41}}
    gh.check_against_oracle({"name": "dst_parts", "buffers": {}, "tensors": [t]})


@pytest.mark.parametrize("quant", [None, "mxfp8"])
@pytest.mark.parametrize("mesh,pl", [([20], [-1]), ([2, 17], [-1, -1]), ([4, 6], [0, -1])])
def test_more_than_16_replicas(mesh, pl, quant):
    """Fan-out groups hold at most 16 destination replicas: 20, 34 and 6
    replicas per shard, each written in full."""
    t = {"name": "w", "shape": [8, 64, 96], "dtype": "bf16", "src": synth.side([2], [0]),
         "dst": synth.side(mesh, pl, quant=quant), "values": {"kind": "normal", "std": 0.02, "seed": 43}}
    plan = gh.check_against_oracle({"name": "fan", "buffers": {}, "tensors": [t]})
    assert max(len(r["dst_index"]) for r in plan.regions()) <= 16


def test_mxfp8_extreme_values():
    """Blocks spanning many binades, zeros, negative zeros, bf16 subnormals,
    the largest bf16 and NaN/Inf blocks (the NaN/Inf convention is the
    library's, shared by the oracle; it is not pinned by any page)."""
    wl = synth.moe_experts(4, 64, 96, 2, 2, 2, seed=3, quant="mxfp8")
    rng = np.random.default_rng(4)
    globals_ = []
    for t in wl["tensors"]:
        shape = t["shape"]
        scale = np.exp2(rng.integers(-140, 120, size=shape[:-1] + [1])).astype(np.float64)
        x = np.clip(rng.standard_normal(shape) * scale, -3e38, 3e38).astype(np.float32)
        b = (x.view(np.uint32) >> 16).astype(np.uint16)
        b[rng.random(shape) < 0.05] = 0x8000
        b[rng.random(shape) < 0.05] = 0x0000
        b[rng.random(shape) < 0.03] = rng.integers(1, 0x80, size=1)[0]
        b[rng.random(shape) < 0.001] = 0x7F7F
        b[rng.random(shape) < 0.001] = 0x7FC0
        b[rng.random(shape) < 0.001] = 0xFF80
        globals_.append(b)
    gh.check_against_oracle(wl, globals_=globals_)


def _all_bf16_orders():
    """Eight arrangements of all 65536 bf16 bit patterns: in order (blocks of
    nearby values, including the NaN/Inf range), three seeded shuffles (blocks
    mixing far-apart binades), and four exponent-windowed shuffles (blocks
    within about a dozen binades, so small elements land on E4M3 subnormals
    and zero)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    out = [allb.copy()]
    rng = np.random.default_rng(12)
    for _ in range(3):
        out.append(rng.permutation(allb))
    order = np.argsort(((allb >> 7) & 0xFF).astype(np.int64) * 65536 + rng.integers(0, 65536, 65536),
                       kind="stable")
    by_exp = allb[order]
    for w in (1024, 2048, 4096, 8192):
        x = by_exp.copy()
        for i in range(0, x.size, w):
            x[i:i + w] = rng.permutation(x[i:i + w])
        out.append(x)
    return np.stack(out)


def test_mxfp8_every_bf16_pattern():
    G = _all_bf16_orders().reshape(8, 64, 1024)
    t = {"name": "allbf16", "shape": [8, 64, 1024], "dtype": "bf16",
         "src": synth.side([2], [0]), "dst": synth.side([2, 2], [0, 1], quant="mxfp8"),
         "values": {"kind": "index"}}
    wl = {"name": "mxfp8_all_bf16", "buffers": {}, "tensors": [t]}
    gh.check_against_oracle(wl, globals_=[G])


@pytest.mark.parametrize("tiny_bytes", [256, 1024])
@pytest.mark.parametrize("reverse", [False, True], ids=["pack", "unpack"])
def test_misc_pack_full_size(reverse, tiny_bytes):
    """61 layers of small tensors (norms, router, bias) packed into one
    buffer, and unpacked again: many regions of mixed sizes in one plan.  With
    a 1 KiB tiny threshold the 1 KiB bias regions go through the wave-scan
    kernel (many granules per wave)."""
    wl = synth.misc_pack()
    if reverse:
        wl = synth.reverse(wl)
    gh.log(wl["name"])
    plan = gh.check_against_oracle(wl, tiny_bytes=tiny_bytes)
    assert (plan.info()["regions"]["tiny"] > 0) == (tiny_bytes == 1024)


@pytest.mark.parametrize("kw", [{}, {"src_split": True}])
def test_fp8_blockwise_layer_small(kw):
    """Blockwise-FP8 weight bytes and their float32 block scales in one plan,
    gate/up fused (weights in w13, scales in s13)."""
    gh.check_against_oracle(synth.fp8_moe_experts(8, 256, 512, 4, 2, 2, seed=3, **kw))


@pytest.mark.parametrize("src_split", [False, True])
@pytest.mark.parametrize("shape", [(10, 256, 768, 4, 3, 2, 128), (6, 320, 384, 2, 3, 3, 64),
                                   (5, 128, 256, 5, 1, 2, 128), (12, 384, 512, 3, 4, 4, 128)])
def test_fp8_blockwise_uneven_expert_splits(shape, src_split):
    """Blockwise FP8 with uneven expert splits (10 experts over 4 -> 3
    ranks), three-way TP, 64-element blocks, a single destination EP rank
    and per-expert source buffers: weight bytes and scales byte for byte."""
    e, h, i, se, de, dt, b = shape
    gh.check_against_oracle(synth.fp8_moe_experts(e, h, i, se, de, dt, seed=6, block=b,
                                                  src_split=src_split))


def test_fp8_blockwise_dsv3_shape_32_experts():
    """32 experts of the DeepSeek-V3 FP8 layer (hidden 7168, intermediate
    2048, 128 x 128 blocks), EP16 -> EP8 x TP8."""
    gh.log("fp8 dsv3 32 experts")
    gh.check_against_oracle(synth.fp8_moe_experts(32, 7168, 2048, 16, 8, 8, seed=4))


@pytest.mark.parametrize("shifts", [(0, 0), (2, 1)])
@pytest.mark.parametrize("i", range(9))
def test_mxfp8_blocks_from_two_sources(i, shifts):
    """MXFP8 blocks that straddle a source shard boundary along the last dim
    (TP3 over 2,048, 257 = 129 + 128, both sides cutting the last dim, rows
    longer than a unit), gathered from two sources in one work unit; also
    with sources on 2-byte and destinations on odd byte boundaries."""
    import test_planner as tp
    gh.check_against_oracle(tp.mx_split_workload(i), src_shift=shifts[0], dst_shift=shifts[1])


@pytest.mark.parametrize("seed", range(0, 40, 3))
def test_mxfp8_random_last_dim_splits(seed):
    import test_planner as tp
    rng = np.random.default_rng(seed)
    nd = int(rng.integers(2, 4))
    shape = [int(rng.integers(1, 6)) for _ in range(nd - 1)] + [int(rng.integers(33, 700))]
    parts = int(rng.integers(2, max(3, min(8, shape[-1] // 32) + 1)))
    smesh, spl = ([parts], [nd - 1]) if rng.integers(2) else ([2, parts], [0, nd - 1])
    dmesh, dpl = [[1], [-1]] if rng.integers(2) else [[2], [int(rng.integers(0, nd))]]
    t = {"name": "w", "shape": shape, "dtype": "bf16", "src": synth.side(smesh, spl),
         "dst": synth.side(dmesh, dpl, quant="mxfp8"), "values": {"kind": "normal", "std": 0.02, "seed": seed}}
    gh.check_against_oracle({"name": "mx_rand_%d" % seed, "buffers": {}, "tensors": [t]})


def test_mxfp8_two_source_blocks_replicated():
    """Two-piece regions with replicated destinations (one read, four
    element and scale replicas written)."""
    t = {"name": "w", "shape": [6, 2048], "dtype": "bf16", "src": synth.side([3], [1]),
         "dst": synth.side([2, 2], [0, -1], quant="mxfp8"),
         "values": {"kind": "normal", "std": 0.02, "seed": 77}}
    plan = gh.check_against_oracle({"name": "mx_two_rep", "buffers": {}, "tensors": [t]})
    two = [r for r in plan.regions() if r["split"] < r["inner"]]
    assert two and all(len(r["dst_index"]) == 2 for r in two)


MISALIGNED_LONG = {
    # TP3 -> TP2 over an odd bf16 width: rows of 683 / 342 / 341 elements at
    # source and destination offsets that differ modulo 16
    "bf16_tp3_to_tp2_2049": ([6, 300, 2049], "bf16", ([3], [2]), ([2], [2])),
    "bf16_rows_to_cols_4097": ([40, 4097], "bf16", ([3], [0]), ([3], [1])),
    "u8_odd_widths": ([33, 3001], "u8", ([7], [1]), ([2, 2], [1, -1])),
    "f32_tp5_to_tp3": ([64, 1001], "f32", ([5], [1]), ([3], [1])),
}


@pytest.mark.parametrize("shifts", [(0, 0), (2, 0), (0, 6), (10, 4), (1, 3)])
@pytest.mark.parametrize("name", sorted(MISALIGNED_LONG))
def test_misaligned_long_rows(name, shifts):
    """Rows whose source and destination differ modulo 16 (odd splits, and
    buffers shifted by a few bytes): 16-byte stores fed by funnel-shifted
    pairs of aligned loads, edges by granules."""
    shape, dtype, src, dst = MISALIGNED_LONG[name]
    if dtype != "u8" and (shifts[0] % 2 or shifts[1] % 2):
        shifts = (shifts[0] & ~1, shifts[1] & ~1)
    if dtype == "f32":
        shifts = (shifts[0] & ~3, shifts[1] & ~3)
    vals = {"kind": "uniform", "seed": 5} if dtype in ("f32", "bf16") else {"kind": "index"}
    t = {"name": "w", "shape": shape, "dtype": dtype, "src": synth.side(*src), "dst": synth.side(*dst),
         "values": vals}
    gh.check_against_oracle({"name": "mis_" + name, "buffers": {}, "tensors": [t]},
                            src_shift=shifts[0], dst_shift=shifts[1], tiny_bytes=0, thin_bytes=1)


@pytest.mark.parametrize("seed", range(0, 60, 3))
def test_high_rank_layouts(seed):
    """Ranks 4-6 with padded views (regions with more than three outer dims
    are peeled by the planner)."""
    gh.log("high rank %d" % seed)
    gh.check_against_oracle(helpers.high_rank_case(seed))


@pytest.mark.parametrize("seed", range(0, 40, 2))
def test_high_rank_mxfp8(seed):
    gh.log("high rank mxfp8 %d" % seed)
    gh.check_against_oracle(helpers.high_rank_case(seed, mx=True))


def _padded_source(shape, mesh, pl, pad):
    """A bf16 source side whose slots are views with `pad` extra elements
    per row (row strides off the 16-byte grid)."""
    from oracle import layout as olayout
    desc = {"shape": shape, "dtype": "bf16", "mesh": mesh, "placements": pl, "slot_of_coord": None,
            "quant": None}
    bufs, slots = {}, []
    for k, (_, ln) in enumerate(olayout.slot_boxes(desc)):
        dims = list(ln)
        st, acc = [], 1
        for i in reversed(range(len(dims))):
            st.append(acc)
            acc *= dims[i] + (pad if i == len(dims) - 1 else 0)
        bufs["s%d" % k] = {"dtype": "bf16", "elems": acc + 3}
        slots.append({"buf": "s%d" % k, "view": (3, list(reversed(st)))})
    return bufs, synth.side(mesh, pl, slots=slots)


MX_MISALIGNED = {
    # source shards off the 8-element grid along the last dim: rows staged as
    # aligned lines (several rows per unit, one row per unit)
    "tp3_last_dim_1000": ([4, 16, 1000], ([3], [2]), ([2], [1]), 0),
    "tp3_last_dim_7168": ([2, 8, 7168], ([3], [2]), ([2, 2], [0, 1]), 0),
    "tp5_last_dim_replicated": ([3, 24, 1337], ([5], [2]), ([2, 2], [1, -1]), 0),
    # padded source rows: row strides off the 16-byte grid; 1,024-element
    # rows leave no spare slots (the register funnel path), 300 and 7,000 do
    "padded_rows_1024": ([4, 12, 1024], ([2], [0]), ([2], [1]), 1),
    "padded_rows_300": ([6, 40, 300], ([1], [-1]), ([3], [1]), 3),
    "padded_rows_7000": ([2, 6, 7000], ([2], [1]), ([1], [-1]), 5),
}


MX_PITCHED = {
    # rows whose units take a slot pitch that is not a power of two (rows of
    # 1,088 elements: 7 per unit at 140 slots instead of 4 at 256), from
    # aligned source rows, with a remainder unit of 5 rows and rows crossing
    # the outer dim inside a unit
    "aligned_rows_1088": ([3, 50, 3264], ([3], [2]), ([2], [1])),
    # misaligned rows of 608 / 576 / 582 elements (two-piece blocks between
    # them), every destination row to two replicas
    "replicated_1830": ([2, 30, 1830], ([3], [2]), ([2, 2], [1, -1])),
    # a last unit of one row
    "one_row_remainder_1088": ([1, 8, 3264], ([3], [2]), ([1], [-1])),
    # the DeepSeek-V3 hidden dim from a TP3 source: 2,368-element rows, 3 per
    # unit at 300 slots
    "dsv3_like_2368": ([4, 64, 7168], ([3], [2]), ([2], [1])),
}


@pytest.mark.parametrize("shifts", [(0, 0), (2, 3)])
@pytest.mark.parametrize("name", sorted(MX_PITCHED))
def test_mxfp8_pitched_units(name, shifts):
    """MXFP8 regions whose rows are staged at a slot pitch that is not a
    power of two (the second MXFP8 kernel, which also takes the two-piece
    regions): several rows per unit, row and scale slots found by a
    multiply by a reciprocal, byte for byte against the oracle."""
    shape, (sm, sp), (dm, dp) = MX_PITCHED[name]
    t = {"name": "w", "shape": shape, "dtype": "bf16", "src": synth.side(sm, sp),
         "dst": synth.side(dm, dp, quant="mxfp8"), "values": {"kind": "normal", "std": 0.02, "seed": 83}}
    gh.log("mx pitched %s %s" % (name, shifts))
    gh.check_against_oracle({"name": "mx_pitch_" + name, "buffers": {}, "tensors": [t]},
                            src_shift=shifts[0], dst_shift=shifts[1])


@pytest.mark.parametrize("shifts", [(0, 0), (2, 3), (6, 0)])
@pytest.mark.parametrize("name", sorted(MX_MISALIGNED))
def test_mxfp8_misaligned_source_rows(name, shifts):
    """MXFP8 installs from source rows that are not 16-byte aligned (source
    shards cut off the 8-element grid, padded row strides, shifted
    pointers): groups rebuilt from aligned lines with funnel shifts, the
    rows' partial first and last lines element by element."""
    shape, (sm, sp), (dm, dp), pad = MX_MISALIGNED[name]
    bufs = {}
    if pad:
        bufs, src = _padded_source(shape, sm, sp, pad)
    else:
        src = synth.side(sm, sp)
    t = {"name": "w", "shape": shape, "dtype": "bf16", "src": src,
         "dst": synth.side(dm, dp, quant="mxfp8"), "values": {"kind": "normal", "std": 0.02, "seed": 81}}
    gh.log("mx misaligned %s %s" % (name, shifts))
    gh.check_against_oracle({"name": "mx_mis_" + name, "buffers": bufs, "tensors": [t]},
                            src_shift=shifts[0], dst_shift=shifts[1])
