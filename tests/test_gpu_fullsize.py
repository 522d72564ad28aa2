"""GPU parity at the full layer sizes, in the launch configuration the
benchmark times (default plan options, one execute on the current stream).

Checks, per layer:
* three whole destination slots of every tensor against the oracle, every
  element (and for MXFP8 every scale byte): the oracle assembles the full
  tensor on the host from the device's source shards and slices, and
  quantises, those slots;
* every destination slot, for the bf16 copies, against torch slicing of the
  seeded global tensor regenerated on the device (position by position);
* sampled destination elements (MXFP8: blocks) located one by one with the
  oracle's own box arithmetic, and no poison byte left anywhere (0xFF bytes
  form a bf16 NaN that N(0, 0.02) never produces and that the MXFP8 encoder
  never emits for finite input);
* the A -> B -> A round trip, every source byte.
A 16-expert slice of the DeepSeek-V3-shaped layer (the same hidden and
intermediate sizes, meshes and unit shapes) is compared with the oracle
element by element in full.  So are the other large layouts the benchmark
times: the uneven [16, 8193, 2049] bf16 TP3 -> TP2 layout and the 16M-row
column slabs, every byte; the MXFP8 install of the DeepSeek-V3 gate and up
projections from a source cut TP3 along the hidden dim, three whole slots
per tensor and sampled blocks.
"""

import numpy as np
import pytest
import torch

from oracle import golden as ogolden
from oracle import layout as olayout
from oracle import mxfp8 as omx
from rl_weight_refit_amd import binding, synth

import gpu_helpers as gh
import helpers
import lib_helpers as lh

pytestmark = pytest.mark.gpu

POISON = 0xFF


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield
    torch.cuda.empty_cache()


def dense_strides(lengths):
    return ogolden.dense_strides(lengths)


def build(wl):
    """Device sources (cut from seeded device-generated globals with the
    oracle's boxes; one buffer per expert for split sources) and poisoned
    destination buffers (every destination of these layers is a view into a
    named buffer)."""
    dev = torch.device("cuda")
    src = []
    for t in wl["tensors"]:
        G = synth.device_values(t, dev).view(torch.int16)
        shards = []
        for off, ln in olayout.slot_boxes(helpers.src_desc_for(t)):
            sl = tuple(slice(o, o + n) for o, n in zip(off, ln))
            if t["src"].get("split0"):
                shards.append([G[o0].contiguous() for o0 in range(off[0], off[0] + ln[0])])
            else:
                shards.append(G[sl].contiguous())
        del G
        src.append(shards)
    torch.cuda.synchronize()
    named = {}
    for key, b in wl["buffers"].items():
        named[key] = torch.full((b["elems"] * synth.ELEM_BYTES[b["dtype"]],), POISON,
                                dtype=torch.uint8, device=dev)
    dst_ptrs = []
    for t in wl["tensors"]:
        d = t["dst"]
        assert d["slots"] is not None
        dst_ptrs += [named[e["buf"]].data_ptr() for e in d["slots"]]
        if d.get("quant") == "mxfp8":
            dst_ptrs += [named[e["buf"]].data_ptr() for e in d["scale_slots"]]
    return src, named, dst_ptrs


def run(wl):
    src, named, dst_ptrs = build(wl)
    plan = lh.plan_workload(wl)
    src_ptrs = [p.data_ptr() for shards in src for s in shards
                for p in (s if isinstance(s, list) else [s])]
    binding.reshard_execute(plan, src_ptrs, dst_ptrs, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return plan, src, named


def dsv3_gate_up_mxfp8_tp3_source():
    """The DSV3 gate and up projections installed as MXFP8 from a source cut
    TP3 along the 7,168-wide hidden dim: rows of 2,390 elements off the
    16-byte grid, and blocks that straddle two source shards."""
    wl = synth.moe_dsv3(quant="mxfp8")
    wl["tensors"] = [dict(t, src=synth.side([3], [2])) for t in wl["tensors"][:2]]
    wl["name"] += "_gate_up_tp3_hidden_src"
    return wl


WORKLOADS = {
    "moe_128e": synth.moe_128e,
    "moe_dsv3": synth.moe_dsv3,
    "moe_dsv3_per_expert_src": lambda: synth.moe_dsv3(src_split=True),
    "moe_dsv3_mxfp8": lambda: synth.moe_dsv3(quant="mxfp8"),
    "moe_dsv3_mxfp8_tp3_src": dsv3_gate_up_mxfp8_tp3_source,
}
_RUNS = {}


def layer_run(key):
    """The layer relaid out once; later tests of the same layer reuse its
    buffers (the previous layer's are released first)."""
    if key not in _RUNS:
        _RUNS.clear()
        torch.cuda.empty_cache()
        wl = WORKLOADS[key]()
        gh.log("full size %s" % wl["name"])
        plan, src, named = run(wl)
        _RUNS[key] = (wl, src, named)
    return _RUNS[key]


def slot_tensor(named, entry, lengths, elem):
    """The destination slot seen through its view (int16 elements for bf16,
    bytes for MXFP8 codes and scales)."""
    buf = named[entry["buf"]]
    flat = buf.view(torch.int16) if elem == "bf16" else buf
    base, strides = entry["view"]
    return torch.as_strided(flat, size=list(lengths), stride=list(strides), storage_offset=base)


def check_every_slot_on_device(wl, named):
    """Every destination slot equals torch slicing of the seeded global
    tensor, regenerated on the device, at the oracle's box."""
    for t in wl["tensors"]:
        G = synth.device_values(t, "cuda").view(torch.int16)
        for k, (off, ln) in enumerate(olayout.slot_boxes(helpers.odesc(t, "dst"))):
            want = G[tuple(slice(o, o + n) for o, n in zip(off, ln))]
            got = slot_tensor(named, t["dst"]["slots"][k], ln, "bf16")
            assert torch.equal(got, want), (wl["name"], t["name"], k)
        del G
        torch.cuda.empty_cache()


def host_source_entries(shards):
    """Oracle source entries (byte images) of one tensor's device shards."""
    out = []
    for s in shards:
        if isinstance(s, list):
            out.append({"parts": [p.cpu().numpy().view(np.uint8).reshape(-1) for p in s]})
        else:
            out.append({"buf": s.cpu().numpy().view(np.uint8).reshape(-1)})
    return out


def check_slots_against_oracle(wl, ti, src, named, slots):
    """Whole destination slots of tensor ti against the oracle: the full
    tensor assembled on the host from the device's source shards, each slot's
    box sliced (and quantised for MXFP8), compared with every element (and
    scale byte) the device installed."""
    t = wl["tensors"][ti]
    d = t["dst"]
    G = ogolden.assemble(helpers.src_desc_for(t), 2, host_source_entries(src[ti]))
    boxes = olayout.slot_boxes(helpers.odesc(t, "dst"))
    for k in slots:
        ln = boxes[k][1]
        V = np.ascontiguousarray(G[ogolden.box_slices(boxes[k])])
        if d.get("quant") == "mxfp8":
            codes, scales = omx.quantize(V)
            got = slot_tensor(named, d["slots"][k], ln, "u8").cpu().numpy()
            np.testing.assert_array_equal(got, codes, err_msg="%s slot %d codes" % (t["name"], k))
            sln = list(ln[:-1]) + [-(-ln[-1] // omx.BLOCK)]
            got = slot_tensor(named, d["scale_slots"][k], sln, "u8").cpu().numpy()
            np.testing.assert_array_equal(got, scales, err_msg="%s slot %d scales" % (t["name"], k))
        else:
            got = slot_tensor(named, d["slots"][k], ln, "bf16").cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(got, V, err_msg="%s slot %d" % (t["name"], k))
    del G


def no_poison(buf, dtype):
    """No element still holds the poison pattern (0xFFFF for bf16, 0xFF for bytes)."""
    flat = buf.view(torch.int16) if dtype == "bf16" else buf
    bad = -1 if dtype == "bf16" else POISON
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        if bool((flat[i:i + step] == bad).any()):
            return False
    return True


def sampled_copy_check(wl, src, named, nsamp, rng):
    """Sampled destination elements equal the source element the oracle names."""
    for ti, t in enumerate(wl["tensors"]):
        sdesc = helpers.src_desc_for(t)
        ddesc = helpers.odesc(t, "dst")
        dboxes = olayout.slot_boxes(ddesc)
        slots = t["dst"]["slots"]
        for _ in range(nsamp):
            k = int(rng.integers(len(dboxes)))
            ln = dboxes[k][1]
            l = [int(rng.integers(n)) for n in ln]
            if t["src"].get("split0"):
                g = [a + b for a, b in zip(dboxes[k][0], l)]
                s, loc = ogolden.source_location(sdesc, g)
                want = int(src[ti][s][loc[0]][tuple(loc[1:])]) & 0xFFFF
            else:
                (s, off), = ogolden.expected_sources(sdesc, [None] * len(src[ti]), ddesc, k, [l])
                want = int(src[ti][s].view(-1)[off]) & 0xFFFF
            view = slots[k]["view"] if slots else None
            buf = named[slots[k]["buf"]] if slots else None
            doff = ogolden.element_offset(view, ln, l)
            got = int(buf.view(torch.int16)[doff]) & 0xFFFF
            assert got == want, (t["name"], k, l, hex(got), hex(want))


def sampled_mx_check(wl, src, named, nblocks, rng):
    """Sampled MXFP8 blocks: the oracle gathers the block's 32 source values
    and quantises them; element bytes and the scale byte must match."""
    for ti, t in enumerate(wl["tensors"]):
        sdesc = helpers.src_desc_for(t)
        ddesc = helpers.odesc(t, "dst")
        dboxes = olayout.slot_boxes(ddesc)
        d = t["dst"]
        for _ in range(nblocks):
            k = int(rng.integers(len(dboxes)))
            ln = dboxes[k][1]
            K = ln[-1]
            row = [int(rng.integers(n)) for n in ln[:-1]]
            b = int(rng.integers(-(-K // 32)))
            cols = list(range(32 * b, min(32 * b + 32, K)))
            locs = [row + [c] for c in cols]
            srcs = ogolden.expected_sources(sdesc, [None] * len(src[ti]), ddesc, k, locs)
            bits = np.array([int(src[ti][s].view(-1)[o]) & 0xFFFF for s, o in srcs], dtype=np.uint16)
            codes, scales = omx.quantize(bits[None, :])
            ebuf = named[d["slots"][k]["buf"]]
            got = [int(ebuf[ogolden.element_offset(d["slots"][k]["view"], ln, l)]) for l in locs]
            assert got == list(codes[0]), (t["name"], k, row, b)
            sln = list(ln[:-1]) + [-(-K // 32)]
            sbuf = named[d["scale_slots"][k]["buf"]]
            so = ogolden.element_offset(d["scale_slots"][k]["view"], sln, row + [b])
            assert int(sbuf[so]) == int(scales[0, 0]), (t["name"], k, row, b)


def three_slots(wl):
    n = len(olayout.slot_boxes(helpers.odesc(wl["tensors"][0], "dst")))
    return [0, n // 2 + 5, n - 1]


@pytest.mark.parametrize("which", ["moe_128e", "moe_dsv3"])
def test_full_size_copy_every_slot(which):
    wl, src, named = layer_run(which)
    for key, buf in named.items():
        assert no_poison(buf, wl["buffers"][key]["dtype"]), key
    check_every_slot_on_device(wl, named)
    sampled_copy_check(wl, src, named, 3000, np.random.default_rng(1))


@pytest.mark.parametrize("ti", [0, 1, 2], ids=["gate", "up", "down"])
@pytest.mark.parametrize("which", ["moe_128e", "moe_dsv3"])
def test_full_size_copy_slots_against_oracle(which, ti):
    wl, src, named = layer_run(which)
    check_slots_against_oracle(wl, ti, src, named, three_slots(wl))


@pytest.mark.parametrize("which", ["moe_128e", "moe_dsv3"])
def test_full_size_round_trip(which):
    """A -> B -> A: the sources to the fused EP x TP destinations and back
    (the reverse plan reads through the fused views); every source byte
    must come back (checked on the device)."""
    wl, src, named = layer_run(which)
    gh.log("full size round trip %s" % wl["name"])
    back = synth.reverse(wl)
    bplan = lh.plan_workload(back)
    b_src_ptrs = []
    for t in back["tensors"]:
        b_src_ptrs += [named[e["buf"]].data_ptr() for e in t["src"]["slots"]]
    out = [[torch.empty_like(s) for s in shards] for shards in src]
    b_dst_ptrs = [o.data_ptr() for shards in out for o in shards]
    binding.reshard_execute(bplan, b_src_ptrs, b_dst_ptrs, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for shards, outs in zip(src, out):
        for a, b in zip(shards, outs):
            assert torch.equal(a, b)
    del out


def test_full_size_copy_per_expert_sources():
    wl, src, named = layer_run("moe_dsv3_per_expert_src")
    for key, buf in named.items():
        assert no_poison(buf, wl["buffers"][key]["dtype"]), key
    check_every_slot_on_device(wl, named)
    sampled_copy_check(wl, src, named, 3000, np.random.default_rng(1))
    check_slots_against_oracle(wl, 2, src, named, [0, 63])


def test_full_size_mxfp8_sampled():
    wl, src, named = layer_run("moe_dsv3_mxfp8")
    for key, buf in named.items():
        assert no_poison(buf, wl["buffers"][key]["dtype"]), key
    sampled_mx_check(wl, src, named, 600, np.random.default_rng(2))


@pytest.mark.parametrize("ti", [0, 1, 2], ids=["gate", "up", "down"])
def test_full_size_mxfp8_slots_against_oracle(ti):
    wl, src, named = layer_run("moe_dsv3_mxfp8")
    check_slots_against_oracle(wl, ti, src, named, three_slots(wl))


def test_full_size_mxfp8_tp3_source_sampled():
    """MXFP8 install from the TP3-on-hidden source at full size: no poison
    left in the gate/up element and scale buffers, and sampled blocks (the
    oracle locates each of a block's 32 values in its own source shard)."""
    wl, src, named = layer_run("moe_dsv3_mxfp8_tp3_src")
    for key, buf in named.items():
        if key.startswith(("w13/", "s13/")):
            assert no_poison(buf, wl["buffers"][key]["dtype"]), key
    sampled_mx_check(wl, src, named, 600, np.random.default_rng(3))


@pytest.mark.parametrize("ti", [0, 1], ids=["gate", "up"])
def test_full_size_mxfp8_tp3_source_slots_against_oracle(ti):
    wl, src, named = layer_run("moe_dsv3_mxfp8_tp3_src")
    check_slots_against_oracle(wl, ti, src, named, three_slots(wl))


def test_release_layer_buffers():
    _RUNS.clear()
    torch.cuda.empty_cache()


def test_uneven_bf16_16x8193x2049_tp3_to_tp2_every_byte():
    """The large uneven bf16 layout, [16, 8193, 2049] TP3 -> TP2 on the last
    dim (rows of 683 / 342 / 341 elements at offsets that differ modulo 16
    on the two sides, and destination rows two source pieces share), at full
    size: every destination byte, poison guards included, against the
    oracle."""
    t = {"name": "w", "shape": [16, 8193, 2049], "dtype": "bf16", "src": synth.side([3], [2]),
         "dst": synth.side([2], [2]), "values": {"kind": "normal", "std": 0.02, "seed": 9}}
    wl = {"name": "uneven_bf16_16x8193x2049_tp3_to_tp2", "buffers": {}, "tensors": [t]}
    gh.log("full size %s" % wl["name"])
    gh.check_against_oracle(wl, poison=POISON)


def test_column_slabs_16M_rows_every_byte():
    """Tall-thin column slabs at full size, [16M, 8] int32 (index values): 2
    row shards -> 4 column shards through the thin group kernel, every
    destination byte against the oracle."""
    t = {"name": "w", "shape": [1 << 24, 8], "dtype": "i32", "src": synth.side([2], [0]),
         "dst": synth.side([4], [1]), "values": {"kind": "index"}}
    wl = {"name": "column_slabs_16Mx8_i32_2row_to_4col", "buffers": {}, "tensors": [t]}
    gh.log("full size %s" % wl["name"])
    plan = gh.check_against_oracle(wl, poison=POISON)
    assert plan.info()["regions"]["thin"] == 8


@pytest.mark.parametrize("quant,ti", [(None, None), ("mxfp8", 0), ("mxfp8", 1), ("mxfp8", 2)],
                         ids=["bf16", "mxfp8_gate", "mxfp8_up", "mxfp8_down"])
def test_dsv3_sixteen_expert_slice_every_byte(quant, ti):
    """16 experts of the DeepSeek-V3-shaped layer (hidden 7168, intermediate
    2048, EP16 -> EP8 x TP8, fused w13): every destination pointer has the
    full layer's shapes (7,168-element gate/up rows, 256-element down rows,
    two source shards per destination), compared byte for byte with the
    oracle, poison outside the views and guards included."""
    wl = synth.moe_experts(16, 7168, 2048, 16, 8, 8, seed=5, quant=quant)
    if ti is not None:
        wl = dict(wl, tensors=[wl["tensors"][ti]])
    gh.log("16-expert slice %s %s" % (wl["name"], [t["name"] for t in wl["tensors"]]))
    globals_ = [synth.device_values(t, "cuda").view(torch.int16).cpu().numpy().view(np.uint16)
                for t in wl["tensors"]]
    gh.check_against_oracle(wl, globals_=globals_)


def test_rows_past_2_31():
    """One byte per row, 2^31 + 1000 rows: a [N, 2] u8 tensor split by
    columns over two sources, gathered into one replicated [N, 2]
    destination.  The planner splits the column regions below 2^31 rows
    (the kernels' row indices are 32-bit).  Shard(1) -> Replicate is
    torch.cat of the columns, so the destination must equal G exactly
    (G[i, j] = (2 i + j) mod 256, the index values): checked for every byte,
    and sampled element by element against the oracle's source lookup,
    around row 2^31 included."""
    N = (1 << 31) + 1000
    t = {"name": "col", "shape": [N, 2], "dtype": "u8", "src": synth.side([2], [1]),
         "dst": synth.side([1], [-1]), "values": {"kind": "index"}}
    wl = {"name": "rows_past_2_31", "buffers": {}, "tensors": [t]}
    plan = lh.plan_workload(wl)
    regs = plan.regions()
    assert all(r["ext"][0] * r["ext"][1] * r["ext"][2] < (1 << 31) for r in regs)
    assert sum(r["inner"] * r["ext"][0] * r["ext"][1] * r["ext"][2] for r in regs) == 2 * N
    dev = torch.device("cuda")
    step = 1 << 28
    src = []
    for j in range(2):
        s = torch.empty(N, dtype=torch.uint8, device=dev)
        for a in range(0, N, step):
            b = min(N, a + step)
            s[a:b] = ((torch.arange(a, b, dtype=torch.int64, device=dev) * 2 + j) & 0xFF).to(torch.uint8)
        src.append(s)
    dst = torch.full((2 * N,), POISON, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    binding.reshard_execute(plan, [s.data_ptr() for s in src], [dst.data_ptr()],
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for a in range(0, 2 * N, step):
        b = min(2 * N, a + step)
        want = (torch.arange(a, b, dtype=torch.int64, device=dev) & 0xFF).to(torch.uint8)
        assert bool(torch.equal(dst[a:b], want)), "bytes %d..%d differ" % (a, b)
    rng = np.random.default_rng(31)
    rows = np.concatenate([rng.integers(0, N, 2000), [0, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, N - 1]])
    sd = helpers.src_desc_for(t)
    for i in rows:
        for j in range(2):
            slot, loc = ogolden.source_location(sd, [int(i), j])
            want = int(src[slot][loc[0]].item())
            assert int(dst[2 * int(i) + j].item()) == want, (i, j)
    del src, dst
    torch.cuda.empty_cache()
