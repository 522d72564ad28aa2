"""Test-side glue: turn a synthetic workload into oracle inputs and buffers.

Source shards are cut from the seeded global tensor with the oracle's own
shard boxes; destinations start as poison-filled byte images so that bytes a
reshard must not touch can be checked too.
"""

import numpy as np

import oracle
from oracle import layout as olayout
from oracle import golden as ogolden
from rl_weight_refit_amd import synth

UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def odesc(tensor, side_name):
    s = tensor[side_name]
    dtype = tensor["dtype"]
    if side_name == "dst" and s.get("quant") == "mxfp8":
        dtype = "u8"
    return {"shape": list(tensor["shape"]), "dtype": dtype, "mesh": list(s["mesh"]),
            "placements": list(s["placements"]), "slot_of_coord": s.get("slot_of_coord"),
            "quant": s.get("quant")}


def src_desc_for(tensor):
    d = odesc(tensor, "src")
    d["dtype"] = tensor["dtype"]
    return d


def dense_bytes(arr):
    return np.ascontiguousarray(arr).view(np.uint8).reshape(-1)


def source_buffers(tensor, G, named_src=None):
    """Per source slot: the byte image holding the slot's shard (oracle
    boxes).  Dense slots get a buffer of their own; slots with views are
    written through the view into the shared buffer named_src[key]."""
    desc = src_desc_for(tensor)
    s = tensor["src"]
    out = []
    for k, box in enumerate(olayout.slot_boxes(desc)):
        part = G[ogolden.box_slices(box)]
        if s.get("split0"):
            out.append({"parts": [dense_bytes(part[i]).copy() for i in range(part.shape[0])],
                        "view": None})
        elif s["slots"] is None:
            out.append({"buf": dense_bytes(part).copy(), "view": None})
        else:
            e = s["slots"][k]
            buf = named_src[e["buf"]]
            if part.size:
                ogolden.view_array(buf, synth.ELEM_BYTES[tensor["dtype"]], e["view"], list(part.shape),
                                   writeable=True)[...] = part
            out.append({"buf": buf, "view": e["view"]})
    return out


def alloc_sources(workload):
    """Zeroed images of every named buffer some tensor reads through a view."""
    keys = set()
    for t in workload["tensors"]:
        if t["src"]["slots"] is not None:
            keys |= {e["buf"] for e in t["src"]["slots"]}
    return {k: np.zeros(workload["buffers"][k]["elems"] *
                        synth.ELEM_BYTES[workload["buffers"][k]["dtype"]], dtype=np.uint8)
            for k in sorted(keys)}


def alloc_destinations(workload, poison=0xA5):
    """Host images for every destination buffer, filled with `poison`.

    Returns (named, per_tensor) where named[key] is the image of a shared
    buffer and per_tensor[t][k] is the dict the oracle writes slot k through.
    """
    named = {}
    for key, b in workload["buffers"].items():
        nbytes = b["elems"] * synth.ELEM_BYTES[b["dtype"]]
        named[key] = np.full(nbytes, poison, dtype=np.uint8)
    per_tensor = []
    for t in workload["tensors"]:
        d = t["dst"]
        desc = odesc(t, "dst")
        esize = 1 if d.get("quant") == "mxfp8" else synth.ELEM_BYTES[t["dtype"]]
        slots = []
        boxes = olayout.slot_boxes(desc)
        for k, box in enumerate(boxes):
            ln = box[1]
            if d.get("split0"):
                # one dense buffer per local dim-0 index (and per-part scales)
                per = olayout.box_volume((None, list(ln[1:]))) if len(ln) > 1 else 1
                e = {"parts": [np.full(per * esize, poison, dtype=np.uint8) for _ in range(ln[0])],
                     "view": None}
                if d.get("quant") == "mxfp8":
                    nsc = olayout.box_volume((None, list(ln[1:-1]) + [-(-ln[-1] // 32)]))
                    e["scale_parts"] = [np.full(nsc, poison, dtype=np.uint8) for _ in range(ln[0])]
                    e["scale_view"] = None
                slots.append(e)
                continue
            if d["slots"] is None:
                nbytes = olayout.box_volume(box) * esize
                e = {"buf": np.full(nbytes, poison, dtype=np.uint8), "view": None}
            else:
                e = {"buf": named[d["slots"][k]["buf"]], "view": d["slots"][k]["view"]}
            if d.get("quant") == "mxfp8":
                if d.get("scale_slots") is None:
                    ln = box[1]
                    nsc = olayout.box_volume((None, list(ln[:-1]) + [-(-ln[-1] // 32)]))
                    e["scale_buf"] = np.full(nsc, poison, dtype=np.uint8)
                    e["scale_view"] = None
                else:
                    e["scale_buf"] = named[d["scale_slots"][k]["buf"]]
                    e["scale_view"] = d["scale_slots"][k]["view"]
            slots.append(e)
        per_tensor.append(slots)
    return named, per_tensor


def golden_workload(workload, poison=0xA5, globals_=None):
    """Run the oracle on a whole workload.

    Returns (globals, sources, named, per_tensor): the global tensors, the
    source byte images per tensor, and the destination images after the
    oracle wrote them.
    """
    if globals_ is None:
        globals_ = [synth.host_values(t) for t in workload["tensors"]]
    named_src = alloc_sources(workload)
    sources = [source_buffers(t, G, named_src) for t, G in zip(workload["tensors"], globals_)]
    named, per_tensor = alloc_destinations(workload, poison)
    for t, src, dst in zip(workload["tensors"], sources, per_tensor):
        ogolden.reshard(src_desc_for(t), odesc(t, "dst"), src, dst)
    return globals_, sources, named, per_tensor


def local_arrays(tensor, G, side_name):
    desc = src_desc_for(tensor) if side_name == "src" else odesc(tensor, side_name)
    return [np.ascontiguousarray(G[ogolden.box_slices(b)]) for b in olayout.slot_boxes(desc)]


def high_rank_case(seed, mx=False):
    """A rank 4-6 tensor over tiny meshes whose slots (either side, at
    random) are padded views into shared buffers, so outer dims do not merge
    and regions keep more than three of them (the planner peels those).
    MXFP8 destinations keep the last dim contiguous; their scale views are
    padded the same way."""
    rng = np.random.Generator(np.random.PCG64(77_000 + seed))
    ndim = int(rng.integers(4, 7))
    shape = [int(rng.integers(1, 5)) if rng.random() < 0.3 else int(rng.integers(2, 4))
             for _ in range(ndim)]
    if mx:
        shape[-1] = int(rng.integers(20, 90))
    dtype = "bf16" if mx else ["i32", "bf16", "u8"][int(rng.integers(3))]
    buffers = {}
    sides = {}
    for name in ("src", "dst"):
        mesh = synth.TINY_MESHES[int(rng.integers(len(synth.TINY_MESHES)))]
        # MXFP8: sources are not cut along the last dim (blocks from several
        # sources are covered by tests of their own)
        top = ndim - 1 if (mx and name == "src") else ndim
        pl = [int(rng.integers(-1, top)) for _ in mesh]
        sd = synth.side(mesh, pl)
        quant = "mxfp8" if (mx and name == "dst") else None
        sd["quant"] = quant
        if rng.random() < 0.8:
            desc = {"shape": shape, "dtype": dtype, "mesh": mesh, "placements": pl,
                    "slot_of_coord": None, "quant": quant}
            slots, sslots = [], []
            for k, (_, ln) in enumerate(olayout.slot_boxes(desc)):
                for kind, last in (("e", ln[-1]), ("s", -(-ln[-1] // 32))):
                    if kind == "s" and not quant:
                        continue
                    dims = list(ln[:-1]) + [last]
                    pad = [int(rng.integers(1, 3)) for _ in dims]
                    pad[-1] = 0 if mx else pad[-1]   # MXFP8: contiguous last dim
                    st, acc = [], 1
                    for n, p in zip(reversed(dims), reversed(pad)):
                        st.append(acc)
                        acc *= max(n + p, 1)
                    st = list(reversed(st))
                    base = int(rng.integers(0, 5))
                    key = "%s%s%d" % (name, kind, k)
                    bdt = "u8" if (quant or kind == "s") else dtype
                    buffers[key] = {"dtype": bdt, "elems": base + acc}
                    (slots if kind == "e" else sslots).append({"buf": key, "view": (base, st)})
            sd["slots"] = slots
            if quant:
                sd["scale_slots"] = sslots
        sides[name] = sd
    return {"name": "high_rank_%d" % seed, "buffers": buffers,
            "tensors": [{"name": "t", "shape": shape, "dtype": dtype, "src": sides["src"],
                         "dst": sides["dst"],
                         "values": {"kind": "normal", "std": 1.0, "seed": seed} if mx
                         else {"kind": "index"}}]}


def random_plan_case(seed, max_bytes=3 << 20):
    """A seeded random plan: 1 to 3 tensors in one plan (so launches share
    the pointer pool and several buckets run in one execute), ranks 1-4,
    u8 / bf16 / i32 / f64, 4 KB to max_bytes (3 MB) each, meshes of 1-2 dims with 1-4
    slots per dim, Shard / Replicate placements, sides held as padded views
    into shared buffers at random, a fifth of the tensors installed as MXFP8;
    random planning options (fan-out, unit, tiny and thin thresholds) and
    pointer offsets.  Returns (workload, plan options, (src_shift,
    dst_shift))."""
    rng = np.random.Generator(np.random.PCG64(90_000 + seed))
    buffers, tensors = {}, []
    any_mx = False
    for ti in range(int(rng.integers(1, 4))):
        mx = rng.random() < 0.2
        ndim = int(rng.integers(2 if mx else 1, 5))
        dtype = "bf16" if mx else ["u8", "bf16", "i32", "f64"][int(rng.integers(4))]
        es = synth.ELEM_BYTES[dtype]
        last_bytes = int(rng.choice([2, 8, 24, 64, 130, 512, 1030, 4096, 9000, 20000]))
        last = max(1, last_bytes // es)
        if mx:
            last = max(last, int(rng.integers(20, 300)))
        total = int(rng.integers(4096, max_bytes)) // es
        rest = max(1, total // last)
        shape = [last]
        for _ in range(ndim - 2):
            k = int(rng.integers(1, 6))
            shape.insert(0, k)
            rest = max(1, rest // k)
        if ndim >= 2:
            shape.insert(0, rest)
        sides = {}
        for name in ("src", "dst"):
            mesh = [int(rng.integers(1, 5)) for _ in range(int(rng.integers(1, 3)))]
            top = ndim - 1 if (mx and name == "src") else ndim
            pl = [int(rng.integers(-1, top)) for _ in mesh]
            quant = "mxfp8" if (mx and name == "dst") else None
            sd = synth.side(mesh, pl, quant=quant)
            if rng.random() < 0.3:
                desc = {"shape": shape, "dtype": "u8" if quant else dtype, "mesh": mesh,
                        "placements": pl, "slot_of_coord": None, "quant": quant}
                slots, sslots = [], []
                for k, (_, ln) in enumerate(olayout.slot_boxes(desc)):
                    for kind, lastn in (("e", ln[-1]), ("s", -(-ln[-1] // 32))):
                        if kind == "s" and not quant:
                            continue
                        dims = list(ln[:-1]) + [lastn]
                        pad = [int(rng.integers(0, 3)) for _ in dims]
                        if mx:
                            pad[-1] = 0
                        st, acc = [], 1
                        for n, p in zip(reversed(dims), reversed(pad)):
                            st.append(acc)
                            acc *= max(n + p, 1)
                        st = list(reversed(st))
                        base = int(rng.integers(0, 9))
                        key = "t%d%s%s%d" % (ti, name, kind, k)
                        buffers[key] = {"dtype": "u8" if (quant or kind == "s") else dtype,
                                        "elems": base + acc}
                        (slots if kind == "e" else sslots).append({"buf": key, "view": (base, st)})
                sd["slots"] = slots
                if quant:
                    sd["scale_slots"] = sslots
            sides[name] = sd
        any_mx |= mx
        vals = {"kind": "normal", "std": 1.0, "seed": seed * 10 + ti} if dtype == "bf16" else \
            {"kind": "index"}
        tensors.append({"name": "t%d" % ti, "shape": shape, "dtype": dtype, "src": sides["src"],
                        "dst": sides["dst"], "values": vals})
    opts = {"fanout": bool(rng.random() < 0.8),
            "unit_bytes": int(rng.choice([4096, 8192, 16384, 65536])),
            "tiny_bytes": int(rng.choice([0, 256, 1024, 4096])),
            "thin_bytes": int(rng.choice([1, 64, 128, 512, 2048]))}
    shifts = [int(rng.choice([0, 0, 2, 6, 8, 10])) for _ in range(2)]
    return ({"name": "random_plan_%d" % seed, "buffers": buffers, "tensors": tensors}, opts,
            tuple(shifts))
