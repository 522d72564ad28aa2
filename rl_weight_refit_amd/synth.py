"""Seeded synthetic workloads for the relayout: layouts, buffers and values.

This module only describes inputs.  It holds none of the relayout's
arithmetic (no shard boxes, no intersections, no quantisation) and imports
nothing else from this package, so the tests can feed the same inputs to the
HIP path and to the independent CPU oracle.

A workload is a dict:

  {"name": str,
   "buffers": {key: {"dtype": str, "elems": int}},   # shared / fused buffers
   "tensors": [ {"name", "shape", "dtype",
                 "src": side, "dst": side,
                 "values": {"kind": "normal"|"uniform"|"index", ...}} ]}

and a side is

  {"mesh": [...], "placements": [...],     # d >= 0: Shard(d); -1: Replicate
   "slot_of_coord": None | [...],          # row-major mesh coord -> slot
   "slots": None | [ {"buf": key, "view": (base, strides)} per slot ],
   "quant": None | "mxfp8",
   "scale_slots": None | [ {"buf": key, "view": (base, strides)} per slot ]}

"slots": None means every slot is a dense buffer of its own, sized by its
local shard shape.  Fused gate/up destinations name the same buffer for the
gate and the up tensor's slot k, at different bases (gate first).

Values are the weights' stand-ins: the pages' workloads are trained FFN / MoE
weights, replaced here by N(0, 0.02) bf16 (or U[-1, 1) for the uneven
layouts, or the global linear index for the worked example and the tiny
cases).
"""

import numpy as np

R = -1  # Replicate

ELEM_BYTES = {"u8": 1, "u16": 2, "bf16": 2, "f16": 2, "i16": 2,
              "i32": 4, "u32": 4, "f32": 4, "i64": 8, "u64": 8, "f64": 8}


def side(mesh, placements, slots=None, slot_of_coord=None, quant=None, scale_slots=None,
         split0=False):
    return {"mesh": list(mesh), "placements": list(placements),
            "slot_of_coord": slot_of_coord, "slots": slots,
            "quant": quant, "scale_slots": scale_slots, "split0": split0}


def _row_major(shape):
    st, acc = [], 1
    for n in reversed(shape):
        st.append(acc)
        acc *= n
    return list(reversed(st))


def _prod(xs):
    p = 1
    for x in xs:
        p *= x
    return p


# ---------------------------------------------------------------------------
# The worked example: 8x8 int32, values i*8+j, two row shards -> four column
# shards.
# ---------------------------------------------------------------------------

def worked_example():
    return {"name": "worked_8x8", "buffers": {},
            "tensors": [{"name": "w", "shape": [8, 8], "dtype": "i32",
                         "src": side([2], [0]), "dst": side([4], [1]),
                         "values": {"kind": "index"}}]}


# ---------------------------------------------------------------------------
# Tiny random layouts: rank 1..3, extents 1..17, meshes up to 2x3, each mesh
# dim Replicate or Shard(d) uniformly; values = global linear index.
# ---------------------------------------------------------------------------

TINY_MESHES = [[1], [2], [3], [4], [5], [6], [1, 2], [2, 1], [1, 3], [3, 1],
               [2, 2], [2, 3], [3, 2]]


def _random_side(rng, ndim):
    mesh = TINY_MESHES[rng.integers(len(TINY_MESHES))]
    pl = [int(rng.integers(-1, ndim)) for _ in mesh]
    soc = None
    if rng.random() < 0.25:
        soc = [int(x) for x in rng.permutation(_prod(mesh))]
    return side(mesh, pl, slot_of_coord=soc)


def tiny_case(seed, dtype="i32"):
    rng = np.random.Generator(np.random.PCG64(seed))
    ndim = int(rng.integers(1, 4))
    shape = [int(rng.integers(1, 18)) for _ in range(ndim)]
    return {"name": "tiny_%d" % seed, "buffers": {},
            "tensors": [{"name": "t", "shape": shape, "dtype": dtype,
                         "src": _random_side(rng, ndim), "dst": _random_side(rng, ndim),
                         "values": {"kind": "index"}}]}


# ---------------------------------------------------------------------------
# Uneven layouts: [1000,3000] and [7,513,257] in f32 and bf16; sources over
# meshes [3] / [2,3], destinations over [7] / [4,2]; each mesh dim Shard(0),
# Shard(1) or Replicate; U[-1, 1) values.
# ---------------------------------------------------------------------------

UNEVEN_SHAPES = [[1000, 3000], [7, 513, 257]]
UNEVEN_SRC_MESHES = [[3], [2, 3]]
UNEVEN_DST_MESHES = [[7], [4, 2]]


def uneven_case(seed, shapes=None):
    rng = np.random.Generator(np.random.PCG64(10_000 + seed))
    shapes = shapes or UNEVEN_SHAPES
    shape = list(shapes[int(rng.integers(len(shapes)))])
    dtype = ["f32", "bf16"][int(rng.integers(2))]
    sm = UNEVEN_SRC_MESHES[int(rng.integers(2))]
    dm = UNEVEN_DST_MESHES[int(rng.integers(2))]
    choices = [0, 1, R]
    spl = [choices[int(rng.integers(3))] for _ in sm]
    dpl = [choices[int(rng.integers(3))] for _ in dm]
    return {"name": "uneven_%d" % seed, "buffers": {},
            "tensors": [{"name": "t", "shape": shape, "dtype": dtype,
                         "src": side(sm, spl), "dst": side(dm, dpl),
                         "values": {"kind": "uniform", "seed": seed}}]}


def reverse(workload):
    """The B -> A workload of an A -> B one (dense slots only)."""
    out = {"name": workload["name"] + "_rev", "buffers": dict(workload["buffers"]),
           "tensors": []}
    for t in workload["tensors"]:
        u = dict(t)
        u["src"], u["dst"] = t["dst"], t["src"]
        out["tensors"].append(u)
    return out


# ---------------------------------------------------------------------------
# FFN layers with fused gate/up destinations.
# ---------------------------------------------------------------------------

def dense_ffn(hidden=4096, inter=14336, src_tp=4, dst_tp=2, dst_dp=2, seed=1):
    """Dense FFN: gate/up [I,H] src TP Shard(0), down [H,I] src TP Shard(1) ->
    destination mesh [TP, DP] with Shard on TP and Replicate on DP; per
    destination slot gate and up share one buffer [2*ceil(I/TP), H], gate
    first, and down has a dense buffer of its own."""
    ip = -(-inter // dst_tp)
    ndst = dst_tp * dst_dp
    bufs = {"w13/%d" % k: {"dtype": "bf16", "elems": 2 * ip * hidden} for k in range(ndst)}
    st = _row_major([2 * ip, hidden])
    gate_slots = [{"buf": "w13/%d" % k, "view": (0, st)} for k in range(ndst)]
    up_slots = [{"buf": "w13/%d" % k, "view": (ip * hidden, st)} for k in range(ndst)]
    vals = lambda i: {"kind": "normal", "std": 0.02, "seed": seed * 1000 + i}
    return {"name": "dense_ffn_h%d_i%d" % (hidden, inter), "buffers": bufs,
            "tensors": [
                {"name": "gate", "shape": [inter, hidden], "dtype": "bf16",
                 "src": side([src_tp], [0]), "dst": side([dst_tp, dst_dp], [0, R], gate_slots),
                 "values": vals(0)},
                {"name": "up", "shape": [inter, hidden], "dtype": "bf16",
                 "src": side([src_tp], [0]), "dst": side([dst_tp, dst_dp], [0, R], up_slots),
                 "values": vals(1)},
                {"name": "down", "shape": [hidden, inter], "dtype": "bf16",
                 "src": side([src_tp], [1]), "dst": side([dst_tp, dst_dp], [1, R]),
                 "values": vals(2)},
            ]}


def moe_experts(experts, hidden, inter, src_ep, dst_ep, dst_tp, seed, quant=None,
                src_split=False):
    """Grouped MoE experts: gate/up [E,I,H], down [E,H,I]; source EP Shard(0)
    on the expert dim; destination mesh [EP, TP] with experts Shard(0) and the
    intermediate dim sharded on TP.  Per destination slot, gate and up share
    one w13 buffer [ceil(E/EP), 2*ceil(I/TP), H] (gate first); down goes to a
    w2 buffer [ceil(E/EP), H, ceil(I/TP)].

    quant="mxfp8": destinations hold E4M3 bytes, plus u8 scale buffers
    [.., ceil(K/32)] along each destination's last dim.

    src_split=True: every source expert is a buffer of its own (the training
    side's per-expert weights, before any stacking)."""
    el = -(-experts // dst_ep)
    ip = -(-inter // dst_tp)
    ndst = dst_ep * dst_tp
    edt = "u8" if quant == "mxfp8" else "bf16"
    bufs = {}
    w13_st = _row_major([el, 2 * ip, hidden])
    w2_st = _row_major([el, hidden, ip])
    for k in range(ndst):
        bufs["w13/%d" % k] = {"dtype": edt, "elems": el * 2 * ip * hidden}
        bufs["w2/%d" % k] = {"dtype": edt, "elems": el * hidden * ip}
    gate = [{"buf": "w13/%d" % k, "view": (0, w13_st)} for k in range(ndst)]
    up = [{"buf": "w13/%d" % k, "view": (ip * hidden, w13_st)} for k in range(ndst)]
    down = [{"buf": "w2/%d" % k, "view": (0, w2_st)} for k in range(ndst)]
    sg = su = sd = None
    if quant == "mxfp8":
        hb = -(-hidden // 32)
        ib = -(-ip // 32)
        s13 = _row_major([el, 2 * ip, hb])
        s2 = _row_major([el, hidden, ib])
        for k in range(ndst):
            bufs["s13/%d" % k] = {"dtype": "u8", "elems": el * 2 * ip * hb}
            bufs["s2/%d" % k] = {"dtype": "u8", "elems": el * hidden * ib}
        sg = [{"buf": "s13/%d" % k, "view": (0, s13)} for k in range(ndst)]
        su = [{"buf": "s13/%d" % k, "view": (ip * hb, s13)} for k in range(ndst)]
        sd = [{"buf": "s2/%d" % k, "view": (0, s2)} for k in range(ndst)]
    vals = lambda i: {"kind": "normal", "std": 0.02, "seed": seed * 1000 + i}
    mesh = [dst_ep, dst_tp]
    name = "moe_e%d_h%d_i%d_ep%d_to_ep%dxtp%d%s%s" % (experts, hidden, inter, src_ep, dst_ep,
                                                        dst_tp, "_mxfp8" if quant else "",
                                                        "_per_expert_src" if src_split else "")
    return {"name": name, "buffers": bufs,
            "tensors": [
                {"name": "gate", "shape": [experts, inter, hidden], "dtype": "bf16",
                 "src": side([src_ep], [0], split0=src_split),
                 "dst": side(mesh, [0, 1], gate, quant=quant, scale_slots=sg),
                 "values": vals(0)},
                {"name": "up", "shape": [experts, inter, hidden], "dtype": "bf16",
                 "src": side([src_ep], [0], split0=src_split),
                 "dst": side(mesh, [0, 1], up, quant=quant, scale_slots=su),
                 "values": vals(1)},
                {"name": "down", "shape": [experts, hidden, inter], "dtype": "bf16",
                 "src": side([src_ep], [0], split0=src_split),
                 "dst": side(mesh, [0, 2], down, quant=quant, scale_slots=sd),
                 "values": vals(2)},
            ]}


def moe_128e(quant=None):
    """128 experts, hidden 4096, expert intermediate 1536: EP8 -> EP4 x TP4."""
    return moe_experts(128, 4096, 1536, 8, 4, 4, seed=2, quant=quant)


def moe_dsv3(quant=None, src_split=False):
    """DeepSeek-V3-shaped MoE layer: 256 experts, hidden 7168, expert
    intermediate 2048 (gate + up + down = 22,548,578,304 bytes of bf16):
    EP16 -> EP8 x TP8."""
    return moe_experts(256, 7168, 2048, 16, 8, 8, seed=5, quant=quant, src_split=src_split)


def fp8_moe_experts(experts, hidden, inter, src_ep, dst_ep, dst_tp, seed, block=128,
                    src_split=False):
    """Blockwise-FP8 grouped MoE experts with their scale tensors: E4M3
    weight bytes gate/up [E,I,H], down [E,H,I] and float32 scales [E,
    ceil(I/block), ceil(H/block)] / [E, ceil(H/block), ceil(I/block)], each
    scale tensor on its weight's meshes and placements (source EP Shard(0) ->
    destination [EP, TP]).  Destinations: gate and up weights fused in w13
    (gate first), their scales fused in s13 the same way; down in w2 / s2."""
    el = -(-experts // dst_ep)
    ip = -(-inter // dst_tp)
    cb = lambda n: -(-n // block)
    ndst = dst_ep * dst_tp
    bufs = {}
    w13_st = _row_major([el, 2 * ip, hidden])
    w2_st = _row_major([el, hidden, ip])
    s13_st = _row_major([el, 2 * cb(ip), cb(hidden)])
    s2_st = _row_major([el, cb(hidden), cb(ip)])
    for k in range(ndst):
        bufs["w13/%d" % k] = {"dtype": "u8", "elems": el * 2 * ip * hidden}
        bufs["w2/%d" % k] = {"dtype": "u8", "elems": el * hidden * ip}
        bufs["s13/%d" % k] = {"dtype": "f32", "elems": el * 2 * cb(ip) * cb(hidden)}
        bufs["s2/%d" % k] = {"dtype": "f32", "elems": el * cb(hidden) * cb(ip)}
    mesh = [dst_ep, dst_tp]

    def w(name, shape, pl, slots, i):
        return {"name": name, "shape": shape, "dtype": "u8",
                "src": side([src_ep], [0], split0=src_split), "dst": side(mesh, pl, slots),
                "values": {"kind": "e4m3", "seed": seed * 1000 + i}}

    def sc(name, shape, pl, slots, of, i):
        t = {"name": name, "shape": shape, "dtype": "f32",
             "src": side([src_ep], [0]), "dst": side(mesh, pl, slots),
             "values": {"kind": "scale", "seed": seed * 1000 + i},
             "scale_of": of, "scale_block": [1, block, block]}
        return t

    slots = lambda key, base, st: [{"buf": "%s/%d" % (key, k), "view": (base, st)}
                                   for k in range(ndst)]
    tensors = [
        w("gate", [experts, inter, hidden], [0, 1], slots("w13", 0, w13_st), 0),
        w("up", [experts, inter, hidden], [0, 1], slots("w13", ip * hidden, w13_st), 1),
        w("down", [experts, hidden, inter], [0, 2], slots("w2", 0, w2_st), 2),
        sc("gate_scale_inv", [experts, cb(inter), cb(hidden)], [0, 1], slots("s13", 0, s13_st), 0, 3),
        sc("up_scale_inv", [experts, cb(inter), cb(hidden)], [0, 1],
           slots("s13", cb(ip) * cb(hidden), s13_st), 1, 4),
        sc("down_scale_inv", [experts, cb(hidden), cb(inter)], [0, 2], slots("s2", 0, s2_st), 2, 5),
    ]
    name = "fp8_moe_e%d_h%d_i%d_ep%d_to_ep%dxtp%d_b%d" % (experts, hidden, inter, src_ep, dst_ep,
                                                          dst_tp, block)
    return {"name": name, "buffers": bufs, "tensors": tensors}


# ---------------------------------------------------------------------------
# Misc-path packing: many small tensors into one contiguous buffer.
# ---------------------------------------------------------------------------

def misc_pack(layers=61, hidden=7168, q_rank=1536, kv_rank=512, experts=256, src_tp=4, seed=7,
              align=16):
    """The small per-layer tensors of a DeepSeek-V3-shaped model packed into
    one buffer, each at a running offset (aligned to `align` bytes): two
    RMSNorm weights [hidden], the q / kv low-rank norms [q_rank], [kv_rank]
    (bf16, replicated over the source TP ranks), the MoE router
    [experts, hidden] (bf16, row-sharded over TP) and its correction bias
    [experts] (f32, replicated).  The destination of every tensor is the one
    slot of mesh [1], viewed into the shared "pack" buffer."""
    specs = []
    for l in range(layers):
        specs += [("l%d.input_norm" % l, [hidden], "bf16", R),
                  ("l%d.post_attn_norm" % l, [hidden], "bf16", R),
                  ("l%d.q_a_norm" % l, [q_rank], "bf16", R),
                  ("l%d.kv_a_norm" % l, [kv_rank], "bf16", R),
                  ("l%d.router" % l, [experts, hidden], "bf16", 0),
                  ("l%d.router_bias" % l, [experts], "f32", R)]
    tensors, off = [], 0
    for i, (name, shape, dt, pl) in enumerate(specs):
        es = ELEM_BYTES[dt]
        off = -(-off // align) * align
        view = (off // es, _row_major(shape))
        kind = {"kind": "normal", "std": 0.02, "seed": seed * 100000 + i} if dt == "bf16" else \
            {"kind": "uniform", "seed": seed * 100000 + i}
        tensors.append({"name": name, "shape": shape, "dtype": dt,
                        "src": side([src_tp], [pl]),
                        "dst": side([1], [R], [{"buf": "pack", "view": view}]),
                        "values": kind})
        off += _prod(shape) * es
    return {"name": "misc_pack_%dlayers" % layers,
            "buffers": {"pack": {"dtype": "u8", "elems": -(-off // align) * align}},
            "tensors": tensors}


# ---------------------------------------------------------------------------
# Values.
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round-to-nearest-even bf16 bit patterns of finite float32 values
    (torch's CPU conversion, which rounds to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def host_values(tensor):
    """Global tensor values on the host, as unsigned-integer bit patterns."""
    shape = tensor["shape"]
    dt = tensor["dtype"]
    v = tensor["values"]
    es = ELEM_BYTES[dt]
    uint = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[es]
    if v["kind"] == "index":
        n = _prod(shape)
        return (np.arange(n, dtype=np.uint64) & np.uint64((1 << (8 * es)) - 1)) \
            .astype(uint).reshape(shape)
    rng = np.random.Generator(np.random.PCG64(v["seed"]))
    if v["kind"] == "e4m3":
        # random E4M3 bytes, the two NaN codes replaced by zero
        b = rng.integers(0, 256, size=shape, dtype=np.uint8)
        b[(b & 0x7F) == 0x7F] = 0
        return b
    if v["kind"] == "scale":
        # positive float32 block scales spread over a few binades
        x = np.exp2(rng.uniform(-12.0, -4.0, size=shape)).astype(np.float32)
        return x.view(np.uint32)
    if v["kind"] == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    elif v["kind"] == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x *= np.float32(v["std"])
    else:
        raise ValueError(v["kind"])
    if dt == "f32":
        return x.view(np.uint32)
    if dt == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError("no %s generator for dtype %s" % (v["kind"], dt))


def device_values(tensor, device):
    """Global tensor values generated on a torch device (for large sizes).

    N(0, std) values come from torch's generator seeded with the tensor's
    seed, drawn in float32 and rounded to bf16 by torch (round to nearest
    even).  Returns a torch tensor of the tensor's dtype.
    """
    import torch
    v = tensor["values"]
    g = torch.Generator(device=device)
    g.manual_seed(v["seed"])
    if v["kind"] == "e4m3":
        b = torch.randint(0, 256, tensor["shape"], generator=g, device=device, dtype=torch.int32)
        b = torch.where((b & 0x7F) == 0x7F, torch.zeros_like(b), b)
        return b.to(torch.uint8)
    if v["kind"] == "scale":
        x = torch.rand(tensor["shape"], generator=g, device=device, dtype=torch.float32)
        return torch.exp2(x * 8.0 - 12.0)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[tensor["dtype"]]
    if v["kind"] == "normal":
        x = torch.randn(tensor["shape"], generator=g, device=device, dtype=torch.float32)
        x.mul_(v["std"])
    elif v["kind"] == "uniform":
        x = torch.rand(tensor["shape"], generator=g, device=device, dtype=torch.float32)
        x.mul_(2.0).sub_(1.0)
    else:
        raise ValueError(v["kind"])
    return x.to(dt)
