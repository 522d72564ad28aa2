"""Python binding of libreshard.so (ctypes): argument marshalling only.

Every step of the relayout runs in the library (planning on the CPU, copies
and MXFP8 installation in HIP kernels).  This module only converts plain
descriptions into the C structs of include/reshard.h, passes device pointers
and the HIP stream through, and turns error codes into exceptions.  If the
library has not been built, loading fails loudly; there is no fallback.

A side description is a dict:
  shape, dtype ("u8", "bf16", "f32", ...), mesh, placements (d >= 0 Shard(d),
  -1 Replicate), and optionally slot_of_coord, views (per slot (base,
  strides) in elements, or None for all-dense), quant ("mxfp8" on a
  destination), scale_views, split0 (one buffer per local dim-0 index), and
  scale_of / scale_block (this tensor holds the block scales of tensor
  scale_of of the same plan).
"""

import array
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libreshard.so")

RS_MAX_DIMS = 8
RS_MAX_MESH = 4
RS_MAX_FANOUT = 16

DTYPES = {"u8": 1, "i8": 2, "u16": 3, "i16": 4, "bf16": 5, "f16": 6,
          "u32": 7, "i32": 8, "f32": 9, "u64": 10, "i64": 11, "f64": 12}
QUANT = {None: 0, "mxfp8": 1}
STATUS = {0: "RS_OK", 1: "RS_ERR_INVALID", 2: "RS_ERR_MISMATCH", 3: "RS_ERR_UNSUPPORTED",
          4: "RS_ERR_ALLOC", 5: "RS_ERR_HIP"}
BUCKETS = ("bulk", "thin", "tiny", "mx")

c_i32, c_i64, c_u32, c_u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64


class View(ctypes.Structure):
    _fields_ = [("base", c_i64), ("strides", c_i64 * RS_MAX_DIMS)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("ndim", c_i32), ("dtype", c_i32), ("global_shape", c_i64 * RS_MAX_DIMS),
                ("mesh_ndim", c_i32), ("placements", c_i32 * RS_MAX_MESH),
                ("mesh_shape", c_i64 * RS_MAX_MESH),
                ("slot_of_coord", ctypes.POINTER(c_i32)), ("views", ctypes.POINTER(View)),
                ("quant", c_i32), ("scale_views", ctypes.POINTER(View)),
                ("split_dim0", c_i32), ("scale_of", c_i32), ("scale_block", c_i32 * RS_MAX_DIMS)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("struct_size", c_u32), ("fanout", c_u32), ("unit_bytes", c_u64),
                ("tiny_bytes", c_u32), ("thin_bytes", c_u32), ("reserved", c_u32 * 4)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tensors", c_u64), ("n_src_ptrs", c_u64), ("n_dst_ptrs", c_u64),
                ("n_regions", c_u64), ("n_regions_bucket", c_u64 * 4),
                ("n_units_bucket", c_u64 * 4), ("n_launches", c_u64), ("bytes_read", c_u64),
                ("bytes_written", c_u64), ("bytes_read_no_fanout", c_u64), ("plan_ns", c_u64),
                ("n_launches_pooled", c_u64)]


class Region(ctypes.Structure):
    _fields_ = [("tensor", c_u32), ("bucket", c_u32), ("src_index", c_u32), ("n_dst", c_u32),
                ("dst_index", c_u32 * RS_MAX_FANOUT), ("scale_index", c_u32 * RS_MAX_FANOUT),
                ("src_off", c_u64), ("dst_off", c_u64), ("scale_off", c_u64), ("inner", c_u64),
                ("ext", c_u64 * 3), ("src_stride", c_u64 * 3), ("dst_stride", c_u64 * 3),
                ("scale_stride", c_u64 * 3), ("scale_inner_stride", c_u64),
                ("split", c_u64), ("src2_index", c_u32), ("reserved0", c_u32), ("src2_off", c_u64),
                ("src2_stride", c_u64 * 3)]


class ReshardError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__("%s: %s" % (STATUS.get(status, status), message.strip()))


_lib = None


def load():
    """Load libreshard.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libreshard.so is not built (expected at %s); run "
                           "python -m rl_weight_refit_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.reshard_plan.argtypes = [ctypes.POINTER(TensorDesc), ctypes.POINTER(TensorDesc), c_i32,
                                 ctypes.POINTER(PlanOpts), ctypes.POINTER(P)]
    lib.reshard_plan.restype = c_i32
    lib.reshard_execute.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P), P]
    lib.reshard_execute.restype = c_i32
    lib.reshard_execute_no_alloc.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P), P]
    lib.reshard_execute_no_alloc.restype = c_i32
    lib.reshard_plan_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.reshard_plan_info.restype = c_i32
    lib.reshard_plan_region.argtypes = [P, c_u64, ctypes.POINTER(Region)]
    lib.reshard_plan_region.restype = c_i32
    lib.reshard_shard_box.argtypes = [ctypes.POINTER(TensorDesc), c_i64,
                                      ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]
    lib.reshard_shard_box.restype = c_i32
    lib.reshard_plan_destroy.argtypes = [P]
    lib.reshard_plan_destroy.restype = None
    lib.reshard_last_error.argtypes = []
    lib.reshard_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise ReshardError(status, load().reshard_last_error().decode())


def _views(vs, ndim):
    if vs is None:
        return None
    arr = (View * len(vs))()
    for i, v in enumerate(vs):
        base, strides = v
        arr[i].base = int(base)
        for d in range(ndim):
            arr[i].strides[d] = int(strides[d])
    return arr


def make_desc(spec):
    """C description of one side; returns (TensorDesc, objects to keep alive).
    The C side reads one entry per mesh slot from slot_of_coord, views and
    scale_views, so their lengths are checked here."""
    d = TensorDesc()
    shape = list(spec["shape"])
    mesh = list(spec["mesh"])
    if len(spec["placements"]) != len(mesh):
        raise ValueError("%d placements for a %d-dim mesh" % (len(spec["placements"]), len(mesh)))
    if len(shape) > RS_MAX_DIMS or len(mesh) > RS_MAX_MESH:
        raise ValueError("rank %d / mesh rank %d above the limits %d / %d"
                         % (len(shape), len(mesh), RS_MAX_DIMS, RS_MAX_MESH))
    nslots = 1
    for m in mesh:
        nslots *= int(m)
    for key in ("slot_of_coord", "views", "scale_views"):
        if spec.get(key) is not None and len(spec[key]) != nslots:
            raise ValueError("%s has %d entries for %d mesh slots" % (key, len(spec[key]), nslots))
    d.ndim = len(shape)
    d.dtype = DTYPES[spec["dtype"]]
    for i, n in enumerate(shape):
        d.global_shape[i] = int(n)
    d.mesh_ndim = len(mesh)
    for i, (m, p) in enumerate(zip(mesh, spec["placements"])):
        d.mesh_shape[i] = int(m)
        d.placements[i] = int(p)
    keep = []
    soc = spec.get("slot_of_coord")
    if soc is not None:
        arr = (c_i32 * len(soc))(*[int(x) for x in soc])
        keep.append(arr)
        d.slot_of_coord = ctypes.cast(arr, ctypes.POINTER(c_i32))
    v = _views(spec.get("views"), d.ndim)
    if v is not None:
        keep.append(v)
        d.views = ctypes.cast(v, ctypes.POINTER(View))
    d.quant = QUANT[spec.get("quant")]
    d.split_dim0 = 1 if spec.get("split0") else 0
    so = spec.get("scale_of")
    if so is not None:
        d.scale_of = int(so) + 1
        for i, b in enumerate(spec["scale_block"]):
            d.scale_block[i] = int(b)
    sv = _views(spec.get("scale_views"), d.ndim)
    if sv is not None:
        keep.append(sv)
        d.scale_views = ctypes.cast(sv, ctypes.POINTER(View))
    return d, keep


class Plan:
    """An immutable plan (owns the C handle)."""

    def __init__(self, handle):
        self._h = ctypes.c_void_p(handle)
        info = self.info()
        self.n_src_ptrs, self.n_dst_ptrs = info["n_src_ptrs"], info["n_dst_ptrs"]

    @property
    def handle(self):
        return self._h

    def info(self):
        out = PlanInfo()
        _check(load().reshard_plan_info(self._h, ctypes.byref(out)))
        return {"n_tensors": out.n_tensors, "n_src_ptrs": out.n_src_ptrs,
                "n_dst_ptrs": out.n_dst_ptrs, "n_regions": out.n_regions,
                "regions": dict(zip(BUCKETS, list(out.n_regions_bucket))),
                "units": dict(zip(BUCKETS, list(out.n_units_bucket))),
                "n_launches": out.n_launches, "bytes_read": out.bytes_read,
                "bytes_written": out.bytes_written,
                "bytes_read_no_fanout": out.bytes_read_no_fanout, "plan_ns": out.plan_ns,
                "n_launches_pooled": out.n_launches_pooled}

    def region(self, i):
        r = Region()
        _check(load().reshard_plan_region(self._h, i, ctypes.byref(r)))
        n = r.n_dst
        return {"tensor": r.tensor, "bucket": BUCKETS[r.bucket], "src_index": r.src_index,
                "dst_index": list(r.dst_index[:n]), "scale_index": list(r.scale_index[:n]),
                "src_off": r.src_off, "dst_off": r.dst_off, "scale_off": r.scale_off,
                "inner": r.inner, "ext": list(r.ext), "src_stride": list(r.src_stride),
                "dst_stride": list(r.dst_stride), "scale_stride": list(r.scale_stride),
                "scale_inner_stride": r.scale_inner_stride, "split": r.split,
                "src2_index": r.src2_index, "src2_off": r.src2_off,
                "src2_stride": list(r.src2_stride)}

    def regions(self):
        return [self.region(i) for i in range(self.info()["n_regions"])]

    def destroy(self):
        if self._h is not None and self._h.value:
            load().reshard_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def reshard_plan(src_specs, dst_specs, fanout=True, unit_bytes=16384, tiny_bytes=256,
                 thin_bytes=128):
    """Plan len(src_specs) tensor pairs into one region table."""
    lib = load()
    n = len(src_specs)
    if len(dst_specs) != n:
        raise ValueError("src_specs and dst_specs differ in length")
    keep = []
    S = (TensorDesc * max(n, 1))()
    D = (TensorDesc * max(n, 1))()
    for i in range(n):
        S[i], k1 = make_desc(src_specs[i])
        D[i], k2 = make_desc(dst_specs[i])
        keep += k1 + k2
    opts = PlanOpts(struct_size=ctypes.sizeof(PlanOpts), fanout=1 if fanout else 0,
                    unit_bytes=unit_bytes, tiny_bytes=tiny_bytes, thin_bytes=thin_bytes)
    h = ctypes.c_void_p()
    _check(lib.reshard_plan(S, D, n, ctypes.byref(opts), ctypes.byref(h)))
    return Plan(h.value)


def _ptr_array(ptrs):
    """(keep-alive buffer, void** view) of a pointer list (None or 0 = NULL)."""
    try:
        buf = array.array("Q", ptrs)
    except TypeError:
        buf = array.array("Q", [int(p) if p else 0 for p in ptrs])
    if not buf:
        buf = array.array("Q", [0])
    return buf, ctypes.cast(buf.buffer_info()[0], ctypes.POINTER(ctypes.c_void_p))


def reshard_execute(plan, src_ptrs, dst_ptrs, stream=None):
    """Enqueue the plan on a HIP stream (an int handle, e.g.
    torch.cuda.current_stream().cuda_stream; None = the default stream)."""
    if len(src_ptrs) != plan.n_src_ptrs or len(dst_ptrs) != plan.n_dst_ptrs:
        raise ValueError("the plan takes %d source and %d destination pointers, got %d and %d"
                         % (plan.n_src_ptrs, plan.n_dst_ptrs, len(src_ptrs), len(dst_ptrs)))
    s_keep, s = _ptr_array(src_ptrs)
    d_keep, d = _ptr_array(dst_ptrs)
    _check(load().reshard_execute(plan.handle, s, d, ctypes.c_void_p(stream or 0)))


def reshard_execute_no_alloc(plan, src_ptrs, dst_ptrs, stream=None):
    """reshard_execute without any device allocation: the plan's tables go
    through the library's static per-GPU table area (calls that overlap on
    one GPU race for it)."""
    if len(src_ptrs) != plan.n_src_ptrs or len(dst_ptrs) != plan.n_dst_ptrs:
        raise ValueError("the plan takes %d source and %d destination pointers, got %d and %d"
                         % (plan.n_src_ptrs, plan.n_dst_ptrs, len(src_ptrs), len(dst_ptrs)))
    s_keep, s = _ptr_array(src_ptrs)
    d_keep, d = _ptr_array(dst_ptrs)
    _check(load().reshard_execute_no_alloc(plan.handle, s, d, ctypes.c_void_p(stream or 0)))


def reshard_shard_box(spec, slot):
    """(offsets, lengths) of one slot's global box."""
    d, keep = make_desc(spec)
    off = (c_i64 * RS_MAX_DIMS)()
    ln = (c_i64 * RS_MAX_DIMS)()
    _check(load().reshard_shard_box(ctypes.byref(d), int(slot), off, ln))
    return list(off[:d.ndim]), list(ln[:d.ndim])


def reshard_last_error():
    return load().reshard_last_error().decode()
