"""Golden reshard: assemble the full tensor, then slice every destination.

Oracle; test infrastructure only.  This is the debugging transport of
"NCCL Reshard Refit (Experimental)", section "xferdtensor Transports": every
destination receives the whole tensor and keeps its own part, which the page
says guarantees functionally correct output.  The shard-to-shard method
("Recasting refit as a DTensor-to-DTensor transfer" in the news summary of
NVIDIA's Reshard announcement; the 8x8 row-shards to column-shards example
there) must give the same destination bytes.

Buffers are host byte images (numpy uint8).  A shard lives in its buffer
through a view: (base, strides), both in elements of the tensor's dtype;
None means a dense row-major array of the shard's local shape at offset 0.
A shard may instead be held as "parts", one buffer per index of its first
dimension (per expert, say); the view then describes every part, with the
first stride unused.
The copy is bitwise: elements are handled as unsigned integers of the same
width, so NaN payloads and signed zeros survive.

Fused destinations (gate and up projections packed into one buffer, the
"slice of a fused vLLM tensor" case of "Execution Flow: Setup Time") are two
tensors whose slot k views point into the same buffer at different bases; the
oracle simply writes both through their views into that one image.

MXFP8 destinations (bf16 source, quantised on install, "Enabling It") take an
element buffer and a scale buffer per slot, each with its own view; the scale
view indexes [..., ceil(K/32)] where K is the shard's last local extent.
"""

import numpy as np
from numpy.lib.stride_tricks import as_strided

from . import layout
from . import mxfp8

ELEM_BYTES = {
    "u8": 1, "i8": 1,
    "u16": 2, "i16": 2, "bf16": 2, "f16": 2,
    "u32": 4, "i32": 4, "f32": 4,
    "u64": 8, "i64": 8, "f64": 8,
}
UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def dense_strides(lengths):
    st = [0] * len(lengths)
    acc = 1
    for d in range(len(lengths) - 1, -1, -1):
        st[d] = acc
        acc *= lengths[d]
    return st


def view_array(buf, esize, view, lengths, writeable=False):
    """Array of shape `lengths` over byte image `buf` through `view`."""
    if view is None:
        base, strides = 0, dense_strides(lengths)
    else:
        base, strides = view
    arr = buf.view(UINT[esize])
    if any(n == 0 for n in lengths):
        return np.zeros(lengths, dtype=UINT[esize])
    last = base + sum((n - 1) * s for n, s in zip(lengths, strides))
    if base < 0 or last >= arr.size or min(strides, default=0) < 0:
        raise ValueError("view does not fit its buffer")
    return as_strided(arr[base:], shape=tuple(lengths),
                      strides=tuple(s * esize for s in strides),
                      writeable=writeable)


def _part_view(view):
    """View of one part of a shard held as one buffer per dim-0 index: the
    same base, the strides of dims 1.. (None stays dense)."""
    if view is None:
        return None
    return view[0], list(view[1])[1:]


def read_shard(entry, esize, lengths, buf_key="buf", parts_key="parts", view_key="view"):
    """The local array of a shard from its buffer (or from its parts)."""
    if parts_key in entry:
        out = np.zeros(lengths, dtype=UINT[esize])
        for i0, part in enumerate(entry[parts_key]):
            out[i0] = view_array(part, esize, _part_view(entry.get(view_key)), lengths[1:])
        return out
    return view_array(entry[buf_key], esize, entry.get(view_key), lengths)


def write_shard(entry, esize, lengths, V, buf_key="buf", parts_key="parts", view_key="view"):
    """Write the local array V of a shard through its view (or into its parts)."""
    if parts_key in entry:
        for i0, part in enumerate(entry[parts_key]):
            view_array(part, esize, _part_view(entry.get(view_key)), lengths[1:],
                       writeable=True)[...] = V[i0]
        return
    view_array(entry[buf_key], esize, entry.get(view_key), lengths, writeable=True)[...] = V


def box_slices(box):
    off, ln = box
    return tuple(slice(o, o + n) for o, n in zip(off, ln))


def assemble(src_desc, esize, src_bufs):
    """Full tensor from the source shards.

    src_bufs[s] = {"buf": uint8 array, "view": view or None}.  Every element
    must be supplied, and replicas must agree bitwise (the Reshard page:
    replication means the same data is available from several sources).
    """
    shape = list(src_desc["shape"])
    G = np.zeros(shape, dtype=UINT[esize])
    seen = np.zeros(shape, dtype=bool)
    for s, box in enumerate(layout.slot_boxes(src_desc)):
        if layout.box_volume(box) == 0:
            continue
        part = read_shard(src_bufs[s], esize, box[1])
        sl = box_slices(box)
        prev = seen[sl]
        if prev.any() and not np.array_equal(G[sl][prev], part[prev]):
            raise AssertionError("source replicas disagree at slot %d" % s)
        G[sl] = part
        seen[sl] = True
    if not seen.all():
        raise AssertionError("source shards do not cover the tensor")
    return G


def reshard(src_desc, dst_desc, src_bufs, dst_bufs, map_fn=None):
    """Write every destination shard through its view(s) into dst_bufs.

    dst_bufs[k] = {"buf": uint8 array, "view": ...} and, when
    dst_desc["quant"] == "mxfp8", also {"scale_buf": ..., "scale_view": ...}.
    The images are modified in place; bytes outside the views are left as
    they were given.

    map_fn (default: the built-in map) applies the per-destination step to
    every destination slot; a thread pool's map runs slots concurrently
    (each slot writes only its own views).
    """
    if list(src_desc["shape"]) != list(dst_desc["shape"]):
        raise ValueError("global shapes differ")
    esize = ELEM_BYTES[src_desc["dtype"]]
    quant = dst_desc.get("quant")
    G = assemble(src_desc, esize, src_bufs)

    def one(kb):
        _install(G, esize, quant, src_desc, dst_desc, kb[0], kb[1], dst_bufs)
    list((map_fn or map)(one, enumerate(layout.slot_boxes(dst_desc))))


def _install(G, esize, quant, src_desc, dst_desc, k, box, dst_bufs):
    """Destination slot k: its box of G, quantised if asked, written through
    its view(s)."""
    ln = box[1]
    if layout.box_volume(box) > 0:
        V = np.ascontiguousarray(G[box_slices(box)])
        if quant is None:
            if ELEM_BYTES[dst_desc["dtype"]] != esize:
                raise ValueError("element sizes differ")
            write_shard(dst_bufs[k], esize, ln, V)
        elif quant == "mxfp8":
            if src_desc["dtype"] != "bf16":
                raise ValueError("mxfp8 install needs a bf16 source")
            codes, scales = mxfp8.quantize(V)
            write_shard(dst_bufs[k], 1, ln, codes)
            sln = list(ln[:-1]) + [-(-ln[-1] // mxfp8.BLOCK)]
            write_shard(dst_bufs[k], 1, sln, scales, buf_key="scale_buf",
                        parts_key="scale_parts", view_key="scale_view")
        else:
            raise ValueError("unknown quant mode %r" % (quant,))


# ---------------------------------------------------------------------------
# Sampled evaluation, for sizes where assembling the full tensor on the host
# is too costly: the expected value of one destination element is the value
# of the same global element in any source shard that holds it.
# ---------------------------------------------------------------------------

def source_location(src_desc, g):
    """(slot, local index) of the first source slot whose box holds global g."""
    for s, (off, ln) in enumerate(layout.slot_boxes(src_desc)):
        if all(o <= x < o + n for x, o, n in zip(g, off, ln)):
            return s, [x - o for x, o in zip(g, off)]
    raise AssertionError("no source shard holds %r" % (g,))


def element_offset(view, lengths, local):
    """Element offset of a local index inside its buffer through a view."""
    if view is None:
        base, strides = 0, dense_strides(lengths)
    else:
        base, strides = view
    return base + sum(i * s for i, s in zip(local, strides))


def expected_sources(src_desc, src_views, dst_desc, dst_slot, locals_):
    """For each destination-local index, where its value lives among the sources.

    Returns a list of (source slot, element offset in that slot's buffer).
    `src_views[s]` is the view of source slot s (None = dense).
    """
    sboxes = layout.slot_boxes(src_desc)
    doff, _ = layout.slot_boxes(dst_desc)[dst_slot]
    out = []
    for l in locals_:
        g = [a + b for a, b in zip(doff, l)]
        s, sl = source_location(src_desc, g)
        out.append((s, element_offset(src_views[s], sboxes[s][1], sl)))
    return out
