"""Per-element ownership brute force (oracle; tiny cases only).

Test infrastructure only.  For every destination element it looks up, by
plain membership tests against every source box, which source shards hold the
same global element, and copies the value from the first of them.  It also
checks the counting facts the Reshard pages imply ("Recasting refit as a
DTensor-to-DTensor transfer": a destination shard may be assembled from parts
of several sources, and replication makes the same data available from
several sources): every global element is held by exactly r_src source slots
with equal values, and lies in exactly r_dst destination boxes.

It works on local arrays (one numpy array per slot, of the shard's local
shape), not on buffers and views, so it shares no path with golden.py.
"""

import itertools

import numpy as np

from . import layout


def _inside(g, box):
    off, ln = box
    return all(o <= x < o + n for x, o, n in zip(g, off, ln))


def reshard_local(src_desc, dst_desc, src_locals):
    """Destination local arrays from source local arrays, element by element."""
    shape = list(src_desc["shape"])
    sboxes = layout.slot_boxes(src_desc)
    dboxes = layout.slot_boxes(dst_desc)
    r_src = layout.replication(src_desc)
    r_dst = layout.replication(dst_desc)
    dtype = src_locals[0].dtype

    for g in itertools.product(*[range(n) for n in shape]):
        nd = sum(1 for b in dboxes if _inside(g, b))
        if nd != r_dst:
            raise AssertionError("element %r lies in %d destination boxes, expected %d"
                                 % (g, nd, r_dst))

    out = []
    for k, (doff, dln) in enumerate(dboxes):
        a = np.zeros(dln, dtype=dtype)
        for l in itertools.product(*[range(n) for n in dln]):
            g = tuple(o + i for o, i in zip(doff, l))
            owners = [s for s, b in enumerate(sboxes) if _inside(g, b)]
            if len(owners) != r_src:
                raise AssertionError("element %r held by %d sources, expected %d"
                                     % (g, len(owners), r_src))
            vals = []
            for s in owners:
                soff = sboxes[s][0]
                vals.append(src_locals[s][tuple(x - o for x, o in zip(g, soff))])
            if any(v != vals[0] for v in vals[1:]):
                raise AssertionError("source replicas disagree at %r" % (g,))
            a[l] = vals[0]
        out.append(a)
    return out
