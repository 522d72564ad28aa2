"""Shard boxes of a DTensor-style layout (oracle; test infrastructure only).

A layout is described the way the Reshard pages describe a DTensor: a global
shape, a device mesh and one placement per mesh dimension, each either
Replicate or Shard(d) ("Recasting refit as a DTensor-to-DTensor transfer" in
the news summary of NVIDIA's Reshard announcement; the per-parameter
global_shape / mesh / placements record in "NCCL Reshard Refit
(Experimental)", section "Execution Flow: Setup Time").

The pages do not say how an uneven split falls.  This oracle takes PyTorch
DTensor's Shard rule: the tensor dimension is cut with torch.chunk, i.e. chunk
size ceil(len / parts), so trailing chunks may be short or empty.  When several
mesh dimensions shard the same tensor dimension they are applied in mesh-dim
order, each one cutting the piece left by the previous one (lower mesh dim
outermost).

Descriptions are plain dicts:
  shape        list of global extents
  mesh         list of mesh extents
  placements   one int per mesh dim: d >= 0 is Shard(d), -1 is Replicate
  slot_of_coord  optional list, row-major mesh coordinate -> buffer slot
"""

import itertools

REPLICATE = -1


def chunk(length, parts, index):
    """torch.chunk-style piece `index` of `length` split into `parts`.

    Returns (start, size).  The chunk size is ceil(length / parts); pieces past
    the end are empty.
    """
    if parts <= 0:
        raise ValueError("parts must be positive")
    size = -(-length // parts) if length > 0 else 0
    start = min(index * size, length)
    stop = min((index + 1) * size, length)
    return start, stop - start


def mesh_coords(mesh):
    """All mesh coordinates in row-major order (last mesh dim fastest)."""
    return list(itertools.product(*[range(m) for m in mesh]))


def shard_box(shape, mesh, placements, coord):
    """Global (offsets, lengths) of the shard held at mesh coordinate `coord`."""
    off = [0] * len(shape)
    ln = list(shape)
    for i, p in enumerate(placements):
        if p == REPLICATE:
            continue
        a, n = chunk(ln[p], mesh[i], coord[i])
        off[p] += a
        ln[p] = n
    return off, ln


def num_slots(desc):
    n = 1
    for m in desc["mesh"]:
        n *= m
    return n


def slot_coords(desc):
    """List indexed by slot: the mesh coordinate that owns the slot."""
    coords = mesh_coords(desc["mesh"])
    soc = desc.get("slot_of_coord")
    if soc is None:
        return coords
    out = [None] * len(coords)
    for ci, c in enumerate(coords):
        out[soc[ci]] = c
    return out


def slot_boxes(desc):
    """List indexed by slot of (offsets, lengths) in global coordinates."""
    return [shard_box(desc["shape"], desc["mesh"], desc["placements"], c)
            for c in slot_coords(desc)]


def replication(desc):
    """Number of slots holding each element: product of Replicate mesh dims."""
    r = 1
    for m, p in zip(desc["mesh"], desc["placements"]):
        if p == REPLICATE:
            r *= m
    return r


def box_volume(box):
    v = 1
    for n in box[1]:
        v *= n
    return v
