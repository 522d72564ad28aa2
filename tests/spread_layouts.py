"""Layouts whose bulk regions take the copy kernel's spread-group paths
(shared by the planner checks on the CPU and the GPU parity tests).

A spread group is eight consecutive whole work units of one region whose
unit is a whole number of 1 KiB pieces.  Rows of whole pieces with two or
three outer dims take the per-wave path that advances row and outer indices
by carries; other rows with at most one outer dim take the per-lane path.
"""

from rl_weight_refit_amd import synth

VALS = {"kind": "normal", "std": 0.02, "seed": 51}


def rows_two_outer():
    """[16, 64, 512] bf16, experts split 2 ways -> rows split 2 ways: per
    region 8 experts x a 32 KiB run, i.e. 16 KiB rows, e0 = 2 per expert."""
    t = {"name": "w", "shape": [16, 64, 512], "dtype": "bf16", "src": synth.side([2], [0]),
         "dst": synth.side([2], [1]), "values": dict(VALS)}
    return {"name": "spread_rows_2", "buffers": {}, "tensors": [t]}


def rows_three_outer(replicas=1):
    """[8, 4, 64, 512] bf16, dim 0 split 2 ways -> dims 2 and 1 split on a
    2 x 2 mesh (times `replicas` destination replicas): 16 KiB rows with
    e0 = 2, e1 = 2, e2 = 4 (nothing merges)."""
    mesh, pl = ([2, 2], [2, 1]) if replicas == 1 else ([2, 2, replicas], [2, 1, -1])
    t = {"name": "w", "shape": [8, 4, 64, 512], "dtype": "bf16", "src": synth.side([2], [0]),
         "dst": synth.side(mesh, pl), "values": dict(VALS)}
    return {"name": "spread_rows_3x%d" % replicas, "buffers": {}, "tensors": [t]}


def rows_seven_pieces():
    """7 KiB rows (seven pieces each, so a wave's next piece is 4 rows and 4
    pieces on) with two outer dims: [6, 40, 7168] bf16, last dim split in
    two on the destination, whose expert pitch is padded by 64 elements."""
    E, R, C = 6, 40, 7168
    half = C // 2
    pitch = R * half + 64
    bufs, slots = {}, []
    for k in range(2):
        bufs["d/%d" % k] = {"dtype": "bf16", "elems": E * pitch}
        slots.append({"buf": "d/%d" % k, "view": (0, [pitch, half, 1])})
    t = {"name": "w", "shape": [E, R, C], "dtype": "bf16", "src": synth.side([2], [0]),
         "dst": synth.side([2], [2], slots=slots), "values": dict(VALS)}
    return {"name": "spread_rows_7", "buffers": bufs, "tensors": [t]}


def flat_short_rows(replicas=1):
    """768-byte rows with one outer dim: [800, 768] bf16, rows split 2 ways ->
    columns split 2 ways (times `replicas` destination replicas).  Units are
    sized to 20 rows (15 KiB, whole pieces); 400 rows per region make two
    whole groups and a four-unit tail."""
    mesh, pl = ([2], [1]) if replicas == 1 else ([2, replicas], [1, -1])
    t = {"name": "w", "shape": [800, 768], "dtype": "bf16", "src": synth.side([2], [0]),
         "dst": synth.side(mesh, pl), "values": dict(VALS)}
    return {"name": "spread_flat_768x%d" % replicas, "buffers": {}, "tensors": [t]}


ALL = {"rows_two_outer": rows_two_outer, "rows_three_outer": rows_three_outer,
       "rows_three_outer_fanout": lambda: rows_three_outer(3),
       "rows_seven_pieces": rows_seven_pieces, "flat_short_rows": flat_short_rows,
       "flat_short_rows_fanout": lambda: flat_short_rows(3)}


def random_case(seed):
    """Seeded random layouts with large regions for the spread paths: 2 to 4
    dims, 1 to 12 MB, a last dim of 16 B .. 20 KiB (16-byte multiples or
    not), source and destination meshes of 1 to 3 dims with Shard / Replicate
    placements (so rows, outer dims, uneven splits and replicas vary), bf16,
    f32 or u8 values."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(70_000 + seed))
    dtype = ["bf16", "f32", "u8"][int(rng.integers(3))]
    es = {"bf16": 2, "f32": 4, "u8": 1}[dtype]
    ndim = int(rng.integers(2, 5))
    last_bytes = int(rng.choice([16, 48, 512, 768, 1024, 1040, 2048, 3072, 4096, 7168, 8192,
                                 14336, 16384, 20480]))
    if rng.random() < 0.3:
        last_bytes += int(rng.integers(1, 16)) * es   # not a 16-byte multiple
    last = max(1, last_bytes // es)
    total = int(rng.integers(1 << 20, 12 << 20)) // es
    rest = max(1, total // last)
    shape = [last]
    for d in range(ndim - 2):
        k = int(rng.integers(2, 9))
        shape.insert(0, k)
        rest = max(1, rest // k)
    shape.insert(0, rest)

    def side_():
        mdim = int(rng.integers(1, 4))
        mesh = [int(rng.integers(1, 5)) for _ in range(mdim)]
        pl = [int(rng.integers(-1, ndim)) for _ in mesh]
        return synth.side(mesh, pl)
    t = {"name": "t", "shape": shape, "dtype": dtype, "src": side_(), "dst": side_(),
         "values": {"kind": "uniform", "seed": seed} if dtype != "u8" else {"kind": "index"}}
    return {"name": "spread_random_%d" % seed, "buffers": {}, "tensors": [t]}
