"""Test-side glue between synthetic workloads and the library binding.

`interpret` walks a plan's region table on the host with numpy copies.  It is
test code only: it checks the planner's geometry on the CPU against the
oracle; the product never executes a plan anywhere but in its HIP kernels.
"""

import numpy as np

from oracle import mxfp8 as omx
from rl_weight_refit_amd import binding


def spec(tensor, side_name):
    s = tensor[side_name]
    dtype = tensor["dtype"]
    if side_name == "dst" and s.get("quant") == "mxfp8":
        dtype = "u8"
    views = None if s["slots"] is None else [e["view"] for e in s["slots"]]
    sviews = None
    if s.get("scale_slots") is not None:
        sviews = [e["view"] for e in s["scale_slots"]]
    return {"shape": tensor["shape"], "dtype": dtype, "mesh": s["mesh"],
            "placements": s["placements"], "slot_of_coord": s.get("slot_of_coord"),
            "views": views, "quant": s.get("quant") if side_name == "dst" else None,
            "scale_views": sviews, "split0": s.get("split0", False),
            "scale_of": tensor.get("scale_of") if side_name == "src" else None,
            "scale_block": tensor.get("scale_block")}


def plan_workload(workload, **kw):
    src = [spec(t, "src") for t in workload["tensors"]]
    dst = [spec(t, "dst") for t in workload["tensors"]]
    return binding.reshard_plan(src, dst, **kw)


def flat_lists(workload, sources, per_tensor_dst):
    """Pointer-order lists: sources tensor by tensor; destinations tensor by
    tensor (element buffers, then scale buffers for MXFP8 tensors)."""
    src_flat, dst_flat = [], []
    for t, src, dst in zip(workload["tensors"], sources, per_tensor_dst):
        for e in src:
            src_flat += e["parts"] if "parts" in e else [e["buf"]]
        for e in dst:
            dst_flat += e["parts"] if "parts" in e else [e["buf"]]
        if t["dst"].get("quant") == "mxfp8":
            for e in dst:
                dst_flat += e["scale_parts"] if "scale_parts" in e else [e["scale_buf"]]
    return src_flat, dst_flat


def _row_offsets(ext, stride):
    e0, e1, e2 = [int(x) for x in ext]
    i0 = np.arange(e0, dtype=np.int64)
    i1 = np.arange(e1, dtype=np.int64)
    i2 = np.arange(e2, dtype=np.int64)
    off = (i2[:, None, None] * int(stride[2]) + i1[None, :, None] * int(stride[1])
           + i0[None, None, :] * int(stride[0]))
    return off.reshape(-1)


def interpret(plan, src_flat, dst_flat, count=None):
    """Execute a plan's regions on host byte images.  If `count` is given
    (a list parallel to dst_flat of int arrays), bump a per-byte write count."""
    for r in plan.regions():
        so = _row_offsets(r["ext"], r["src_stride"]) + r["src_off"]
        do = _row_offsets(r["ext"], r["dst_stride"]) + r["dst_off"]
        inner = int(r["inner"])
        src = src_flat[r["src_index"]]
        if r["bucket"] != "mx":
            idx_s = so[:, None] + np.arange(inner)[None, :]
            data = src[idx_s]
            for j in r["dst_index"]:
                idx_d = do[:, None] + np.arange(inner)[None, :]
                dst_flat[j][idx_d] = data
                if count is not None:
                    np.add.at(count[j], idx_d.reshape(-1), 1)
        else:
            # Columns [0, split) from the source, [split, inner) from the
            # second piece (a block two source shards share).
            split = int(r["split"])
            idx_s = so[:, None] + np.arange(2 * split)[None, :]
            raw = src[idx_s]
            if split < inner:
                so2 = _row_offsets(r["ext"], r["src2_stride"]) + r["src2_off"]
                idx2 = so2[:, None] + np.arange(2 * (inner - split))[None, :]
                raw = np.concatenate([raw, src_flat[r["src2_index"]][idx2]], axis=1)
            bits = raw.reshape(len(so), inner, 2).copy().view(np.uint16)[..., 0]
            codes, scales = omx.quantize(bits)
            co = _row_offsets(r["ext"], r["scale_stride"]) + r["scale_off"]
            nb = scales.shape[1]
            for j, sj in zip(r["dst_index"], r["scale_index"]):
                idx_d = do[:, None] + np.arange(inner)[None, :]
                dst_flat[j][idx_d] = codes
                idx_c = co[:, None] + np.arange(nb)[None, :] * int(r["scale_inner_stride"])
                dst_flat[sj][idx_c] = scales
                if count is not None:
                    np.add.at(count[j], idx_d.reshape(-1), 1)
                    np.add.at(count[sj], idx_c.reshape(-1), 1)
