#!/usr/bin/env python3
"""Benchmark of the single-GPU M->N relayout on the DeepSeek-V3-shaped MoE
layer: 256 experts, hidden 7168, expert intermediate 2048 (gate, up, down =
22,548,578,304 bytes of bf16), source EP16 Shard(0) -> destination EP8 x TP8
with fused gate/up (w13) destinations, N(0, 0.02) values generated on the
GPU.

One step = one pass of the whole path over that layer:
  1. the bf16 -> bf16 relayout (reshard_execute of the plain plan), and
  2. the BF16 -> MXFP8 install variant (reshard_execute of the MXFP8 plan).
Both plans are built once before timing (plans are reused across refits);
their CPU cost is reported separately as plan_us (p50 / p99 over 1000
calls).  Inputs are resident in HBM before the timed region.

Output: one JSON line.  value = algorithmic bytes (each needed source byte
read once + every destination byte written, both variants) per second of
the timed steps, in GB/s.  The roofline object is for the dominant kernel
(the bulk copy kernel of step 1), timed with HIP events on the stream it is
launched on.
"""

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "rs_bulk_kernel_moe_dsv3_counters.json")
PROFILE_COUNTERS_MX = os.path.join(ROOT, "profiles", "rs_mx_kernel_moe_dsv3_mxfp8_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "rl_weight_refit_amd", "csrc", f)
                  for f in ("kernels.hip", "rs_device.hpp")]


def kernel_hash():
    """Hash of the device code (kernels and the tables they read), comments
    and blank lines left out; counter profiles taken from other code are not
    reported as this kernel's."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1, help="must be 1: the relayout runs on one GPU")
    ap.add_argument("--steps", type=int, default=10, help="timed steps")
    ap.add_argument("--warmup", type=int, default=1, help="untimed steps before them")
    ap.add_argument("--variant", choices=["both", "copy", "mxfp8"], default="both",
                    help="what a step runs: the bf16 relayout, the MXFP8 install, or both")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other layouts")
    ap.add_argument("--plan-reps", type=int, default=1000, help="planner calls timed for plan_us")
    ap.add_argument("--ceiling-bytes", type=int, default=8 << 30,
                    help="size of the plain device copy timed as copy_ceiling_GBps")
    ap.add_argument("--ceiling-torch-only", action="store_true",
                    help="time only torch's copy for the ceiling (no launch of this library's kernels "
                         "outside the workload, e.g. for counter runs)")
    ap.add_argument("--poison-reps", type=int, default=5,
                    help="poison-filled reps per variant after the timed steps (0: none)")
    ap.add_argument("--procs", type=int, default=1,
                    help="run the bench in this many fresh processes and report their median")
    return ap.parse_args()


def run_processes(args):
    """Runs the bench in args.procs fresh child processes (this process never
    touches the GPU) and prints the median one's line, with every process's
    figures attached."""
    import subprocess
    argv = [a for a in sys.argv[1:]]
    lines = []
    for k in range(args.procs):
        print("process %d of %d ..." % (k + 1, args.procs), file=sys.stderr, flush=True)
        r = subprocess.run([sys.executable, os.path.abspath(__file__)] + argv + ["--procs", "1"],
                           stdout=subprocess.PIPE, text=True)
        if r.returncode != 0:
            return r.returncode
        lines.append(json.loads(r.stdout.strip().splitlines()[-1]))
    lines.sort(key=lambda d: d["value"])
    out = lines[len(lines) // 2]
    out["processes"] = {
        "n": len(lines),
        "value": [d["value"] for d in lines],
        "bf16_ms_median": [d["bf16"]["ms_median"] for d in lines if d.get("bf16")],
        "mxfp8_ms_median": [d["mxfp8"]["ms_median"] for d in lines if d.get("mxfp8")]}
    print(json.dumps(out), flush=True)
    return 0


def spec(tensor, side_name):
    s = tensor[side_name]
    dtype = tensor["dtype"]
    if side_name == "dst" and s.get("quant") == "mxfp8":
        dtype = "u8"
    return {"shape": tensor["shape"], "dtype": dtype, "mesh": s["mesh"],
            "placements": s["placements"], "slot_of_coord": s.get("slot_of_coord"),
            "views": None if s["slots"] is None else [e["view"] for e in s["slots"]],
            "quant": s.get("quant") if side_name == "dst" else None,
            "scale_views": None if s.get("scale_slots") is None
            else [e["view"] for e in s["scale_slots"]],
            "split0": s.get("split0", False),
            "scale_of": tensor.get("scale_of") if side_name == "src" else None,
            "scale_block": tensor.get("scale_block")}


def plan_of(binding, wl):
    return binding.reshard_plan([spec(t, "src") for t in wl["tensors"]],
                                [spec(t, "dst") for t in wl["tensors"]])


def plan_times(binding, wl, reps):
    src = [spec(t, "src") for t in wl["tensors"]]
    dst = [spec(t, "dst") for t in wl["tensors"]]
    ns = []
    for i in range(reps + 10):
        p = binding.reshard_plan(src, dst)
        if i >= 10:
            ns.append(p.info()["plan_ns"])
        p.destroy()
    ns.sort()
    return {"p50": ns[len(ns) // 2] / 1e3, "p99": ns[min(len(ns) - 1, int(len(ns) * 0.99))] / 1e3}


def device_sources(torch, binding, wl):
    """Source shards cut from the seeded device-generated global tensors, with
    the library's own shard boxes."""
    from rl_weight_refit_amd import synth
    out = []
    for t in wl["tensors"]:
        G = synth.device_values(t, "cuda")
        sp = spec(t, "src")
        nslots = int(np.prod(sp["mesh"]))
        shards = []
        for k in range(nslots):
            off, ln = binding.reshard_shard_box(sp, k)
            sl = tuple(slice(o, o + n) for o, n in zip(off, ln))
            if t["src"].get("split0"):
                part = G[sl]
                shards += [part[i].contiguous() for i in range(ln[0])]   # one buffer per expert
            else:
                shards.append(G[sl].contiguous())
        del G
        out.append(shards)
    torch.cuda.synchronize()
    return out


def device_destinations(torch, binding, wl):
    from rl_weight_refit_amd import synth
    named = {k: torch.empty(b["elems"] * synth.ELEM_BYTES[b["dtype"]], dtype=torch.uint8,
                            device="cuda") for k, b in wl["buffers"].items()}
    ptrs = []
    for t in wl["tensors"]:
        d = t["dst"]
        if d["slots"] is None:
            # Dense per-slot buffers, sized by the library's own shard boxes.
            sp = spec(t, "dst")
            es = synth.ELEM_BYTES[sp["dtype"]]
            for k in range(int(np.prod(d["mesh"]))):
                _, ln = binding.reshard_shard_box(sp, k)
                key = "%s/%d" % (t["name"], k)
                named[key] = torch.empty(max(1, int(np.prod(ln)) * es), dtype=torch.uint8,
                                         device="cuda")
                ptrs.append(named[key].data_ptr())
        else:
            ptrs += [named[e["buf"]].data_ptr() for e in d["slots"]]
        if d.get("quant") == "mxfp8" and d.get("scale_slots") is not None:
            ptrs += [named[e["buf"]].data_ptr() for e in d["scale_slots"]]
        elif d.get("quant") == "mxfp8":
            # Dense per-slot scale buffers: the slot's box with its last
            # extent in 32-element blocks.
            sp = spec(t, "dst")
            for k in range(int(np.prod(d["mesh"]))):
                _, ln = binding.reshard_shard_box(sp, k)
                nsc = int(np.prod(ln[:-1])) * (-(-ln[-1] // 32)) if ln else 0
                key = "%s/scale/%d" % (t["name"], k)
                named[key] = torch.empty(max(1, nsc), dtype=torch.uint8, device="cuda")
                ptrs.append(named[key].data_ptr())
    return named, ptrs


def copy_ceiling(torch, binding, nbytes, stream, library=True):
    """Plain contiguous device-to-device copies of nbytes, GB/s of read +
    write: torch's copy_ (best of 6) and this library's own copy of the
    same bytes as one region (identity layout, median of 10).  The ceiling
    is the faster of the two."""
    from rl_weight_refit_amd import synth
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    best = 0.0
    with torch.cuda.stream(stream):
        for _ in range(6):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            b.copy_(a)
            e1.record(stream)
            e1.synchronize()
            best = max(best, 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    lib = 0.0
    if library:
        t = {"name": "flat", "shape": [nbytes], "dtype": "u8", "src": synth.side([1], [-1]),
             "dst": synth.side([1], [-1]), "values": {"kind": "index"}}
        plan = binding.reshard_plan([spec(t, "src")], [spec(t, "dst")])
        ms = time_plan(torch, binding, plan, [a.data_ptr()], [b.data_ptr()], stream)
        plan.destroy()
        lib = 2 * nbytes / (ms * 1e-3) / 1e9
    del a, b
    return {"GBps": round(max(best, lib), 1), "torch_copy_GBps": round(best, 1),
            "library_copy_GBps": round(lib, 1), "bytes_each_way": nbytes}


_SWEEP = []


def cache_sweep(torch):
    """Reads 1 GiB (four times the 256 MB Infinity Cache): afterwards no cache
    holds a destination line, clean or dirty, so a timed rep neither finds
    its output cached nor pays for writing back a poison fill."""
    if not _SWEEP:
        _SWEEP.append(torch.ones(1 << 28, dtype=torch.float32, device="cuda"))
    _SWEEP[0].sum()


def time_plan(torch, binding, plan, src_ptrs, dst_ptrs, stream, reps=10, poison=()):
    """Median event-timed execute of a plan on `stream` (ms).  The buffers
    in `poison` are filled with 0xFF on the stream before every timed rep,
    and the caches swept, outside the timed events, so no rep finds the
    previous rep's output in a cache."""
    for _ in range(2):
        binding.reshard_execute(plan, src_ptrs, dst_ptrs, stream.cuda_stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        if poison:
            with torch.cuda.stream(stream):
                for t in poison:
                    t.fill_(0xFF)
                cache_sweep(torch)
        a.record(stream)
        binding.reshard_execute(plan, src_ptrs, dst_ptrs, stream.cuda_stream)
        b.record(stream)
    stream.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in evs)


def time_back_to_back(torch, binding, plan, src_ptrs, dst_ptrs, stream, reps=20):
    """Mean time of `reps` executes enqueued back to back between two events
    (ms): the steady state, where every execute also pays for the write-backs
    the previous one left in the caches."""
    for _ in range(2):
        binding.reshard_execute(plan, src_ptrs, dst_ptrs, stream.cuda_stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        binding.reshard_execute(plan, src_ptrs, dst_ptrs, stream.cuda_stream)
    b.record(stream)
    stream.synchronize()
    return a.elapsed_time(b) / reps


def secondary(torch, binding, stream):
    """Other layer-sized layouts and the kernels' special paths, measured
    after the timed region (not part of `value`)."""
    from rl_weight_refit_amd import synth
    out = {}
    for name, wl in (("dense_ffn_4096x14336_tp4_to_tp2xdp2", synth.dense_ffn()),
                     ("moe_128e_4096x1536_ep8_to_ep4xtp4", synth.moe_128e())):
        src = device_sources(torch, binding, wl)
        sp = [x.data_ptr() for t in src for x in t]
        named, dp = device_destinations(torch, binding, wl)
        plan = plan_of(binding, wl)
        info = plan.info()
        ms = time_plan(torch, binding, plan, sp, dp, stream, poison=list(named.values()))
        bb = time_back_to_back(torch, binding, plan, sp, dp, stream)
        nb = info["bytes_read"] + info["bytes_written"]
        nbf = info["bytes_read_no_fanout"] + info["bytes_written"]
        out[name] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1), "bytes": nb,
                     "bytes_no_fanout": nbf, "GBps_no_fanout_credit": round(nbf / ms / 1e6, 1),
                     "regions": info["n_regions"], "ms_back_to_back": round(bb, 4),
                     "GBps_back_to_back": round(nb / bb / 1e6, 1),
                     "plan_us": plan_times(binding, wl, 1000)}
        del src, named
    # The DSV3 layer with every source expert in a buffer of its own (no
    # stacking copy on the training side): 768 source pointers.
    wl = synth.moe_dsv3(src_split=True)
    src = device_sources(torch, binding, wl)
    sp = [x.data_ptr() for t in src for x in t]
    named, dp = device_destinations(torch, binding, wl)
    plan = plan_of(binding, wl)
    info = plan.info()
    ms = time_plan(torch, binding, plan, sp, dp, stream, poison=list(named.values()))
    nb = info["bytes_read"] + info["bytes_written"]
    out["moe_dsv3_per_expert_sources"] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1),
                                          "bytes": nb, "regions": info["n_regions"],
                                          "launches": info["n_launches"],
                                          "plan_us": info["plan_ns"] / 1e3}
    del src, named
    torch.cuda.empty_cache()
    # The DSV3 layer as blockwise-FP8 weights (E4M3 bytes) with their float32
    # 128 x 128 block scales, gate/up fused with their scales: 6 tensors.
    wl = synth.fp8_moe_experts(256, 7168, 2048, 16, 8, 8, seed=6)
    src = device_sources(torch, binding, wl)
    sp = [x.data_ptr() for t in src for x in t]
    named, dp = device_destinations(torch, binding, wl)
    plan = plan_of(binding, wl)
    info = plan.info()
    ms = time_plan(torch, binding, plan, sp, dp, stream, poison=list(named.values()))
    nb = info["bytes_read"] + info["bytes_written"]
    out["fp8_blockwise_dsv3_with_scales"] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1),
                                             "bytes": nb, "regions": info["regions"],
                                             "launches": info["n_launches"],
                                             "plan_us": info["plan_ns"] / 1e3}
    del src, named
    torch.cuda.empty_cache()
    # Misc-path packing: 61 layers of small tensors into one buffer, and back.
    wl = synth.misc_pack()
    for label, w in (("misc_pack_61layers", wl), ("misc_unpack_61layers", synth.reverse(wl))):
        if label.startswith("misc_pack"):
            src = device_sources(torch, binding, w)
            sp = [x.data_ptr() for t in src for x in t]
            named, dp = device_destinations(torch, binding, w)
        else:
            pack = named["pack"]
            sp = [pack.data_ptr()] * len(w["tensors"])
            named2, dp = device_destinations(torch, binding, w)
        plan = plan_of(binding, w)
        info = plan.info()
        ms = time_plan(torch, binding, plan, sp, dp, stream,
                       poison=list((named if label.startswith("misc_pack") else named2).values()))
        nb = info["bytes_read"] + info["bytes_written"]
        out[label] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1), "bytes": nb,
                      "tensors": info["n_tensors"], "regions": info["regions"],
                      "launches": info["n_launches"], "plan_us": info["plan_ns"] / 1e3}
    del src, named, named2
    # Tall-thin column slabs (the worked example's shape at scale): [R, 8]
    # int32, rows split over 2 sources, columns over 4 destinations, each
    # region R/2 rows x 8 bytes; R = 1M (32 MiB, cache-resident) and 16M
    # (512 MiB each way, past the caches: the four column regions of a source
    # row block share their reads only when they run together, as thin
    # sibling groups).  LDS-staged thin kernel vs the bulk kernel's direct
    # path (thin bucket disabled).
    for rows, key in ((1 << 20, "column_slabs_1Mx8_i32_2row_to_4col"),
                      (1 << 24, "column_slabs_16Mx8_i32_2row_to_4col")):
        t = {"name": "w", "shape": [rows, 8], "dtype": "i32", "src": synth.side([2], [0]),
             "dst": synth.side([4], [1]), "values": {"kind": "uniform", "seed": 1}}
        srcs = [torch.empty((rows // 2) * 8 * 4, dtype=torch.uint8, device="cuda").fill_(7)
                for _ in range(2)]
        dsts = [torch.empty(rows * 2 * 4, dtype=torch.uint8, device="cuda") for _ in range(4)]
        sp = [x.data_ptr() for x in srcs]
        dp = [x.data_ptr() for x in dsts]
        slab = {}
        for label, kw in (("lds_thin_kernel", {}), ("bulk_direct", {"thin_bytes": 1})):
            plan = binding.reshard_plan([spec(t, "src")], [spec(t, "dst")], **kw)
            info = plan.info()
            ms = time_plan(torch, binding, plan, sp, dp, stream, poison=dsts)
            nb = info["bytes_read"] + info["bytes_written"]
            slab[label] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1),
                           "regions": info["regions"]}
            if label == "lds_thin_kernel":
                bb = time_back_to_back(torch, binding, plan, sp, dp, stream)
                slab[label].update(ms_back_to_back=round(bb, 4),
                                   GBps_back_to_back=round(nb / bb / 1e6, 1))
        out[key] = slab
        del srcs, dsts
    # The DSV3 gate and up projections installed as MXFP8 from a source cut
    # TP3 along the 7,168-wide hidden dim: source rows of 2,390 elements
    # (4,780 B apart, off the 16-byte grid) and blocks that straddle two
    # source shards.
    wl = synth.moe_dsv3(quant="mxfp8")
    wl["tensors"] = [dict(t, src=synth.side([3], [2])) for t in wl["tensors"][:2]]
    src = device_sources(torch, binding, wl)
    sp = [x.data_ptr() for t in src for x in t]
    named, dp = device_destinations(torch, binding, wl)
    plan = plan_of(binding, wl)
    info = plan.info()
    ms = time_plan(torch, binding, plan, sp, dp, stream, poison=list(named.values()))
    nb = info["bytes_read"] + info["bytes_written"]
    out["mxfp8_dsv3_gate_up_from_tp3_hidden"] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1),
                                                 "bytes": nb, "regions": info["regions"],
                                                 "launches": info["n_launches"]}
    plan.destroy()
    del src, named
    torch.cuda.empty_cache()
    # A large uneven bf16 layout: TP3 -> TP2 over an odd last dim (2,049),
    # so regions start at source/destination offsets that differ modulo 16
    # (the misaligned path: funnel-shifted 16-byte loads, aligned stores).
    t = {"name": "w", "shape": [16, 8193, 2049], "dtype": "bf16", "src": synth.side([3], [2]),
         "dst": synth.side([2], [2]), "values": {"kind": "normal", "std": 0.02, "seed": 9}}
    wl = {"name": "uneven_tp3_to_tp2", "buffers": {}, "tensors": [t]}
    src = device_sources(torch, binding, wl)
    sp = [x.data_ptr() for tt in src for x in tt]
    named, dp = device_destinations(torch, binding, wl)
    plan = plan_of(binding, wl)
    info = plan.info()
    ms = time_plan(torch, binding, plan, sp, dp, stream, poison=list(named.values()))
    nb = info["bytes_read"] + info["bytes_written"]
    out["uneven_bf16_16x8193x2049_tp3_to_tp2"] = {"ms": round(ms, 4), "GBps": round(nb / ms / 1e6, 1),
                                                  "bytes": nb, "regions": info["regions"]}
    plan.destroy()
    del src, named
    torch.cuda.empty_cache()
    # Execution time of the uneven layouts (fp32 / bf16 [1000,3000] and
    # [7,513,257], meshes [3] / [2,3] -> [7] / [4,2]); small, cache-resident.
    ex = []
    for seed in range(0, 500, 10):
        w = synth.uneven_case(seed)
        u = w["tensors"][0]
        plan = plan_of(binding, w)
        info = plan.info()
        ssp, dsp = spec(u, "src"), spec(u, "dst")
        es = synth.ELEM_BYTES[u["dtype"]]
        sbufs = [torch.empty(max(1, int(np.prod(binding.reshard_shard_box(ssp, k)[1])) * es),
                             dtype=torch.uint8, device="cuda") for k in range(int(np.prod(u["src"]["mesh"])))]
        dbufs = [torch.empty(max(1, int(np.prod(binding.reshard_shard_box(dsp, k)[1])) * es),
                             dtype=torch.uint8, device="cuda") for k in range(int(np.prod(u["dst"]["mesh"])))]
        ms = time_plan(torch, binding, plan, [b.data_ptr() for b in sbufs],
                       [b.data_ptr() for b in dbufs], stream)
        ex.append((ms * 1e3, info["bytes_read"] + info["bytes_written"], info["n_launches"]))
    us = sorted(e[0] for e in ex)
    out["uneven_50_layouts_exec_us"] = {"p50": round(us[len(us) // 2], 2), "max": round(us[-1], 2),
                                        "bytes_p50": sorted(e[1] for e in ex)[len(ex) // 2],
                                        "launches_max": max(e[2] for e in ex)}
    # Plan time over the 500 uneven layouts (CPU).
    ns = []
    for seed in range(500):
        u = synth.uneven_case(seed)["tensors"][0]
        p = binding.reshard_plan([spec(u, "src")], [spec(u, "dst")])
        ns.append(p.info()["plan_ns"])
        p.destroy()
    ns.sort()
    out["uneven_500_plan_us"] = {"p50": ns[250] / 1e3, "p99": ns[494] / 1e3, "max": ns[-1] / 1e3}
    return out


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "memory_GiB": round(p.total_memory / 2**30, 1)}


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def host_workers():
    """Worker processes for the parallel oracle leg: the host CPUs available
    to this process, at most 16 (the CPU share of one GPU on an eight-GPU
    MI355X node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, os.cpu_count() or n, 16))


_FORK_JOB = None


def _fork_call(i):
    fn, items = _FORK_JOB
    fn(items[i])
    return 0


def fork_map(n):
    """A map over n forked worker processes: the function and its items are
    inherited by the workers (nothing is pickled but an index), so a worker
    sees the oracle's assembled tensor and writes its destination slots into
    the shared-memory images the parent reads."""
    import multiprocessing as mp

    def run(fn, items):
        global _FORK_JOB
        _FORK_JOB = (fn, list(items))
        with mp.get_context("fork").Pool(n) as pool:
            pool.map(_fork_call, range(len(_FORK_JOB[1])), chunksize=1)
        _FORK_JOB = None
        return []
    return run


def shared_image(arr):
    """Copy of a host byte image in anonymous shared memory (visible to
    forked workers' writes)."""
    import mmap
    m = mmap.mmap(-1, max(arr.nbytes, 1))
    out = np.frombuffer(m, dtype=np.uint8, count=arr.nbytes)
    out[:] = arr.reshape(-1)
    return out


def cpu_baseline(experts=16):
    """The oracle (as it stands) on a bounded sample of the same workload: the
    same layer shape and meshes with `experts` experts instead of 256, bf16
    relayout plus MXFP8 install, on the host.  Timed once with the six oracle
    calls (3 tensors x 2 variants) one after another in this process, and once
    with each call's destination slots spread over forked worker processes,
    one per available host CPU (the oracle's MXFP8 step is a Python loop over
    blocks that holds the GIL, so threads would not run it in parallel).
    Must run before this process touches the GPU.  Returns (parallel,
    single)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import golden as ogolden
    from rl_weight_refit_amd import synth
    import helpers  # test-side glue: oracle inputs from a workload

    jobs = []
    total_bytes = 0
    for quant in (None, "mxfp8"):
        wl = synth.moe_experts(experts, 7168, 2048, 16, 8, 8, seed=5, quant=quant)
        for t in wl["tensors"]:
            G = synth.host_values(t)
            src = helpers.source_buffers(t, G)
            del G
            one = dict(wl)
            one["tensors"] = [t]
            _, per = helpers.alloc_destinations(one)
            shared = {}
            for e in per[0]:
                for key in ("buf", "scale_buf"):
                    if key in e:
                        if id(e[key]) not in shared:
                            shared[id(e[key])] = shared_image(e[key])
                        e[key] = shared[id(e[key])]
            jobs.append((helpers.src_desc_for(t), helpers.odesc(t, "dst"), src, per[0]))
            n = int(np.prod(t["shape"]))
            # bf16 relayout: 2n read + 2n written; MXFP8: 2n read + n codes + n/32 scales
            total_bytes += 4 * n if quant is None else 3 * n + n // 32

    t0 = time.perf_counter()
    for job in jobs:
        ogolden.reshard(*job)
    single = time.perf_counter() - t0
    nw = host_workers()
    t0 = time.perf_counter()
    for job in jobs:
        ogolden.reshard(*job, map_fn=fork_map(nw))
    parallel = time.perf_counter() - t0
    sample = ("same layer shape and meshes with %d of 256 experts (%d/256 of the bytes), bf16 relayout + "
              "MXFP8 install, numpy on the host" % (experts, experts))
    many = {"value": round(total_bytes / parallel / 1e9, 4), "unit": "GB/s", "cores": nw,
            "kind": "oracle", "sample": sample + ", each of the %d oracle calls (tensor x variant) with "
                                                 "its destination slots on %d forked worker processes, "
                                                 "%.1f s" % (len(jobs), nw, parallel),
            "host": host_info()}
    one = {"value": round(total_bytes / single / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle", "sample": sample + ", one call after another in one process, %.1f s" % single}
    return many, one


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this relayout runs all source and destination "
              "shards in one GPU's memory; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        return 2
    if args.procs > 1:
        return run_processes(args)
    # The oracle's CPU baseline forks worker processes, so it runs before
    # anything here touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        print("cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    import torch
    from rl_weight_refit_amd import binding, synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    binding.load()
    torch.cuda.set_device(0)

    wl_copy = synth.moe_dsv3()
    wl_mx = synth.moe_dsv3(quant="mxfp8")
    do_copy = args.variant in ("both", "copy")
    do_mx = args.variant in ("both", "mxfp8")

    plan_us = {}
    if args.plan_reps > 0:
        if do_copy:
            plan_us["bf16"] = plan_times(binding, wl_copy, args.plan_reps)
        if do_mx:
            plan_us["mxfp8"] = plan_times(binding, wl_mx, args.plan_reps)
    p_copy = plan_of(binding, wl_copy)
    p_mx = plan_of(binding, wl_mx)
    i_copy, i_mx = p_copy.info(), p_mx.info()
    print("planned: bf16 %d regions %d launches; mxfp8 %d regions %d launches"
          % (i_copy["n_regions"], i_copy["n_launches"], i_mx["n_regions"], i_mx["n_launches"]),
          file=sys.stderr, flush=True)

    stream = torch.cuda.Stream()
    ceil_info = copy_ceiling(torch, binding, args.ceiling_bytes, stream,
                             library=not args.ceiling_torch_only) if args.ceiling_bytes else None
    ceiling = ceil_info["GBps"] if ceil_info else None
    print("copy ceiling %.1f GB/s" % (ceiling or 0), file=sys.stderr, flush=True)

    src = device_sources(torch, binding, wl_copy)
    src_ptrs = [s.data_ptr() for shards in src for s in shards]
    d_copy, ptr_copy = device_destinations(torch, binding, wl_copy) if do_copy else ({}, [])
    d_mx, ptr_mx = device_destinations(torch, binding, wl_mx) if do_mx else ({}, [])
    torch.cuda.synchronize()
    print("buffers ready", file=sys.stderr, flush=True)

    sh = stream.cuda_stream

    # The first execute of a plan uploads its tables to the device (a
    # blocking allocation and copy); it runs before the warm-up, timed on the
    # host.  Later executes only validate pointers and enqueue launches.
    first_call_us = {}
    for name, plan, dptrs, on in (("bf16", p_copy, ptr_copy, do_copy), ("mxfp8", p_mx, ptr_mx, do_mx)):
        if on:
            t = time.perf_counter()
            binding.reshard_execute(plan, src_ptrs, dptrs, sh)
            first_call_us[name] = round((time.perf_counter() - t) * 1e6, 1)
            stream.synchronize()
    host_us = {"bf16": [], "mxfp8": []}

    def step(ev, record_host=False):
        if do_copy:
            ev[0].record(stream)
            t = time.perf_counter()
            binding.reshard_execute(p_copy, src_ptrs, ptr_copy, sh)
            if record_host:
                host_us["bf16"].append((time.perf_counter() - t) * 1e6)
            ev[1].record(stream)
        if do_mx:
            ev[2].record(stream)
            t = time.perf_counter()
            binding.reshard_execute(p_mx, src_ptrs, ptr_mx, sh)
            if record_host:
                host_us["mxfp8"].append((time.perf_counter() - t) * 1e6)
            ev[3].record(stream)

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k], record_host=True)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print("timed %d steps in %.3f s" % (args.steps, wall), file=sys.stderr, flush=True)

    # The same executes again, outside the timed steps, with every
    # destination byte poison-filled (0xFF) on the stream before each rep
    # and outside its events: no rep can find the previous one's output in
    # a cache.
    poisoned = {}
    if do_copy and args.poison_reps > 0:
        poisoned["bf16"] = time_plan(torch, binding, p_copy, src_ptrs, ptr_copy, stream,
                                     reps=args.poison_reps, poison=list(d_copy.values()))
    if do_mx and args.poison_reps > 0:
        poisoned["mxfp8"] = time_plan(torch, binding, p_mx, src_ptrs, ptr_mx, stream,
                                      reps=args.poison_reps, poison=list(d_mx.values()))

    t_copy = [e[0].elapsed_time(e[1]) for e in evs] if do_copy else []
    t_mx = [e[2].elapsed_time(e[3]) for e in evs] if do_mx else []
    bytes_copy = i_copy["bytes_read"] + i_copy["bytes_written"]
    bytes_mx = i_mx["bytes_read"] + i_mx["bytes_written"]
    step_bytes = (bytes_copy if do_copy else 0) + (bytes_mx if do_mx else 0)
    value = step_bytes * args.steps / wall / 1e9

    def stats(ts, nbytes):
        if not ts:
            return None
        med = statistics.median(ts)
        return {"ms_median": round(med, 4), "ms_min": round(min(ts), 4),
                "ms_max": round(max(ts), 4),
                "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
                "pct_peak": round(100 * nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                "pct_ceiling": round(100 * nbytes / (med * 1e-3) / 1e9 / ceiling, 2)
                if ceiling else None,
                "bytes": nbytes}

    dominant = "rs_bulk_kernel" if do_copy else "rs_mx_kernel"
    dom_ts = t_copy if do_copy else t_mx
    dom_bytes = bytes_copy if do_copy else bytes_mx
    achieved = dom_bytes / (statistics.mean(dom_ts) * 1e-3) / 1e9
    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        with open(PROFILE_COUNTERS) as f:
            c = json.load(f)
        if c.get("kernel_source_sha256_16") == kernel_hash() and c.get("kernel") == dominant:
            traffic = c.get("traffic_bytes_per_launch")

    # The MXFP8 kernel's own roofline (achieved per execute, from the same
    # HIP events; the plan takes rs_plan_info.n_launches launches).
    roof_mx = None
    if do_mx:
        ach_mx = bytes_mx / (statistics.mean(t_mx) * 1e-3) / 1e9
        traffic_mx = None
        if os.path.exists(PROFILE_COUNTERS_MX):
            with open(PROFILE_COUNTERS_MX) as f:
                c = json.load(f)
            if c.get("kernel_source_sha256_16") == kernel_hash():
                traffic_mx = c.get("traffic_bytes_per_execute")
        roof_mx = {"kernel": "rs_mx_kernel", "bound": "hbm", "achieved": round(ach_mx, 1),
                   "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach_mx / HBM_PEAK_GBPS, 4),
                   "traffic": traffic_mx, "per": "execute (%d launches)" % i_mx["n_launches"]}

    out = {
        "metric": "reshard effective HBM GB/s (read+write) and % of MI355X HBM peak; plan us",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->bf16 copy + bf16->mxfp8(e4m3/e8m0)" if args.variant == "both"
        else ("bf16" if do_copy else "bf16->mxfp8"),
        "data": "synthetic: N(0,0.02) bf16 generated on the GPU (torch generator, seed 5000+i)",
        "config": {"workload": "moe_dsv3_layer: 256 experts x hidden 7168 x expert intermediate "
                               "2048, gate/up/down bf16, EP16 Shard(0) -> EP8xTP8, fused w13; "
                               "plus the BF16->MXFP8 install variant",
                   "variant": args.variant, "step_bytes": step_bytes},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "copy_ceiling_GBps": ceiling,
        "copy_ceiling": ceil_info,
        "bf16": stats(t_copy, bytes_copy),
        "mxfp8": stats(t_mx, bytes_mx),
        "poison_filled_ms_median": {k: round(v, 4) for k, v in poisoned.items()},
        "plan_us": plan_us,
        "execute_host_us": {k: {"first_call_with_upload": first_call_us[k],
                                "p50": round(statistics.median(v), 1)}
                            for k, v in host_us.items() if v},
        "plan": {"bf16": {k: i_copy[k] for k in ("n_regions", "n_launches", "bytes_read",
                                                  "bytes_written")},
                 "mxfp8": {k: i_mx[k] for k in ("n_regions", "n_launches", "bytes_read",
                                                 "bytes_written")}},
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "roofline_mxfp8": roof_mx,
        "device": device_info(torch),
    }
    del src, d_copy, d_mx
    torch.cuda.empty_cache()
    if not args.no_secondary:
        print("secondary workloads ...", file=sys.stderr, flush=True)
        out["secondary"] = secondary(torch, binding, stream)
        torch.cuda.empty_cache()
    if cpu is not None:
        out["cpu_baseline"], out["cpu_baseline_single_process"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
