"""GPU-side test glue: device buffers for a workload, one HIP-path run through
the C ABI, and comparisons with the oracle.

Destinations are filled with a poison byte and followed by a guard area of
the same poison, so stray writes past a buffer or outside a view show up.
Pointers can be offset by a few bytes from the allocation to exercise the
kernels' misaligned paths.
"""

import sys

import numpy as np
import torch

from oracle import golden as ogolden
from oracle import layout as olayout
from rl_weight_refit_amd import binding

import helpers
import lib_helpers as lh

GUARD = 4096


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


class DevBuf:
    """A device byte buffer with a leading misalignment and a trailing guard."""

    def __init__(self, nbytes, fill=None, data=None, shift=0, guard=GUARD, poison=0xA5):
        self.nbytes = int(nbytes)
        self.shift = int(shift)
        total = self.shift + self.nbytes + guard
        self.t = torch.full((max(total, 1),), poison, dtype=torch.uint8, device="cuda")
        if data is not None:
            self.t[self.shift:self.shift + self.nbytes].copy_(torch.from_numpy(np.ascontiguousarray(data)))
        self.poison = poison
        self.guard = guard

    @property
    def ptr(self):
        return self.t.data_ptr() + self.shift

    def body(self):
        return self.t[self.shift:self.shift + self.nbytes]

    def host(self):
        return self.body().cpu().numpy()

    def guard_ok(self):
        g = self.t[self.shift + self.nbytes:self.shift + self.nbytes + self.guard]
        head = self.t[:self.shift]
        return bool((g == self.poison).all()) and bool((head == self.poison).all())


def device_buffers(workload, sources, per_tensor_dst_host, poison=0xA5, src_shift=0, dst_shift=0):
    """Upload sources and allocate poisoned destinations shaped like the host
    images.  Returns (src_dev, src_ptrs, dst_ptrs, dst_dev_flat) in the
    library's pointer order; dst_dev_flat pairs each destination pointer's
    host image with its device buffer."""
    src_dev = []
    src_seen = {}
    for t_src in sources:
        row = []
        for e in t_src:
            for hb in (e["parts"] if "parts" in e else [e["buf"]]):
                if id(hb) not in src_seen:   # shared (packed) source buffers upload once
                    src_seen[id(hb)] = DevBuf(hb.size, data=hb, shift=src_shift)
                row.append(src_seen[id(hb)])
        src_dev.append(row)
    # Shared (fused) buffers are the same numpy object in the host images.
    seen = {}
    dst_ptrs = []
    dst_dev_flat = []
    for t, slots in zip(workload["tensors"], per_tensor_dst_host):
        for key, parts_key in (("buf", "parts"), ("scale_buf", "scale_parts")):
            if key == "scale_buf" and t["dst"].get("quant") != "mxfp8":
                continue
            for e in slots:
                for hb in (e[parts_key] if parts_key in e else [e[key]]):
                    if id(hb) not in seen:
                        seen[id(hb)] = DevBuf(hb.size, shift=dst_shift, poison=poison)
                    dst_ptrs.append(seen[id(hb)].ptr)
                    dst_dev_flat.append((hb, seen[id(hb)]))
    src_ptrs = [b.ptr for ts in src_dev for b in ts]
    return src_dev, src_ptrs, dst_ptrs, dst_dev_flat


def check_device(workload_name, dst_dev_flat):
    """Every destination buffer equals its oracle image (poison outside the
    views included) and its guard bytes are intact."""
    checked = set()
    for host_img, dev in dst_dev_flat:
        if id(dev) in checked:
            continue
        checked.add(id(dev))
        got = dev.host()
        if not np.array_equal(got, host_img):
            bad = np.nonzero(got != host_img)[0]
            raise AssertionError("%s: %d bytes differ, first at %d (got %#x want %#x)"
                                 % (workload_name, bad.size, bad[0], got[bad[0]], host_img[bad[0]]))
        assert dev.guard_ok(), "%s: guard bytes overwritten" % workload_name


def device_run(workload, sources, per_tensor_dst_host, poison=0xA5, src_shift=0, dst_shift=0,
               plan=None, stream=None, **plan_kw):
    """Upload sources, allocate poisoned destinations shaped like the host
    images, execute the HIP path, return the device buffers in pointer order.
    """
    src_dev, src_ptrs, dst_ptrs, dst_dev_flat = device_buffers(
        workload, sources, per_tensor_dst_host, poison, src_shift, dst_shift)
    if plan is None:
        plan = lh.plan_workload(workload, **plan_kw)
    s = stream if stream is not None else torch.cuda.current_stream()
    binding.reshard_execute(plan, src_ptrs, dst_ptrs, s.cuda_stream)
    torch.cuda.synchronize()
    return plan, src_dev, dst_dev_flat


def check_against_oracle(workload, poison=0xA5, src_shift=0, dst_shift=0, globals_=None,
                         **plan_kw):
    """Full byte-for-byte comparison of every destination buffer with the
    oracle's golden image (poison outside the views included), guards intact,
    sources unchanged."""
    G, sources, named, per = helpers.golden_workload(workload, poison=poison, globals_=globals_)
    # Fresh poisoned host images shaped like the oracle's, for allocation only.
    plan, src_dev, dst_dev = device_run(workload, sources, per, poison=poison,
                                        src_shift=src_shift, dst_shift=dst_shift, **plan_kw)
    check_device(workload["name"], dst_dev)
    for t_src, t_dev in zip(sources, src_dev):
        host = [hb for e in t_src for hb in (e["parts"] if "parts" in e else [e["buf"]])]
        for hb, d in zip(host, t_dev):
            assert np.array_equal(d.host(), hb), "source modified"
    return plan
