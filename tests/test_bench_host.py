"""Host-side checks of bench.py (no GPU): the one-GPU refusal, and the
device-source hash that decides whether committed counter profiles belong to
the kernels being timed (comments and blank lines do not count, code does)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    copies = []
    for path in bench.KERNEL_SOURCES:
        q = tmp_path / os.path.basename(path)
        q.write_text(open(path, encoding="utf-8").read(), encoding="utf-8")
        copies.append(q)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(q) for q in copies])
    h0 = bench.kernel_hash()
    text = copies[0].read_text(encoding="utf-8")
    copies[0].write_text("// a new comment line\n\n" + text.replace("\n", "  \n", 3) +
                         "\n/* a block\n   comment */\n", encoding="utf-8")
    assert bench.kernel_hash() == h0
    copies[0].write_text(text.replace("kThreads", "kThreads ", 1) + "\nstatic int x;\n",
                         encoding="utf-8")
    assert bench.kernel_hash() != h0


def test_forked_oracle_leg_writes_the_same_bytes():
    """The CPU baseline's parallel leg (destination slots on forked workers,
    images in shared memory) produces the serial oracle's bytes."""
    import numpy as np
    from oracle import golden as ogolden
    from rl_weight_refit_amd import synth
    import helpers
    for quant in (None, "mxfp8"):
        wl = synth.moe_experts(8, 256, 96, 4, 2, 2, seed=11, quant=quant)
        for t in wl["tensors"]:
            G = synth.host_values(t)
            src = helpers.source_buffers(t, G)
            one = dict(wl, tensors=[t])
            _, serial = helpers.alloc_destinations(one)
            _, forked = helpers.alloc_destinations(one)
            shared = {}
            for e in forked[0]:
                for key in ("buf", "scale_buf"):
                    if key in e:
                        if id(e[key]) not in shared:
                            shared[id(e[key])] = bench.shared_image(e[key])
                        e[key] = shared[id(e[key])]
            sd, dd = helpers.src_desc_for(t), helpers.odesc(t, "dst")
            ogolden.reshard(sd, dd, src, serial[0])
            ogolden.reshard(sd, dd, src, forked[0], map_fn=bench.fork_map(3))
            for a, b in zip(serial[0], forked[0]):
                for key in ("buf", "scale_buf"):
                    if key in a:
                        assert np.array_equal(a[key].reshape(-1), b[key].reshape(-1)), (quant, t["name"])
