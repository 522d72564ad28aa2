"""reshard_execute_no_alloc: the same relayout with no device allocation (the
plan's tables go through the library's static per-GPU table area).

Each GPU case runs both entry points on the same seeded inputs into
separately poisoned destinations and requires byte equality between them and
with the oracle's golden images.  Two no-alloc calls follow each other on one
stream, the second with a smaller plan, so the second call's tables overwrite
the first call's in the shared area.
"""

import numpy as np
import pytest
import torch

from rl_weight_refit_amd import binding, synth

import gpu_helpers as gh
import helpers
import lib_helpers as lh


def many_region_workload():
    """A [4096, 4096] u8 tensor, 256 column shards -> 256 row shards: 65,536
    regions of 16 x 16 bytes, whose tables (over 8 MB) exceed the area."""
    t = {"name": "w", "shape": [4096, 4096], "dtype": "u8", "src": synth.side([256], [1]),
         "dst": synth.side([256], [0]), "values": {"kind": "index"}}
    return {"name": "many_regions", "buffers": {}, "tensors": [t]}


def test_tables_larger_than_the_area_are_refused():
    """Checked on the host before anything is copied or launched (no GPU)."""
    plan = lh.plan_workload(many_region_workload())
    assert plan.info()["n_regions"] == 65536
    fake = 0x100000
    with pytest.raises(binding.ReshardError) as e:
        binding.reshard_execute_no_alloc(plan, [fake + i * 65536 for i in range(256)],
                                         [fake + (1 << 30) + i * 65536 for i in range(256)])
    assert e.value.status == 3 and "static table area" in str(e.value)


def _prepare(wl):
    G, sources, named, per = helpers.golden_workload(wl, poison=0xA5)
    plan = lh.plan_workload(wl)
    ref = gh.device_buffers(wl, sources, per, poison=0xA5)
    mine = gh.device_buffers(wl, sources, per, poison=0xA5)
    return plan, ref, mine


def _compare(name, ref, mine):
    for (img, a), (_, b) in zip(ref[3], mine[3]):
        got = b.host()
        assert np.array_equal(got, a.host()), "%s: no-alloc output differs from reshard_execute" % name
    gh.check_device(name, mine[3])


@pytest.mark.gpu
def test_no_alloc_matches_execute_twice_smaller_second():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    big = synth.moe_experts(8, 256, 96, 4, 2, 2, seed=11, quant="mxfp8")
    small = synth.worked_example()
    gh.log("no-alloc: %s then %s" % (big["name"], small["name"]))
    pb, ref_b, mine_b = _prepare(big)
    ps, ref_s, mine_s = _prepare(small)
    assert pb.info()["n_regions"] > ps.info()["n_regions"]
    stream = torch.cuda.current_stream().cuda_stream
    binding.reshard_execute(pb, ref_b[1], ref_b[2], stream)
    binding.reshard_execute(ps, ref_s[1], ref_s[2], stream)
    # Back to back on one stream: the small plan's tables replace the big
    # one's in the area only after the big plan's kernels have run.
    binding.reshard_execute_no_alloc(pb, mine_b[1], mine_b[2], stream)
    binding.reshard_execute_no_alloc(ps, mine_s[1], mine_s[2], stream)
    torch.cuda.synchronize()
    _compare(big["name"], ref_b, mine_b)
    _compare(small["name"], ref_s, mine_s)


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", [
    (("dense", {}), ("uneven", {"seed": 3})),
    (("moe", {"quant": None}), ("uneven", {"seed": 17})),
    # 768 per-expert source pointers: reshard_execute runs the plan's table
    # form (one launch), the no-alloc call its pooled form (two launches)
    (("experts", {"quant": "mxfp8"}), ("uneven", {"seed": 29})),
])
def test_no_alloc_sequences(first, second):
    """More pairs of calls, larger plan first, each checked against
    reshard_execute and the oracle after both have run."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()

    def make(kind, kw):
        if kind == "dense":
            return synth.dense_ffn(hidden=64, inter=320, src_tp=4, dst_tp=2, dst_dp=2)
        if kind == "moe":
            return synth.moe_experts(16, 512, 128, 4, 2, 2, seed=5, **kw)
        if kind == "experts":
            return synth.moe_experts(256, 256, 96, 8, 4, 2, seed=5, src_split=True, **kw)
        return synth.uneven_case(kw["seed"], shapes=[[100, 300], [7, 51, 25]])

    wa, wb = make(*first), make(*second)
    gh.log("no-alloc: %s then %s" % (wa["name"], wb["name"]))
    pa, ref_a, mine_a = _prepare(wa)
    pb, ref_b, mine_b = _prepare(wb)
    assert pa.info()["n_regions"] > pb.info()["n_regions"]
    if first[0] == "experts":
        assert pa.info()["n_launches"] < pa.info()["n_launches_pooled"]
    stream = torch.cuda.current_stream().cuda_stream
    binding.reshard_execute(pa, ref_a[1], ref_a[2], stream)
    binding.reshard_execute(pb, ref_b[1], ref_b[2], stream)
    binding.reshard_execute_no_alloc(pa, mine_a[1], mine_a[2], stream)
    binding.reshard_execute_no_alloc(pb, mine_b[1], mine_b[2], stream)
    torch.cuda.synchronize()
    _compare(wa["name"], ref_a, mine_a)
    _compare(wb["name"], ref_b, mine_b)
