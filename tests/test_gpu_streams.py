"""GPU execution contract: plans on non-default streams, one plan executed
concurrently on several streams (and from several host threads) into
separate destinations, two plans at once, an execute captured into a HIP
graph and replayed, and a plan with more pointers than one launch's
arguments hold (its device pointer tables, and the pooled launches it falls
back to).  Every result is compared byte for byte with the CPU oracle,
poison and guard bytes included.
"""

import threading

import pytest
import torch

from rl_weight_refit_amd import binding, synth

import gpu_helpers as gh
import helpers
import lib_helpers as lh

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield


WORKLOADS = {
    "worked_8x8_tiny": synth.worked_example,
    "moe_small": lambda: synth.moe_experts(16, 512, 192, 8, 4, 4, seed=9),
    "moe_small_mxfp8": lambda: synth.moe_experts(16, 512, 192, 8, 4, 4, seed=9, quant="mxfp8"),
    "uneven_7": lambda: synth.uneven_case(7),
    "dense_ffn_fanout": lambda: synth.dense_ffn(hidden=256, inter=1000, src_tp=4, dst_tp=2, dst_dp=2),
    # 61 layers of small tensors unpacked from one buffer into 4 TP slots
    # each: 1,465 pointers, more than one launch's kernel arguments hold.
    "misc_unpack_many_ptrs": lambda: synth.reverse(synth.misc_pack(hidden=256, q_rank=64, kv_rank=32,
                                                                   experts=8)),
}


def _setup(name, copies=1):
    wl = WORKLOADS[name]()
    _, sources, _, per = helpers.golden_workload(wl)
    bufs = [gh.device_buffers(wl, sources, per) for _ in range(copies)]
    torch.cuda.synchronize()   # poison fills ran on the current stream
    return wl, lh.plan_workload(wl), bufs


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_non_default_stream(name):
    wl, plan, [(src_dev, sp, dp, flat)] = _setup(name)
    s = torch.cuda.Stream()
    binding.reshard_execute(plan, sp, dp, s.cuda_stream)
    s.synchronize()
    gh.check_device(wl["name"], flat)


@pytest.mark.parametrize("name", ["moe_small", "moe_small_mxfp8", "uneven_7", "misc_unpack_many_ptrs"])
def test_one_plan_on_several_streams(name):
    """The same plan, four streams, four destination sets, no synchronisation
    between the executes."""
    wl, plan, bufs = _setup(name, copies=4)
    streams = [torch.cuda.Stream() for _ in bufs]
    for rep in range(3):
        for (src_dev, sp, dp, flat), s in zip(bufs, streams):
            binding.reshard_execute(plan, sp, dp, s.cuda_stream)
    torch.cuda.synchronize()
    for _, _, _, flat in bufs:
        gh.check_device(wl["name"], flat)


@pytest.mark.parametrize("name", ["moe_small_mxfp8", "misc_unpack_many_ptrs"])
def test_one_plan_from_several_threads(name):
    """Host threads share one plan (the first execute uploads its tables
    under the plan's lock; with more pointers than one launch's arguments
    hold, each thread's pointer set gets its device table under that lock
    too); each thread has its own stream and buffers."""
    wl, plan, bufs = _setup(name, copies=4)
    errors = []

    def work(k):
        try:
            s = torch.cuda.Stream()
            _, sp, dp, _ = bufs[k]
            for _ in range(10):
                binding.reshard_execute(plan, sp, dp, s.cuda_stream)
            s.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(bufs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for _, _, _, flat in bufs:
        gh.check_device(wl["name"], flat)


def test_two_plans_at_once():
    wa, pa, [(_, spa, dpa, fa)] = _setup("moe_small_mxfp8")
    wb, pb, [(_, spb, dpb, fb)] = _setup("dense_ffn_fanout")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    binding.reshard_execute(pa, spa, dpa, s1.cuda_stream)
    binding.reshard_execute(pb, spb, dpb, s2.cuda_stream)
    torch.cuda.synchronize()
    gh.check_device(wa["name"], fa)
    gh.check_device(wb["name"], fb)


@pytest.mark.parametrize("name", ["worked_8x8_tiny", "moe_small_mxfp8", "uneven_7", "dense_ffn_fanout",
                                  "misc_unpack_many_ptrs"])
def test_graph_capture_and_replay(name):
    """After its first execute (which uploads the tables) a plan only enqueues
    kernels, so it can be captured into a HIP graph.  Each replay follows an
    eager re-poisoning of every destination and must rewrite them exactly."""
    wl, plan, [(src_dev, sp, dp, flat)] = _setup(name)
    s = torch.cuda.Stream()
    binding.reshard_execute(plan, sp, dp, s.cuda_stream)
    s.synchronize()
    gh.check_device(wl["name"], flat)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.reshard_execute(plan, sp, dp, torch.cuda.current_stream().cuda_stream)
    dsts = {id(d): d for _, d in flat}.values()
    for rep in range(4):
        for d in dsts:
            d.body().fill_(d.poison)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gh.check_device(wl["name"], flat)


def test_debug_checks_reject_a_short_allocation(monkeypatch):
    """With RESHARD_DEBUG_CHECKS=1 every pointer is checked against its
    allocation before anything is launched.  Destination 2 of the worked
    example gets a 60-byte allocation where the plan writes 64 bytes: the
    call fails naming it.  (Allocations are rounded up to whole pages, so
    even a missed check could not write outside mapped memory.)"""
    import ctypes
    wl = WORKLOADS["worked_8x8_tiny"]()
    _, sources, _, per = helpers.golden_workload(wl)
    _, sp, dp, flat = gh.device_buffers(wl, sources, per)
    torch.cuda.synchronize()
    plan = lh.plan_workload(wl)
    hip = ctypes.CDLL("libamdhip64.so")
    short = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(short), ctypes.c_size_t(60)) == 0
    try:
        monkeypatch.setenv("RESHARD_DEBUG_CHECKS", "1")
        bad = list(dp)
        bad[2] = short.value
        stream = torch.cuda.current_stream().cuda_stream
        with pytest.raises(binding.ReshardError) as e:
            binding.reshard_execute(plan, sp, bad, stream)
        assert e.value.status == 1
        assert "dst_ptrs[2] needs 64 bytes but its allocation ends 60 bytes after it" in str(e.value)
        # the right buffers pass the same checks
        binding.reshard_execute(plan, sp, dp, stream)
        torch.cuda.synchronize()
        gh.check_device(wl["name"], flat)
    finally:
        torch.cuda.synchronize()
        hip.hipFree(short)


def test_pointer_tables_and_pooled_fallback():
    """A plan with more pointers than one launch's arguments hold runs in one
    launch per kernel from a device table of the call's pointers, one table
    per pointer set, up to 8 sets per device; a ninth and tenth set run the
    pooled launches.  Each set, executed twice (the second time from its
    table), and the sets run after the limit all match the oracle."""
    wl, plan, bufs = _setup("misc_unpack_many_ptrs", copies=10)
    info = plan.info()
    assert info["n_src_ptrs"] + info["n_dst_ptrs"] > 500
    assert info["n_launches"] < info["n_launches_pooled"], info
    s = torch.cuda.Stream()
    for rep in range(2):
        for src_dev, sp, dp, flat in bufs:
            if rep:
                for d in {id(d): d for _, d in flat}.values():
                    d.body().fill_(d.poison)
                torch.cuda.synchronize()
            binding.reshard_execute(plan, sp, dp, s.cuda_stream)
            s.synchronize()
            gh.check_device(wl["name"], flat)


def test_graph_capture_of_a_new_pointer_set():
    """After a first execute (which uploads the plan's tables), an execute
    captured with pointers the plan has not seen (no pointer table may be
    made while capturing) records the pooled launches; replays rewrite the
    destinations exactly."""
    wl, plan, [(_, sp0, dp0, flat0), (_, sp, dp, flat)] = _setup("misc_unpack_many_ptrs", copies=2)
    s = torch.cuda.Stream()
    binding.reshard_execute(plan, sp0, dp0, s.cuda_stream)
    s.synchronize()
    gh.check_device(wl["name"], flat0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.reshard_execute(plan, sp, dp, torch.cuda.current_stream().cuda_stream)
    dsts = {id(d): d for _, d in flat}.values()
    for rep in range(3):
        for d in dsts:
            d.body().fill_(d.poison)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gh.check_device(wl["name"], flat)
