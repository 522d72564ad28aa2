"""GPU parity on seeded random plans: 1 to 3 tensors per plan, ranks 1-4,
u8 / bf16 / i32 / f64 and MXFP8 installs, padded views into shared buffers,
random planning options (fan-out, unit, tiny and thin thresholds) and
misaligned pointers (helpers.random_plan_case), byte for byte against the
oracle with poisoned destinations and guard areas; 100 more with tensors of up
to 48 MB."""

import pytest
import torch

from rl_weight_refit_amd import binding

import gpu_helpers as gh
import helpers

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield


@pytest.mark.parametrize("seed", range(500))
def test_random_plan(seed):
    wl, opts, (ss, ds) = helpers.random_plan_case(seed)
    gh.log("random plan %d %s shifts %d %d" % (seed, opts, ss, ds))
    gh.check_against_oracle(wl, src_shift=ss, dst_shift=ds, **opts)


@pytest.mark.parametrize("seed", range(1000, 1100))
def test_random_plan_large(seed):
    """The same generator with tensors of up to 48 MB: many work units per
    region, whole spread groups, long misaligned rows staged through LDS."""
    wl, opts, (ss, ds) = helpers.random_plan_case(seed, max_bytes=48 << 20)
    gh.log("random plan large %d %s shifts %d %d" % (seed, opts, ss, ds))
    gh.check_against_oracle(wl, src_shift=ss, dst_shift=ds, **opts)
