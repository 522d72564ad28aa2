"""GPU parity of the copy kernel's spread groups against the CPU oracle,
byte for byte: rows of whole 1 KiB pieces with two and three outer dims
(row and outer indices advanced by carries, outer extents as small as 2),
7 KiB rows whose pieces wrap across rows, 768-byte rows numbered lane by
lane, with and without destination replicas, at work units of 8 to 64 KiB
(several load batches per workgroup at the larger ones), whole groups and
the tail units after them."""

import pytest
import torch

from rl_weight_refit_amd import binding

import gpu_helpers as gh
import spread_layouts as sl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield


@pytest.mark.parametrize("unit_bytes", [8192, 16384, 32768, 65536])
@pytest.mark.parametrize("name", sorted(sl.ALL))
def test_spread_layouts(name, unit_bytes):
    gh.log("spread %s unit %d" % (name, unit_bytes))
    plan = gh.check_against_oracle(sl.ALL[name](), unit_bytes=unit_bytes)
    assert plan.info()["regions"]["bulk"] > 0


@pytest.mark.parametrize("shifts", [(16, 0), (0, 32), (4, 0)])
@pytest.mark.parametrize("name", ["rows_three_outer", "flat_short_rows"])
def test_spread_layouts_shifted_pointers(name, shifts):
    """Buffers moved by 16 or 32 bytes keep the 16-byte alignment the spread
    paths need; a 4-byte shift takes the misaligned path instead."""
    gh.check_against_oracle(sl.ALL[name](), src_shift=shifts[0], dst_shift=shifts[1])


@pytest.mark.parametrize("seed", range(80))
def test_spread_random_layouts(seed):
    """Seeded random layouts with large regions (row lengths, outer dims,
    uneven splits and replicas all vary), a work unit of 8, 16 or 32 KiB and
    buffers shifted by 0, 16 or 4 bytes."""
    unit = (8192, 16384, 32768)[seed % 3]
    shift = (0, 16, 4)[(seed // 3) % 3]
    gh.log("spread random %d unit %d shift %d" % (seed, unit, shift))
    gh.check_against_oracle(sl.random_case(seed), unit_bytes=unit, src_shift=shift,
                            dst_shift=(shift * 3) % 32)
