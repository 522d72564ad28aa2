"""GPU parity of the LDS-staged thin kernel's sibling groups against the CPU
oracle, byte for byte: column slabs whose regions read the same source rows
(groups of 2 to 8 members, several work units each, a partial last unit),
uneven column splits (members of different widths, grouped when loaded
whole),
groups loaded whole by one workgroup per row block (contiguous spans, spans
narrower than the source row, wide spans, several units with a ragged
tail, replicas without fan-out, members of 4 bytes or less read through
swizzled LDS slots),
destination replicas, three-dim tensors with several outer dims, and
shifted buffers."""

import pytest
import torch

from rl_weight_refit_amd import binding, synth

import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield


def _slabs(shape, dtype, src, dst, seed=61):
    vals = {"kind": "uniform", "seed": seed} if dtype in ("f32", "bf16") else {"kind": "index"}
    t = {"name": "w", "shape": shape, "dtype": dtype, "src": synth.side(*src),
         "dst": synth.side(*dst), "values": vals}
    return {"name": "thin_%s" % "x".join(map(str, shape)), "buffers": {}, "tensors": [t]}


CASES = {
    "rows_2_to_cols_4": ([65536 + 300, 8], "i32", ([2], [0]), ([4], [1])),
    "rows_2_to_cols_8": ([40000, 8], "i32", ([2], [0]), ([8], [1])),
    "rows_3_to_cols_3_uneven": ([50000, 8], "i32", ([3], [0]), ([3], [1])),
    "cols_2_replicated_3": ([30000, 16], "bf16", ([2], [0]), ([2, 3], [1, -1])),
    "three_dim_outer_dims": ([6, 9000, 8], "f32", ([2], [1]), ([2, 4], [0, 2])),
    "u8_narrow_columns": ([100000, 12], "u8", ([1], [-1]), ([6], [1])),
    # groups loaded whole: one workgroup reads each block of source rows once
    "whole_many_units_ragged": ([262144 + 77, 8], "i32", ([2], [0]), ([4], [1])),
    "whole_partial_span_u8": ([70000, 10], "u8", ([2], [0]), ([3], [1])),
    "whole_wide_span_bf16": ([20000, 96], "bf16", ([2], [0]), ([16], [1])),
    "whole_f64_pairs": ([30000, 4], "f64", ([3], [0]), ([2], [1])),
    # members of 4 bytes or less (swizzled LDS slots), a last unit of 5 rows
    # per source (its block not a whole number of 128-byte slot groups)
    "narrow_f32_8_cols_ragged": ([2 * (512 * 3 + 5), 8], "f32", ([2], [0]), ([8], [1])),
    "narrow_bf16_8_cols": ([40000, 16], "bf16", ([2], [0]), ([8], [1])),
    "narrow_u8_16_cols": ([50000, 16], "u8", ([2], [0]), ([16], [1])),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_thin_sibling_groups(name):
    gh.log("thin %s" % name)
    plan = gh.check_against_oracle(_slabs(*CASES[name]))
    assert plan.info()["regions"]["thin"] > 0


@pytest.mark.parametrize("shifts", [(4, 0), (0, 8), (3, 5)])
def test_thin_sibling_groups_shifted(shifts):
    gh.check_against_oracle(_slabs(*CASES["rows_2_to_cols_4"]), src_shift=shifts[0],
                            dst_shift=shifts[1])


def test_thin_group_replicas_without_fanout():
    """Replicated column slabs planned without fan-out: members of one group
    read the same columns for different replicas."""
    gh.check_against_oracle(_slabs([40000, 8], "i32", ([2], [0]), ([4, 2], [1, -1])), fanout=False)


@pytest.mark.parametrize("shifts", [(2, 0), (0, 3), (1, 7)])
def test_thin_group_partial_span_shifted(shifts):
    gh.check_against_oracle(_slabs(*CASES["whole_partial_span_u8"]), src_shift=shifts[0],
                            dst_shift=shifts[1])
