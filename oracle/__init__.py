"""CPU oracle for the DTensor-to-DTensor M->N relayout (the Reshard collective).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP path
(no kernels, headers, helpers or constant tables) and imports nothing from it.

What it computes is the "golden" transport described on the NeMo RL design
page "NCCL Reshard Refit (Experimental)", section "xferdtensor Transports":
the full logical tensor is assembled and every destination keeps only its own
part.  The Reshard pages ("Recasting refit as a DTensor-to-DTensor transfer")
state that the shard-to-shard method reaches exactly that result while moving
only the overlapping regions, so the golden is the plain definition the GPU
path must match byte for byte.

Modules:
  layout  -- shard boxes of a (global shape, mesh, placements) description
  golden  -- gather-then-slice reshard, writing through destination views
  brute   -- per-element ownership brute force (tiny cases only)
  mxfp8   -- BF16 -> MXFP8 (E4M3 elements, E8M0 block scale) rule
  fp8block -- blockwise-FP8 weights and their scale tensors
"""

from . import layout, golden, brute, mxfp8, fp8block  # noqa: F401
