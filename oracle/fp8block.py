"""Blockwise-FP8 weights with per-block scales (oracle; test infrastructure only).

"NCCL Reshard Refit (Experimental)", section "Enabling It", supports a
blockwise-FP8 training side feeding an FP8 generation side; section "Design
Overview" lists the weights' _scale_inv siblings.  The pages give no block
size; the reading taken here is the blockwise recipe of DeepSeek-V3-style FP8
training: E4M3 weight bytes with one float32 scale per 128 x 128 block of the
last two dims (a block size of 1 leaves a dim unblocked).  A weight of shape
[..., N, K] then has scales of shape [..., ceil(N/128), ceil(K/128)], and the
real value of element (n, k) is decode(w[n, k]) * scale[n // 128, k // 128].

For a reshard to carry the scales with their weights, every shard of the
weight must consist of whole blocks (or end at the tensor's edge) and the
scale tensor, laid out on the same mesh with the same placements, must hold
exactly those blocks' scales.
"""

import numpy as np

from . import layout
from . import mxfp8


def aligned(weight_desc, scale_desc, block):
    """True if every slot's weight box is its scale box scaled by the block
    (clipped to the weight's extent), slot by slot."""
    wb = layout.slot_boxes(weight_desc)
    sb = layout.slot_boxes(scale_desc)
    if len(wb) != len(sb):
        return False
    shape = weight_desc["shape"]
    for (wo, wl), (so, sl) in zip(wb, sb):
        for d in range(len(shape)):
            if wl[d] == 0:
                if sl[d] != 0:
                    return False
                continue
            if wo[d] != so[d] * block[d] or wo[d] + wl[d] != min((so[d] + sl[d]) * block[d], shape[d]):
                return False
    return True


def aligned_brute(weight_desc, scale_desc, block):
    """The same fact element by element (tiny cases): each slot's weight
    elements fall in blocks that its scale box holds, and every block its
    scale box holds has a weight element in the slot."""
    wb = layout.slot_boxes(weight_desc)
    sb = layout.slot_boxes(scale_desc)
    shape = weight_desc["shape"]
    for (wo, wl), (so, sl) in zip(wb, sb):
        blocks_from_weights = set()
        for idx in np.ndindex(*wl):
            g = [o + i for o, i in zip(wo, idx)]
            blocks_from_weights.add(tuple(x // b for x, b in zip(g, block)))
        blocks_held = set(tuple(o + i for o, i in zip(so, idx)) for idx in np.ndindex(*sl))
        if blocks_from_weights != blocks_held:
            return False
    return True


def dequantize(w_bytes, scales, block):
    """float64 values of E4M3 weight bytes [..., N, K] with block scales."""
    v = mxfp8.e4m3_decode(w_bytes)
    s = np.asarray(scales, dtype=np.float64)
    for d, b in enumerate(block):
        if b > 1:
            s = np.repeat(s, b, axis=d)
    s = s[tuple(slice(0, n) for n in w_bytes.shape)]
    return v * s
