"""CPU oracle for whole-block maintenance of paged KV caches.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package: only tests/,
``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may use it).

A region is one cache seen as bytes: block b of a region is the byte range
[b * block_stride, b * block_stride + block_bytes).  Both functions are the
definition written out with numpy slicing, region by region, item by item:

  zero_blocks  -- vLLM v0.17.1 release notes, fix #35219: newly allocated
                  attention blocks are cleared on the GPU before use, in every
                  cache of the pool.  Every listed block of every region
                  becomes zero bytes; nothing else changes.
  copy_blocks  -- copy-on-write of a shared block (vLLM internals blog,
                  section 1, page-table analogy and figure 1) and swap out /
                  swap in of a preempted sequence's blocks (vLLM concept page,
                  "15-minute deep dive", scheduler item): block src of every
                  source region is copied over block dst of the matching
                  destination region.  All copies read the sources as they
                  were before the call.

Ids outside [0, num_blocks) are skipped and reported with the block-id error
bit (0x1), as the GPU library documents.  Parity pinned in
tests/test_oracle_blocks.py (a byte-by-byte membership definition, closed-form
special cases, round trips).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

DEVERR_BLOCK_ID = 0x1


def _as_bytes(region) -> np.ndarray:
    a = np.asarray(region)
    return a.reshape(-1).view(np.uint8)


def zero_blocks(regions: Sequence, block_ids, block_stride: int, block_bytes: int,
                num_blocks: int) -> Tuple[List[np.ndarray], int]:
    """Copies of ``regions`` (byte arrays) with every listed block cleared, and
    the error bits the call raises."""
    out = [_as_bytes(r).copy() for r in regions]
    flag = 0
    for b in np.asarray(block_ids, dtype=np.int64).reshape(-1):
        if b < 0 or b >= num_blocks:
            flag |= DEVERR_BLOCK_ID
            continue
        for r in out:
            r[b * block_stride:b * block_stride + block_bytes] = 0
    return out, flag


def copy_blocks(src_regions: Sequence, dst_regions: Sequence, block_pairs, block_stride: int,
                block_bytes: int, src_num_blocks: int,
                dst_num_blocks: int) -> Tuple[List[np.ndarray], int]:
    """Copies of ``dst_regions`` after copying every valid (src, dst) pair, and
    the error bits the call raises."""
    src = [_as_bytes(r).copy() for r in src_regions]
    out = [_as_bytes(r).copy() for r in dst_regions]
    flag = 0
    for s, d in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        if s < 0 or s >= src_num_blocks or d < 0 or d >= dst_num_blocks:
            flag |= DEVERR_BLOCK_ID
            continue
        for rs, rd in zip(src, out):
            rd[d * block_stride:d * block_stride + block_bytes] = \
                rs[s * block_stride:s * block_stride + block_bytes]
    return out, flag
