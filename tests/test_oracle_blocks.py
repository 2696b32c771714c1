"""Pins of the block-maintenance oracle (oracle/blocks.py) against things
other than itself: the byte-by-byte definition (a byte is cleared exactly when
its block is listed and its offset lies inside the cleared part), closed-form
special cases (empty list, whole pool, duplicates, idempotence), and copy
round trips.  The pins are written as check functions so that planted
mistakes in a copy of the oracle can be shown to fail at least one of them.
"""
import importlib.util
import os
import tempfile

import numpy as np
import pytest

import oracle.blocks as blocks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "blocks.py")


def _regions(rng, R, NB, stride):
    return [rng.integers(1, 256, size=NB * stride, dtype=np.uint8) for _ in range(R)]


def check_bytewise_definition(mod):
    """Each byte (block x // stride, offset x % stride) is zero afterwards iff
    its block is a listed valid id and offset < block_bytes; others keep their
    value.  Inputs have no zero bytes, so every cleared byte is visible."""
    rng = np.random.default_rng(1)
    R, NB, stride, nbytes = 3, 11, 48, 32
    regs = _regions(rng, R, NB, stride)
    ids = np.array([7, 2, 2, 10, -1, 11, 0], dtype=np.int32)
    out, flag = mod.zero_blocks(regs, ids, stride, nbytes, NB)
    valid = {int(i) for i in ids if 0 <= i < NB}
    x = np.arange(NB * stride)
    cleared = np.isin(x // stride, sorted(valid)) & (x % stride < nbytes)
    for before, after in zip(regs, out):
        assert np.array_equal(after[cleared], np.zeros(cleared.sum(), np.uint8))
        assert np.array_equal(after[~cleared], before[~cleared])
    assert flag == blocks.DEVERR_BLOCK_ID


def check_special_cases(mod):
    rng = np.random.default_rng(2)
    R, NB, stride = 2, 6, 64
    regs = _regions(rng, R, NB, stride)
    out, flag = mod.zero_blocks(regs, np.array([], np.int32), stride, stride, NB)
    assert flag == 0 and all(np.array_equal(a, b) for a, b in zip(out, regs))
    out, flag = mod.zero_blocks(regs, np.arange(NB, dtype=np.int32), stride, stride, NB)
    assert flag == 0 and all(not a.any() for a in out)
    once, _ = mod.zero_blocks(regs, np.array([3, 1], np.int32), stride, 32, NB)
    dup, _ = mod.zero_blocks(regs, np.array([3, 1, 3, 1, 1], np.int32), stride, 32, NB)
    twice, _ = mod.zero_blocks(once, np.array([1, 3], np.int32), stride, 32, NB)
    for a, b, c in zip(once, dup, twice):
        assert np.array_equal(a, b) and np.array_equal(a, c)


def check_copy_matches_block_view(mod):
    """A copy equals assigning rows of the [NB, stride] view, reading the
    sources as they were (the pairs form a permutation of some blocks)."""
    rng = np.random.default_rng(3)
    R, NB, stride, nbytes = 2, 9, 32, 16
    src = _regions(rng, R, NB, stride)
    dst = _regions(rng, R, NB + 3, stride)
    pairs = np.array([[4, 0], [0, 11], [8, 4], [2, 9], [9, 1], [1, -2]], dtype=np.int32)
    out, flag = mod.copy_blocks(src, dst, pairs, stride, nbytes, NB, NB + 3)
    assert flag == blocks.DEVERR_BLOCK_ID
    for s_reg, d_reg, o_reg in zip(src, dst, out):
        sv, dv = s_reg.reshape(NB, stride), d_reg.reshape(NB + 3, stride).copy()
        for s, d in pairs:
            if 0 <= s < NB and 0 <= d < NB + 3:
                dv[d, :nbytes] = sv[s, :nbytes]
        assert np.array_equal(o_reg, dv.reshape(-1))


def check_swap_round_trip(mod):
    """Swap a set of device blocks out to host slots and back into other
    device blocks: the moved blocks equal the originals, the rest is intact."""
    rng = np.random.default_rng(4)
    R, NB, NH, stride = 3, 10, 4, 48
    dev = _regions(rng, R, NB, stride)
    host = [np.zeros(NH * stride, np.uint8) for _ in range(R)]
    out_pairs = np.array([[6, 0], [2, 3], [9, 1]], dtype=np.int32)
    host2, f1 = mod.copy_blocks(dev, host, out_pairs, stride, stride, NB, NH)
    in_pairs = np.array([[0, 1], [3, 4], [1, 5]], dtype=np.int32)
    dev2, f2 = mod.copy_blocks(host2, dev, in_pairs, stride, stride, NH, NB)
    assert f1 == 0 and f2 == 0
    for before, after in zip(dev, dev2):
        b, a = before.reshape(NB, stride), after.reshape(NB, stride)
        assert np.array_equal(a[[1, 4, 5]], b[[6, 2, 9]])
        keep = [i for i in range(NB) if i not in (1, 4, 5)]
        assert np.array_equal(a[keep], b[keep])


CHECKS = [check_bytewise_definition, check_special_cases, check_copy_matches_block_view,
          check_swap_round_trip]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(blocks)


MUTANTS = {
    "clears_whole_stride": ("r[b * block_stride:b * block_stride + block_bytes] = 0",
                            "r[b * block_stride:(b + 1) * block_stride] = 0"),
    "off_by_one_block": ("r[b * block_stride:b * block_stride + block_bytes] = 0",
                         "r[(b + 1) * block_stride:(b + 1) * block_stride + block_bytes] = 0"),
    "no_range_check": ("if b < 0 or b >= num_blocks:", "if False:"),
    "copy_swapped_roles": ("rd[d * block_stride:d * block_stride + block_bytes] = \\\n"
                           "                rs[s * block_stride:s * block_stride + block_bytes]",
                           "rd[s * block_stride:s * block_stride + block_bytes] = \\\n"
                           "                rs[d * block_stride:d * block_stride + block_bytes]"),
    "copy_checks_src_against_dst_pool": ("if s < 0 or s >= src_num_blocks or",
                                         "if s < 0 or s >= dst_num_blocks or"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "blocks_mutant.py")
        with open(path, "w") as f:
            f.write(text.replace(old, new))
        spec = importlib.util.spec_from_file_location("blocks_mutant", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        failed = []
        for check in CHECKS:
            try:
                check(mod)
            except (AssertionError, IndexError, ValueError):
                failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
