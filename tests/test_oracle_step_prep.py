"""Pins of the step-metadata oracle (oracle/step_prep.py) against things other
than itself: the seeded workload generator's own slot mapping, lengths and
query layout (a separate derivation of the same quantities, from the block
placement it drew), vectorised numpy formulas for every output, closed-form
padding and capacity behaviour, and planted mistakes."""
import importlib.util
import os
import tempfile

import numpy as np
import pytest

import oracle.step_prep as sp
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "step_prep.py")


def state_from_batch(b, rng, R_extra=5):
    """A state table holding the batch's requests at shuffled rows (plus
    unused rows), each with L - q_len tokens computed, and random token ids."""
    S = b.num_seqs
    lens = b.seq_lens.cpu().numpy().astype(np.int64)
    qsl = (b.query_start_loc.cpu().numpy() if b.query_start_loc is not None
           else np.arange(S + 1))
    qlens = np.diff(qsl)
    R = S + R_extra
    rows = rng.permutation(R)[:S]
    computed = np.zeros(R, np.int32)
    computed[rows] = lens - qlens
    bt = np.full((R, b.max_blocks_per_seq), -1, np.int32)
    bt[rows] = b.block_tables.cpu().numpy()
    toks = rng.integers(0, 50000, size=(R, b.max_blocks_per_seq * b.block_size), dtype=np.int32)
    return rows.astype(np.int32), qlens.astype(np.int32), computed, bt, toks


def check_reproduces_generator(mod):
    rng = np.random.default_rng(1)
    for over in (dict(), dict(query_lens=("uniform", 0, 6))):
        name = "llama3_8b_bf16_spec8" if over else "llama3_8b_bf16"
        b = workloads.make_batch(name, num_seqs=9, lens=("uniform", 1, 200), max_len=208,
                                 seed=3, **over)
        rows, qlens, computed, bt, toks = state_from_batch(b, rng)
        T = int(qlens.sum())
        out = mod.prepare_step(rows, qlens, computed, bt, toks, b.block_size, T + 7, b.num_blocks)
        assert out["flag"] == 0
        assert np.array_equal(out["seq_lens"], b.seq_lens.cpu().numpy())
        assert np.array_equal(out["block_tables"], b.block_tables.cpu().numpy())
        assert np.array_equal(out["slot_mapping"][:T], b.slot_mapping.cpu().numpy())
        if b.query_start_loc is not None:
            assert np.array_equal(out["query_start_loc"], b.query_start_loc.cpu().numpy())
        assert (out["slot_mapping"][T:] == -1).all() and (out["positions"][T:] == 0).all()
        assert (out["input_ids"][T:] == 0).all()


def check_vectorised_definition(mod):
    rng = np.random.default_rng(2)
    R, max_nb, bs, NB = 12, 6, 4, 40
    computed = rng.integers(0, 15, R).astype(np.int32)
    bt = rng.integers(0, NB, size=(R, max_nb)).astype(np.int32)
    toks = rng.integers(0, 1000, size=(R, max_nb * bs)).astype(np.int32)
    idx = rng.permutation(R)[:7].astype(np.int32)
    n = rng.integers(0, 6, 7).astype(np.int32)
    n = np.minimum(n, max_nb * bs - computed[idx])
    out = mod.prepare_step(idx, n, computed, bt, toks, bs, 64, NB)
    T = int(n.sum())
    qsl = np.concatenate([[0], np.cumsum(n)])
    assert np.array_equal(out["query_start_loc"], qsl)
    assert np.array_equal(out["seq_lens"], computed[idx] + n)
    assert np.array_equal(out["block_tables"], bt[idx])
    seq_of = np.repeat(np.arange(7), n)
    pos = computed[idx][seq_of] + np.arange(T) - qsl[:-1][seq_of]
    assert np.array_equal(out["positions"][:T], pos)
    assert np.array_equal(out["input_ids"][:T], toks[idx[seq_of], pos])
    assert np.array_equal(out["slot_mapping"][:T],
                          bt[idx[seq_of], pos // bs].astype(np.int64) * bs + pos % bs)
    assert out["flag"] == 0


def check_capacity_and_bad_entries(mod):
    R, max_nb, bs, NB = 4, 4, 4, 16
    computed = np.array([2, 0, 5, 1], np.int32)
    bt = np.arange(R * max_nb, dtype=np.int32).reshape(R, max_nb)
    bt[3, 1] = NB + 3                               # outside the pool
    toks = np.arange(R * max_nb * bs, dtype=np.int32).reshape(R, -1)
    out = mod.prepare_step(np.array([1, 0, 2], np.int32), np.array([3, 4, 5], np.int32),
                           computed, bt, toks, bs, 9, NB)
    assert list(out["query_start_loc"]) == [0, 3, 7, 9]   # last entry cut from 5 to 2
    assert list(out["seq_lens"]) == [3, 6, 7]
    assert out["flag"] == sp.DEVERR_STEP
    out = mod.prepare_step(np.array([3, 9, 0], np.int32), np.array([6, 2, 1], np.int32),
                           computed, bt, toks, bs, 16, NB)
    assert list(out["query_start_loc"]) == [0, 6, 6, 7]   # row 9 does not exist
    assert list(out["slot_mapping"][:7]) == [49, 50, 51, -1, -1, -1, 2]
    assert out["flag"] == sp.DEVERR_STEP | sp.DEVERR_BLOCK_ID
    assert list(out["block_tables"][1]) == [-1] * max_nb


CHECKS = [check_reproduces_generator, check_vectorised_definition,
          check_capacity_and_bad_entries]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(sp)


MUTANTS = {
    "position_off_by_one": ("            p = computed[r] + k\n", "            p = computed[r] + k + 1\n"),
    "row_not_gathered": ("        tables[i, :] = bt_state[r, :]", "        tables[i, :] = bt_state[i, :]"),
    "seq_len_without_new": ("        seq_lens[i] = computed[r] + n", "        seq_lens[i] = computed[r]"),
    "slot_next_block": ("            j = p // block_size\n", "            j = p // block_size + 1\n"),
    "scan_drops_previous": ("        qsl[i + 1] = qsl[i] + n\n", "        qsl[i + 1] = n\n"),
    "no_capacity_cut": ("        if n > room:", "        if False:"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "prep_mutant.py")
        with open(path, "w") as f:
            f.write(text.replace(old, new))
        spec = importlib.util.spec_from_file_location("prep_mutant", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        failed = []
        for check in CHECKS:
            try:
                check(mod)
            except (AssertionError, IndexError, ValueError):
                failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
