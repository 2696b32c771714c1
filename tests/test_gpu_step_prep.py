"""GPU parity of pa_prepare_step against the oracle (oracle/step_prep.py),
bit for bit on every output and on the error word: decode steps (one token per
request) and mixed steps (chunks of new tokens, requests without tokens),
shuffled state rows, padding up to the capacity, the capacity cut, bad
entries; and the outputs driving a whole step -- prepare, append, multi-token
decode -- checked against the oracle's attention."""
import numpy as np
import pytest
import torch

import oracle.step_prep as osp
import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def random_state(rng, R, max_nb, bs, NB, max_len):
    computed = rng.integers(0, max_len // 2, R).astype(np.int32)
    bt = rng.integers(0, NB, size=(R, max_nb)).astype(np.int32)
    toks = rng.integers(0, 150000, size=(R, max_len)).astype(np.int32)
    return computed, bt, toks


def run_both(idx, n, computed, bt, toks, bs, NB, max_tokens):
    want = osp.prepare_step(idx, n, computed, bt, toks, bs, max_tokens, NB)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    got = pa.prepare_step(d(idx), d(n), d(computed), d(bt), d(toks), bs, NB, max_tokens,
                          err_flag=flag)
    torch.cuda.synchronize()
    for k in ("query_start_loc", "seq_lens", "positions", "input_ids", "slot_mapping",
              "block_tables"):
        g = got[k].cpu().numpy()
        assert np.array_equal(g, want[k].astype(g.dtype)), k
    assert int(flag.item()) == want["flag"], (int(flag.item()), want["flag"])
    return got


@pytest.mark.parametrize("S,R,max_tokens,chunk", [
    (64, 100, 64, 1),          # decode step: one token each
    (64, 100, 80, 1),          # with padding
    (300, 512, 4096, 40),      # mixed chunks, several workgroups of token rows
    (2048, 2048, 2048, 1),     # the largest batch
    (7, 9, 200, 64),           # long chunks crossing blocks
])
def test_prepare_step_parity(S, R, max_tokens, chunk):
    rng = np.random.default_rng(S + R)
    bs, NB, max_nb = 16, 5000, 64
    computed, bt, toks = random_state(rng, R, max_nb, bs, NB, max_nb * bs)
    idx = rng.permutation(R)[:S].astype(np.int32)
    n = rng.integers(0 if chunk > 1 else 1, chunk + 1, S).astype(np.int32)
    n = np.minimum(n, max_nb * bs - computed[idx])
    print("CASE prep", S, R, max_tokens, chunk, flush=True)
    run_both(idx, n, computed, bt, toks, bs, NB, max_tokens)


def test_capacity_cut_and_bad_entries():
    rng = np.random.default_rng(7)
    bs, NB, max_nb, R = 16, 300, 8, 20
    computed, bt, toks = random_state(rng, R, max_nb, bs, NB, max_nb * bs)
    bt[3, :] = NB + 5                          # blocks outside the pool
    computed[4] = max_nb * bs - 2              # runs past the table
    idx = np.array([0, 3, 25, 4, 7, -1, 1], np.int32)
    n = np.array([5, 3, 2, 6, 4, 1, 50], np.int32)
    print("CASE prep violations", flush=True)
    run_both(idx, n, computed, bt, toks, bs, NB, 30)


def test_prepared_inputs_drive_a_verify_step():
    """State rows for a multi-token batch; prepare_step builds slots, lengths,
    tables and query layout; append and multi-token decode then run on
    them and match the oracle."""
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=12,
                             lens=("uniform", 1, 400), max_len=400, query_lens=("uniform", 0, 8),
                             seed=61)
    rng = np.random.default_rng(8)
    S = b.num_seqs
    lens = b.seq_lens.cpu().numpy()
    qlens = np.diff(b.query_start_loc.cpu().numpy())
    R = S + 6
    rows = rng.permutation(R)[:S].astype(np.int32)
    computed = np.zeros(R, np.int32)
    computed[rows] = lens - qlens
    bt = np.full((R, b.max_blocks_per_seq), -1, np.int32)
    bt[rows] = b.block_tables.cpu().numpy()
    toks = rng.integers(0, 1000, size=(R, b.max_blocks_per_seq * b.block_size)).astype(np.int32)
    T = int(qlens.sum())
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    print("CASE prep -> append -> decode_multi", flush=True)
    got = pa.prepare_step(d(rows), d(qlens.astype(np.int32)), d(computed), d(bt), d(toks),
                          b.block_size, b.num_blocks, T + 5)
    kc, vc = gpu_caches(b)
    k_new = torch.cat([b.k_new, torch.zeros_like(b.k_new[:5])])
    v_new = torch.cat([b.v_new, torch.zeros_like(b.v_new[:5])])
    pa.kv_append(k_new, v_new, got["slot_mapping"], kc, vc)       # padding rows skipped
    out = pa.decode_multi(b.q, got["query_start_loc"], 8, kc, vc, got["block_tables"],
                          got["seq_lens"], b.scale)
    torch.cuda.synchronize()
    ref, _, _ = oracle_step(b)
    check_close(out, ref, "bf16", "prepared verify step")
