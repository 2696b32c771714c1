"""CPU oracle for building one step's attention metadata from a persistent
per-request state table.

TEST INFRASTRUCTURE ONLY (only tests/, ``__graft_entry__.smoke()`` and
bench.py's ``cpu_baseline`` leg may use it).

What it computes (Model Runner V2 page, "better persistent batch and
GPU-native input preparation"; the same design on the page about vLLM's
model runner rewrite): every active request keeps a stable row of a fixed-size
state table -- here the number of its tokens already in the KV cache, its
block table and its token ids -- and each step gathers, in the step's request
order, the inputs of that step: query_start_loc, seq_lens, positions,
input_ids, the ordered block table and the slot of every new token.  Written
out as plain loops, in the order a reader would check them:

  for batch entry i (state row r = idx_mapping[i], n_i = num_scheduled[i]):
      query_start_loc[i+1] = query_start_loc[i] + n_i      (query_start_loc[0] = 0)
      seq_lens[i]          = num_computed[r] + n_i          (new tokens included)
      block_tables[i, :]   = state_block_table[r, :]
      for k in 0 .. n_i - 1, token t = query_start_loc[i] + k:
          positions[t]    = num_computed[r] + k
          input_ids[t]    = token_ids[r, positions[t]]
          slot_mapping[t] = block_tables[i, p // bs] * bs + p % bs,  p = positions[t]

Token rows beyond the step's total up to the outputs' capacity are padding:
slot -1 (an append skips them), position 0, input id 0.  Readings where the
pages are silent: a request whose new tokens would run past the outputs'
capacity has its count cut (and the later ones get none), raising error bit
0x20; an entry whose state row is outside the table, or whose count or
computed-token number is negative, contributes no tokens (0x20); a position
beyond the token table gives input id 0 (0x20); a block needed for a slot
that lies outside the table or the pool gives slot -1 (0x20 or 0x1).
Parity pinned in tests/test_oracle_step_prep.py.
"""
from __future__ import annotations

import numpy as np

DEVERR_BLOCK_ID = 0x1
DEVERR_STEP = 0x20


def prepare_step(idx_mapping, num_scheduled, num_computed, state_block_table, token_ids,
                 block_size: int, max_tokens: int, num_blocks: int):
    """Returns dict(query_start_loc, seq_lens, positions, input_ids, slot_mapping,
    block_tables, flag)."""
    idx = np.asarray(idx_mapping, dtype=np.int64)
    n_sched = np.asarray(num_scheduled, dtype=np.int64)
    computed = np.asarray(num_computed, dtype=np.int64)
    bt_state = np.asarray(state_block_table, dtype=np.int64)
    toks = np.asarray(token_ids, dtype=np.int64)
    S = idx.shape[0]
    R, max_nb = bt_state.shape
    max_len = toks.shape[1]
    flag = 0

    qsl = np.zeros(S + 1, dtype=np.int32)
    seq_lens = np.zeros(S, dtype=np.int32)
    tables = np.full((S, max_nb), -1, dtype=np.int32)
    positions = np.zeros(max_tokens, dtype=np.int64)
    input_ids = np.zeros(max_tokens, dtype=np.int32)
    slots = np.full(max_tokens, -1, dtype=np.int64)

    for i in range(S):
        r = idx[i]
        n = n_sched[i]
        if r < 0 or r >= R or n < 0 or computed[r] < 0:
            flag |= DEVERR_STEP
            qsl[i + 1] = qsl[i]
            continue
        room = max_tokens - qsl[i]
        if n > room:
            flag |= DEVERR_STEP
            n = room
        qsl[i + 1] = qsl[i] + n
        seq_lens[i] = computed[r] + n
        tables[i, :] = bt_state[r, :]
        for k in range(n):
            t = qsl[i] + k
            p = computed[r] + k
            positions[t] = p
            if p < max_len:
                input_ids[t] = toks[r, p]
            else:
                flag |= DEVERR_STEP
            j = p // block_size
            if j >= max_nb:
                flag |= DEVERR_STEP
                continue
            b = bt_state[r, j]
            if b < 0 or b >= num_blocks:
                flag |= DEVERR_BLOCK_ID
                continue
            slots[t] = b * block_size + p % block_size
    return dict(query_start_loc=qsl, seq_lens=seq_lens, positions=positions,
                input_ids=input_ids, slot_mapping=slots, block_tables=tables, flag=flag)
