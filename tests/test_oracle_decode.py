"""Pins for the oracle's paged decode attention.

Each test checks the oracle against something other than itself: a 50-digit
decimal brute force, torch's fp64 scaled_dot_product_attention on K/V laid out
contiguously by numpy indexing, closed forms (one token, constant V, zero
scale), invariants the pages state (physical placement does not matter,
shared prefix blocks, unused tail slots) and the block-table figures printed
on the pages (tests/golden/).
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def contiguous_kv(cache, tables, lens, s, bs):
    """[L, Hkv, D] float64: the logical rows of sequence s, gathered by numpy
    fancy indexing from flat slot numbers (block * bs + offset)."""
    L = int(lens[s])
    pos = np.arange(L)
    slots = tables[s, pos // bs].astype(np.int64) * bs + pos % bs
    flat = cache.reshape(-1, cache.shape[2], cache.shape[3])
    return flat[slots]


def as_f64(t):
    return t.to(torch.float64).numpy() if torch.is_tensor(t) else np.asarray(t, np.float64)


def sdpa_reference(q, kc, vc, tables, lens, scale):
    """torch fp64 SDPA per sequence over K/V built by ``contiguous_kv``;
    query head h uses KV head h // G."""
    q = as_f64(q)
    kc, vc = as_f64(kc), as_f64(vc)
    tables, lens = np.asarray(tables), np.asarray(lens)
    S, H, D = q.shape
    Hkv = kc.shape[2]
    G = H // Hkv
    bs = kc.shape[1]
    out = np.zeros((S, H, D))
    for s in range(S):
        K = contiguous_kv(kc, tables, lens, s, bs)   # [L, Hkv, D]
        V = contiguous_kv(vc, tables, lens, s, bs)
        kv_of = np.arange(H) // G
        Kh = torch.from_numpy(np.ascontiguousarray(K[:, kv_of, :].transpose(1, 0, 2)))
        Vh = torch.from_numpy(np.ascontiguousarray(V[:, kv_of, :].transpose(1, 0, 2)))
        qh = torch.from_numpy(np.ascontiguousarray(q[s][:, None, :]))   # [H, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qh, Kh, Vh, scale=scale)
        out[s] = o[:, 0, :].numpy()
    return out


def tiny_case(rng, S, H, Hkv, D, bs, max_len, NB=None, dyadic=True):
    lens = rng.integers(1, max_len + 1, size=S).astype(np.int32)
    max_nb = -(-max_len // bs)
    nblk = -(-lens // bs)
    NB = NB or int(nblk.sum()) + 3
    perm = rng.permutation(NB)
    tables = np.full((S, max_nb), -1, np.int32)
    c = 0
    for s in range(S):
        tables[s, :nblk[s]] = perm[c:c + nblk[s]]
        c += nblk[s]
    def draw(shape):
        if dyadic:
            return (rng.integers(-16, 17, size=shape) / 8.0).astype(np.float32)
        return rng.standard_normal(shape).astype(np.float32)
    q = draw((S, H, D))
    kc = draw((NB, bs, Hkv, D))
    vc = draw((NB, bs, Hkv, D))
    return q, kc, vc, tables, lens


# ----------------------------------------------------------------- brute force
def decimal_attention(q, kc, vc, tables, lens, scale):
    """Attention written out in 50-digit decimal arithmetic."""
    getcontext().prec = 50
    S, H, D = q.shape
    Hkv, bs = kc.shape[2], kc.shape[1]
    G = H // Hkv
    out = np.zeros((S, H, D))
    sc = Decimal(repr(float(scale)))
    for s in range(S):
        L = int(lens[s])
        for h in range(H):
            kv = h // G
            rows = [(int(tables[s, t // bs]), t % bs) for t in range(L)]
            z = [sc * sum(Decimal(float(q[s, h, d])) * Decimal(float(kc[b, o, kv, d]))
                          for d in range(D)) for (b, o) in rows]
            m = max(z)
            e = [(zi - m).exp() for zi in z]
            tot = sum(e)
            for d in range(D):
                out[s, h, d] = float(sum(ei * Decimal(float(vc[b, o, kv, d]))
                                         for ei, (b, o) in zip(e, rows)) / tot)
    return out


@pytest.mark.parametrize("seed,S,H,Hkv,D,bs,max_len", [
    (1, 2, 2, 2, 4, 2, 7),     # MHA, odd lengths
    (2, 3, 4, 2, 8, 4, 11),    # GQA 2, partial last blocks
    (3, 2, 4, 1, 8, 4, 9),     # MQA
    (4, 1, 3, 1, 5, 2, 5),     # odd head_dim
])
def test_brute_force_decimal(seed, S, H, Hkv, D, bs, max_len):
    rng = np.random.default_rng(seed)
    q, kc, vc, tables, lens = tiny_case(rng, S, H, Hkv, D, bs, max_len)
    scale = 1 / math.sqrt(D)
    ours = oracle.decode(q, kc, vc, tables, lens, scale)
    ref = decimal_attention(q, kc, vc, tables, lens, scale)
    assert np.max(np.abs(ours - ref)) <= 1e-13


# ----------------------------------------------------------------- library routine
@pytest.mark.parametrize("name,over", [
    ("tiny_f32", {}),
    ("llama3_8b_bf16", dict(num_seqs=3, lens=("uniform", 1, 90), max_len=90)),
    ("qwen3_0p6b_bf16", dict(num_seqs=4, lens=("uniform", 30, 70), max_len=70)),
    ("shared_prefix_bf16", dict(num_seqs=3, lens=("prefix", 32, 1, 20), max_len=52)),
])
def test_matches_torch_sdpa_fp64(name, over):
    b = workloads.make_batch(name, **over)
    ours = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    ref = sdpa_reference(b.q, b.key_pool, b.value_pool, b.block_tables.numpy(),
                         b.seq_lens.numpy(), b.scale)
    assert np.max(np.abs(ours - ref)) <= 1e-12


def test_fp8_cache_matches_sdpa_on_dequantised_values():
    b = workloads.make_batch("long_fp8", num_seqs=2, lens=("uniform", 40, 120), max_len=128)
    kc = torch.randint(0, 256, b.key_pool.shape, dtype=torch.uint8,
                       generator=torch.Generator().manual_seed(3))
    kc[(kc & 0x7F) == 0x7F] = 0x11                     # no NaN codes in readable slots
    vc = torch.flip(kc, dims=[0])
    ks, vs = 0.0125, 0.03
    deq = lambda c, s: c.view(torch.float8_e4m3fn).to(torch.float64) * s   # torch's own decode
    ours = oracle.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, k_scale=ks, v_scale=vs)
    ref = sdpa_reference(b.q, deq(kc, ks), deq(vc, vs), b.block_tables.numpy(),
                         b.seq_lens.numpy(), b.scale)
    assert np.max(np.abs(ours - ref)) <= 1e-12


# ----------------------------------------------------------------- closed forms / invariants
def test_weights_sum_to_one_and_reproduce_output():
    b = workloads.make_batch("tiny_f32")
    out, w = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale,
                           with_weights=True)
    S, H = b.num_seqs, b.num_heads
    lens = b.seq_lens.numpy()
    vc = b.value_pool.numpy()
    for r in range(S * H):
        s, h = divmod(r, H)
        L = lens[s]
        p = w[r, :L]
        assert np.all(p >= 0) and abs(p.sum() - 1.0) <= 1e-12
        assert np.all(np.isnan(w[r, L:]))
        V = contiguous_kv(vc, b.block_tables.numpy(), lens, s, b.block_size)[:, h // (H // b.num_kv_heads)]
        assert np.max(np.abs(p @ V - out[s, h])) <= 1e-12


def test_single_token_returns_v_exactly():
    b = workloads.make_batch("tiny_f32", lens=("fixed", 1))
    out = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    G = b.group_size
    for s in range(b.num_seqs):
        blk = int(b.block_tables[s, 0])
        for h in range(b.num_heads):
            assert np.array_equal(out[s, h], b.value_pool[blk, 0, h // G].double().numpy())


def test_constant_v_gives_that_constant():
    b = workloads.make_batch("tiny_f32")
    for c in (0.7, -3.25, 1e-3):
        vc = torch.full_like(b.value_pool, c)
        out = oracle.decode(b.q, b.key_pool, vc, b.block_tables, b.seq_lens, b.scale)
        cf = float(np.float32(c))
        assert np.max(np.abs(out - cf)) <= 1e-15 * abs(cf) * 4


def test_zero_scale_gives_mean_of_v():
    b = workloads.make_batch("tiny_f32")
    out = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, 0.0)
    lens = b.seq_lens.numpy()
    for s in range(b.num_seqs):
        V = contiguous_kv(b.value_pool.double().numpy(), b.block_tables.numpy(), lens, s,
                          b.block_size)
        for h in range(b.num_heads):
            assert np.max(np.abs(out[s, h] - V[:, h // b.group_size].mean(axis=0))) <= 1e-14


def test_physical_placement_does_not_change_result_bitwise():
    b = workloads.make_batch("tiny_f32")
    base = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    rng = np.random.default_rng(11)
    for _ in range(3):
        perm = rng.permutation(b.num_blocks)          # old block i -> new position perm[i]
        kc = torch.empty_like(b.key_pool)
        vc = torch.empty_like(b.value_pool)
        kc[perm] = b.key_pool
        vc[perm] = b.value_pool
        tbl = b.block_tables.numpy().copy()
        used = tbl >= 0
        tbl[used] = perm[tbl[used]]
        out = oracle.decode(b.q, kc, vc, tbl, b.seq_lens, b.scale)
        assert np.array_equal(out, base)


def test_gqa_equals_mha_with_replicated_kv_heads():
    b = workloads.make_batch("llama3_8b_bf16", num_seqs=3, lens=("uniform", 1, 70), max_len=70)
    G = b.group_size
    base = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    kc = b.key_pool.repeat_interleave(G, dim=2).contiguous()
    vc = b.value_pool.repeat_interleave(G, dim=2).contiguous()
    out = oracle.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale)
    assert np.array_equal(out, base)
    # and a different head mapping (h % Hkv) would give a different answer
    kc2 = b.key_pool.repeat(1, 1, G, 1).contiguous()
    vc2 = b.value_pool.repeat(1, 1, G, 1).contiguous()
    alt = oracle.decode(b.q, kc2, vc2, b.block_tables, b.seq_lens, b.scale)
    assert not np.allclose(alt, base)


def test_shared_prefix_equals_private_copies():
    b = workloads.make_batch("shared_prefix_bf16", num_seqs=4, lens=("prefix", 64, 1, 40),
                             max_len=104)
    base = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    n_shared = 64 // b.block_size
    tbl = b.block_tables.numpy().copy()
    # give every sequence its own copy of the shared prefix blocks
    extra_k, extra_v = [], []
    nxt = b.num_blocks
    for s in range(b.num_seqs):
        for j in range(n_shared):
            extra_k.append(b.key_pool[tbl[s, j]])
            extra_v.append(b.value_pool[tbl[s, j]])
            tbl[s, j] = nxt
            nxt += 1
    kc = torch.cat([b.key_pool, torch.stack(extra_k)])
    vc = torch.cat([b.value_pool, torch.stack(extra_v)])
    assert len(np.unique(tbl[tbl >= 0])) == (tbl >= 0).sum()     # nothing shared any more
    out = oracle.decode(b.q, kc, vc, tbl, b.seq_lens, b.scale)
    assert np.array_equal(out, base)


def test_nan_in_unread_slots_does_not_leak():
    clean = workloads.make_batch("tiny_f32")
    dirty = workloads.make_batch("tiny_f32", poison=True)
    assert torch.isnan(dirty.key_pool).any()
    a = oracle.decode(clean.q, clean.key_pool, clean.value_pool, clean.block_tables,
                      clean.seq_lens, clean.scale)
    b = oracle.decode(dirty.q, dirty.key_pool, dirty.value_pool, dirty.block_tables,
                      dirty.seq_lens, dirty.scale)
    assert np.isfinite(b).all() and np.array_equal(a, b)


def test_tail_rows_are_excluded():
    """Changing a slot at position >= L of the last block changes nothing;
    changing the slot at position L-1 does."""
    b = workloads.make_batch("tiny_f32", lens=("fixed", 21))     # last block holds 5 of 16
    base = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    last = b.block_tables[:, 1].long()
    kc = b.key_pool.clone()
    kc[last, 5:] = 1e6
    assert np.array_equal(oracle.decode(b.q, kc, b.value_pool, b.block_tables, b.seq_lens,
                                        b.scale), base)
    kc[last, 4] = 5.0
    assert not np.allclose(oracle.decode(b.q, kc, b.value_pool, b.block_tables, b.seq_lens,
                                         b.scale), base)


def test_zero_length_row_is_zero():
    b = workloads.make_batch("tiny_f32")
    lens = b.seq_lens.clone()
    lens[1] = 0
    out = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, lens, b.scale)
    assert np.array_equal(out[1], np.zeros_like(out[1]))


def test_rows_subset_matches_full():
    b = workloads.make_batch("tiny_f32")
    full = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale)
    rows = [31, 0, 17, 9]
    part = oracle.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale,
                         rows=rows)
    assert np.array_equal(part, full.reshape(-1, b.head_dim)[rows])


def test_block_id_outside_pool_is_an_error():
    b = workloads.make_batch("tiny_f32")
    tbl = b.block_tables.clone()
    tbl[0, 0] = b.num_blocks
    with pytest.raises(ValueError):
        oracle.decode(b.q, b.key_pool, b.value_pool, tbl, b.seq_lens, b.scale)


# ----------------------------------------------------------------- the pages' figures
@pytest.mark.parametrize("fixture", ["page_table_concept.json", "block_pool_internals.json"])
def test_golden_block_tables(fixture):
    g = json.load(open(os.path.join(GOLDEN, fixture)))
    names = list(g["sequences"])
    tables = [g["sequences"][n] for n in names]
    used = sorted(b for t in tables for b in t)
    assert sorted(used + g["free_blocks"]) == list(range(g["pool_blocks"]))
    bs, Hkv, D, H = 4, 1, 8, 2
    rng = np.random.default_rng(5)
    # logical token t of sequence n carries values drawn for (n, t); the pool
    # holds them at the physical places the figure shows, free blocks hold NaN
    max_nb = max(len(t) for t in tables)
    logical_k = rng.standard_normal((len(names), max_nb * bs, Hkv, D)).astype(np.float32)
    logical_v = rng.standard_normal((len(names), max_nb * bs, Hkv, D)).astype(np.float32)
    kc = np.full((g["pool_blocks"], bs, Hkv, D), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    tbl = np.full((len(names), max_nb), -1, np.int32)
    for i, t in enumerate(tables):
        for j, phys in enumerate(t):
            kc[phys] = logical_k[i, j * bs:(j + 1) * bs]
            vc[phys] = logical_v[i, j * bs:(j + 1) * bs]
            tbl[i, j] = phys
    lens = np.array([len(t) * bs - 1 for t in tables], np.int32)    # last block not full
    q = rng.standard_normal((len(names), H, D)).astype(np.float32)
    out = oracle.decode(q, kc, vc, tbl, lens, 0.5)
    for i in range(len(names)):
        L = lens[i]
        Kh = torch.from_numpy(logical_k[i, :L, 0].astype(np.float64))[None].expand(H, L, D)
        Vh = torch.from_numpy(logical_v[i, :L, 0].astype(np.float64))[None].expand(H, L, D)
        qh = torch.from_numpy(q[i].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qh, Kh, Vh, scale=0.5)[:, 0]
        assert np.max(np.abs(out[i] - ref.numpy())) <= 1e-12
