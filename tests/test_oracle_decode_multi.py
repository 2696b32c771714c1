"""Pins for the oracle's multi-token decode (several new query tokens per
sequence, each attending causally): torch's fp64 scaled_dot_product_attention
with an explicit causal mask over K/V laid out by numpy indexing, a 50-digit
decimal brute force, closed forms (a sequence made only of new tokens: its
first token sees only itself, so its output is exactly V[0]), the reduction
to one new token, and the invariants of the paged layout."""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from test_oracle_decode import as_f64, contiguous_kv, tiny_case


def multi_case(rng, S, H, Hkv, D, bs, max_len, qmax, dyadic=True):
    q1, kc, vc, tables, lens = tiny_case(rng, S, H, Hkv, D, bs, max_len, dyadic=dyadic)
    qlens = np.array([rng.integers(0, min(qmax, int(L)) + 1) for L in lens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    if dyadic:
        q = (rng.integers(-16, 17, size=(T, H, D)) / 8.0).astype(np.float32)
    else:
        q = rng.standard_normal((T, H, D)).astype(np.float32)
    return q, qsl, kc, vc, tables, lens


def sdpa_causal(q, qsl, kc, vc, tables, lens, scale):
    """torch fp64 SDPA per sequence: the q_len queries against all L keys with
    mask[i, t] = t <= L - q_len + i."""
    q, kc, vc = as_f64(q), as_f64(kc), as_f64(vc)
    T, H, D = q.shape
    Hkv, bs = kc.shape[2], kc.shape[1]
    G = H // Hkv
    out = np.zeros((T, H, D))
    for s in range(len(lens)):
        L, a, b = int(lens[s]), int(qsl[s]), int(qsl[s + 1])
        ql = b - a
        if ql == 0:
            continue
        K = contiguous_kv(kc, tables, lens, s, bs)
        V = contiguous_kv(vc, tables, lens, s, bs)
        kv_of = np.arange(H) // G
        Kh = torch.from_numpy(np.ascontiguousarray(K[:, kv_of, :].transpose(1, 0, 2)))
        Vh = torch.from_numpy(np.ascontiguousarray(V[:, kv_of, :].transpose(1, 0, 2)))
        qh = torch.from_numpy(np.ascontiguousarray(q[a:b].transpose(1, 0, 2)))   # [H, ql, D]
        mask = torch.from_numpy(np.arange(L)[None, :] <= (L - ql + np.arange(ql))[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(qh, Kh, Vh, attn_mask=mask,
                                                             scale=scale)
        out[a:b] = o.numpy().transpose(1, 0, 2)
    return out


@pytest.mark.parametrize("seed,S,H,Hkv,D,bs,max_len,qmax", [
    (11, 3, 8, 2, 16, 4, 40, 5),
    (12, 4, 4, 4, 8, 2, 23, 8),
    (13, 2, 16, 2, 32, 16, 90, 16),
    (14, 5, 2, 1, 8, 4, 12, 12),        # q_len up to L: whole sequences of new tokens
])
def test_matches_causal_sdpa_fp64(seed, S, H, Hkv, D, bs, max_len, qmax):
    rng = np.random.default_rng(seed)
    q, qsl, kc, vc, tables, lens = multi_case(rng, S, H, Hkv, D, bs, max_len, qmax, dyadic=False)
    got = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.3)
    ref = sdpa_causal(q, qsl, kc, vc, tables, lens, 0.3)
    assert np.abs(got - ref).max() <= 1e-12


def decimal_multi(q, qsl, kc, vc, tables, lens, scale):
    getcontext().prec = 50
    T, H, D = q.shape
    Hkv, bs = kc.shape[2], kc.shape[1]
    G = H // Hkv
    out = np.zeros((T, H, D))
    sc = Decimal(repr(float(scale)))
    for s in range(len(lens)):
        L, a, b = int(lens[s]), int(qsl[s]), int(qsl[s + 1])
        for i, tok in enumerate(range(a, b)):
            vis = L - (b - a) + i + 1
            rows = [(int(tables[s, t // bs]), t % bs) for t in range(vis)]
            for h in range(H):
                kv = h // G
                z = [sc * sum(Decimal(float(q[tok, h, d])) * Decimal(float(kc[bb, o, kv, d]))
                              for d in range(D)) for (bb, o) in rows]
                m = max(z)
                e = [(zi - m).exp() for zi in z]
                tot = sum(e)
                for d in range(D):
                    out[tok, h, d] = float(sum(ei * Decimal(float(vc[bb, o, kv, d]))
                                               for ei, (bb, o) in zip(e, rows)) / tot)
    return out


def test_brute_force_decimal():
    rng = np.random.default_rng(21)
    q, qsl, kc, vc, tables, lens = multi_case(rng, 3, 4, 2, 4, 2, 7, 4)
    got = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.5)
    ref = decimal_multi(q, qsl, kc, vc, tables, lens, 0.5)
    assert np.abs(got - ref).max() <= 1e-13


def test_first_of_all_new_tokens_returns_v0_exactly():
    """q_len = L: token 0 of the sequence sees only position 0."""
    rng = np.random.default_rng(22)
    q1, kc, vc, tables, lens = tiny_case(rng, 3, 4, 2, 8, 4, 20, dyadic=False)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), 4, 8)).astype(np.float32)
    got = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.7)
    for s in range(3):
        V = contiguous_kv(as_f64(vc), tables, lens, s, 4)
        for h in range(4):
            assert np.array_equal(got[qsl[s], h], V[0, h // 2])


def test_one_new_token_equals_single_token_decode():
    rng = np.random.default_rng(23)
    q, kc, vc, tables, lens = tiny_case(rng, 4, 8, 2, 16, 4, 50, dyadic=False)
    qsl = np.arange(5, dtype=np.int32)
    got = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.25)
    ref = oracle.decode(q, kc, vc, tables, lens, 0.25)
    assert np.array_equal(got, ref)


def test_query_token_equals_decode_over_its_prefix():
    """Token i of q_len equals single-token decode with seq_len cut to
    L - q_len + i + 1 (the definition of causal visibility)."""
    rng = np.random.default_rng(24)
    q, qsl, kc, vc, tables, lens = multi_case(rng, 3, 4, 1, 8, 4, 30, 6, dyadic=False)
    got = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.4)
    for s in range(3):
        ql = int(qsl[s + 1] - qsl[s])
        for i in range(ql):
            cut = lens.copy()
            cut[s] = lens[s] - ql + i + 1
            one = oracle.decode(q[qsl[s] + i][None].repeat(3, 0), kc, vc, tables, cut, 0.4)
            assert np.array_equal(got[qsl[s] + i], one[s])


def test_physical_placement_is_bitwise_irrelevant_and_rows_subset():
    rng = np.random.default_rng(25)
    q, qsl, kc, vc, tables, lens = multi_case(rng, 3, 4, 2, 8, 4, 33, 5, dyadic=False)
    base = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.5)
    NB = kc.shape[0]
    perm = rng.permutation(NB)                      # block b moves to perm[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    moved = oracle.decode_multi(q, qsl, kc2, vc2, tables2, lens, 0.5)
    assert np.array_equal(base, moved)
    rows = [1, 5, 9, int(qsl[-1]) * 4 - 1]
    sub = oracle.decode_multi(q, qsl, kc, vc, tables, lens, 0.5, rows=rows)
    assert np.array_equal(sub, base.reshape(-1, 8)[rows])


def test_bad_query_layout_is_an_error():
    rng = np.random.default_rng(26)
    q, qsl, kc, vc, tables, lens = multi_case(rng, 2, 2, 1, 8, 4, 10, 3)
    bad = qsl.copy()
    bad[-1] += 1
    with pytest.raises(ValueError):
        oracle.decode_multi(q, bad, kc, vc, tables, lens, 0.5)
    too_many = np.array([0, int(lens[0]) + 1, int(lens[0]) + 1], np.int32)
    qq = np.zeros((int(lens[0]) + 1, 2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.decode_multi(qq, too_many, kc, vc, tables, lens, 0.5)
