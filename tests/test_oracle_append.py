"""Pins for the oracle's KV-append scatter: numpy fancy indexing of flat slot
numbers for the bit-copy caches, and torch's float8_e4m3fn rounding (after the
binary32 multiply by 1/scale) for the 8-bit cache."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _expected_copy(cache, k, slots):
    exp = cache.clone()
    flat = exp.view(-1, cache.shape[2], cache.shape[3])
    keep = slots >= 0
    flat[slots[keep]] = k[keep]
    return exp


@pytest.mark.parametrize("name", ["tiny_f32", "llama3_8b_bf16"])
def test_bit_copy_append_writes_exactly_the_named_slots(name):
    b = workloads.make_batch(name, num_seqs=6, lens=("uniform", 1, 60), max_len=60)
    kc = b.key_pool.clone()
    vc = b.value_pool.clone()
    slots = b.slot_mapping.clone()
    slots[2] = -1                                       # padding token: skipped
    exp_k = _expected_copy(kc, b.k_new, slots)
    exp_v = _expected_copy(vc, b.v_new, slots)
    oracle.kv_append(b.k_new, b.v_new, slots, kc, vc)
    bits = torch.int32 if kc.dtype == torch.float32 else torch.int16
    assert torch.equal(kc.view(bits), exp_k.view(bits))
    assert torch.equal(vc.view(bits), exp_v.view(bits))


def test_append_then_decode_reads_the_new_row_last():
    b = workloads.make_batch("tiny_f32", lens=("fixed", 1))
    kc, vc = b.key_pool.clone(), b.value_pool.clone()
    oracle.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc)
    out = oracle.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale)
    G = b.group_size
    for s in range(b.num_seqs):
        for h in range(b.num_heads):
            assert np.array_equal(out[s, h], b.v_new[s, h // G].double().numpy())


@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float32])
def test_fp8_append_matches_torch_rounding(in_dtype):
    b = workloads.make_batch("long_fp8", num_seqs=5, lens=("uniform", 1, 90), max_len=96)
    T = 40
    gen = torch.Generator().manual_seed(9)
    k = (torch.randn((T, b.num_kv_heads, b.head_dim), generator=gen) * 3).to(in_dtype)
    v = (torch.randn((T, b.num_kv_heads, b.head_dim), generator=gen) * 0.01).to(in_dtype)
    k[0, 0, :4] = torch.tensor([float("nan"), 1e6, -1e6, 0.0])   # NaN kept, saturation
    slots = torch.randperm(b.num_blocks * b.block_size, generator=gen)[:T].to(torch.int64)
    ks, vs = 0.02, 3e-5
    kc = torch.full(b.key_pool.shape, 0x5A, dtype=torch.uint8)
    vc = torch.full(b.key_pool.shape, 0xA5, dtype=torch.uint8)
    exp_k, exp_v = kc.clone(), vc.clone()
    oracle.kv_append(k, v, slots, kc, vc, ks, vs)

    def torch_codes(x, scale):
        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
        y = x.to(torch.float32) * inv
        y = torch.where(torch.isnan(y), y, y.clamp(-448.0, 448.0))
        return y.to(torch.float8_e4m3fn).view(torch.uint8)

    exp_k.view(-1, b.num_kv_heads, b.head_dim)[slots] = torch_codes(k, ks)
    exp_v.view(-1, b.num_kv_heads, b.head_dim)[slots] = torch_codes(v, vs)
    nan_k = (exp_k & 0x7F) == 0x7F
    assert torch.equal(nan_k, (kc & 0x7F) == 0x7F)            # NaN where torch has NaN
    assert torch.equal(kc[~nan_k], exp_k[~nan_k])
    assert torch.equal(vc, exp_v)


def test_slot_outside_pool_is_an_error_and_writes_nothing():
    b = workloads.make_batch("tiny_f32")
    kc, vc = b.key_pool.clone(), b.value_pool.clone()
    slots = b.slot_mapping.clone()
    slots[-1] = b.num_blocks * b.block_size
    with pytest.raises(ValueError):
        oracle.kv_append(b.k_new, b.v_new, slots, kc, vc)
    assert torch.equal(kc, b.key_pool) and torch.equal(vc, b.value_pool)


def test_dtype_mismatch_is_an_error():
    b = workloads.make_batch("tiny_f32")
    with pytest.raises(ValueError):
        oracle.kv_append(b.k_new.to(torch.bfloat16), b.v_new.to(torch.bfloat16),
                         b.slot_mapping, b.key_pool.clone(), b.value_pool.clone())
