"""The path in caches larger than 4 GiB: every block a batch names lies past
byte 2^32 of its cache, so any 32-bit byte offset in the append, the block
walk, the buffer resources or the block operations would read or write the
wrong place.  Each case builds a small batch, places its pool at the end of
a > 4 GiB cache (block ids shifted, slots shifted by the same number of
blocks) and checks the result against the oracle on the small batch, or the
cache bytes against the same operation on the small pool."""
import pytest
import torch

import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _big(b):
    """The batch's device caches placed past 4 GiB, and its tables and slots
    shifted to match."""
    kc, vc = gpu_caches(b)
    block_bytes = kc[0].numel() * kc.element_size()
    off = (1 << 32) // block_bytes + 97          # first block id of the batch's pool
    shape = (off + kc.shape[0],) + tuple(kc.shape[1:])
    big_k = torch.empty(shape, dtype=kc.dtype, device=DEV)
    big_v = torch.empty(shape, dtype=vc.dtype, device=DEV)
    big_k[off:] = kc
    big_v[off:] = vc
    assert off * block_bytes >= 1 << 32 and big_k.numel() * big_k.element_size() > 1 << 32
    bt = torch.where(b.block_tables >= 0, b.block_tables + off, b.block_tables)
    slots = torch.where(b.slot_mapping >= 0, b.slot_mapping + off * b.block_size,
                        b.slot_mapping)
    return big_k, big_v, bt, slots, off, (kc, vc)


@pytest.mark.parametrize("base,variant", [("llama3_8b_bf16", pa.VARIANT_MFMA),
                                          ("llama3_8b_bf16", pa.VARIANT_VALU),
                                          ("long_fp8", pa.VARIANT_MFMA)])
def test_append_and_decode_past_4gib(base, variant):
    b = workloads.make_batch(base, device=DEV, num_seqs=6, num_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=16, lens=("uniform", 1, 300), max_len=300,
                             pool=("factor", 1.2), seed=71)
    ref, _, _ = oracle_step(b)
    print("CASE >4GiB decode", base, "variant", variant, flush=True)
    big_k, big_v, bt, slots, off, (kc, vc) = _big(b)
    pa.kv_append(b.k_new, b.v_new, slots, big_k, big_v, b.k_scale, b.v_scale)
    pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, b.k_scale, b.v_scale)
    out = pa.decode(b.q, big_k, big_v, bt, b.seq_lens, b.scale, k_scale=b.k_scale,
                    v_scale=b.v_scale, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(big_k[off:], kc) and torch.equal(big_v[off:], vc), "append bytes"
    check_close(out, ref, b.cache_dtype, f">4GiB decode {base} variant {variant}")


def test_multi_token_and_cascade_past_4gib():
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=5, num_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16,
                             lens=("uniform", 8, 260), max_len=260, seed=72)
    ref, _, _ = oracle_step(b)
    print("CASE >4GiB multi-token", flush=True)
    big_k, big_v, bt, slots, off, _ = _big(b)
    pa.kv_append(b.k_new, b.v_new, slots, big_k, big_v, b.k_scale, b.v_scale)
    out = pa.decode_multi(b.q, b.query_start_loc, b.max_query_len, big_k, big_v, bt,
                          b.seq_lens, b.scale)
    torch.cuda.synchronize()
    check_close(out, ref, b.cache_dtype, ">4GiB multi-token")
    del big_k, big_v

    c = workloads.make_batch("shared_prefix_bf16", device=DEV, num_seqs=12,
                             lens=("prefix", 160, 1, 90), max_len=160 + 96, seed=73)
    ref, _, _ = oracle_step(c)
    print("CASE >4GiB cascade", flush=True)
    big_k, big_v, bt, slots, off, _ = _big(c)
    pa.kv_append(c.k_new, c.v_new, slots, big_k, big_v, c.k_scale, c.v_scale)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pa.decode_cascade(c.q, big_k, big_v, bt, c.seq_lens, c.shared_prefix_blocks, c.scale,
                            err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    check_close(out, ref, c.cache_dtype, ">4GiB cascade")


def test_block_clear_and_copy_past_4gib():
    """Clear and copy blocks whose bytes start past 4 GiB, in two caches at
    once; every other byte of the touched blocks' neighbours stays."""
    per = (1 << 32) // (16 * 8 * 128 * 2) + 200
    caches = [torch.full((per, 16, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
              for _ in range(2)]
    regs = pa.region_table(caches)
    ids = torch.tensor([per - 1, per - 5, per - 150], dtype=torch.int32, device=DEV)
    print("CASE >4GiB block clear", flush=True)
    pa.zero_blocks(ids, regs)
    torch.cuda.synchronize()
    for cache in caches:
        assert not cache[ids.long()].any()
        assert (cache[per - 2] == 3).all() and (cache[per - 151] == 3).all()
    caches[0][per - 7] = 5.0
    pairs = torch.tensor([[per - 7, per - 3]], dtype=torch.int32, device=DEV)
    print("CASE >4GiB block copy", flush=True)
    pa.copy_blocks(pairs, regs, regs)
    torch.cuda.synchronize()
    assert (caches[0][per - 3] == 5).all() and (caches[1][per - 3] == 3).all()
