"""GPU parity of pa_decode_cascade (shared prefix read once per group of
sequences, then each sequence's own blocks, joined by log-sum-exp) against
the oracle, and against pa_decode on the same caches: bf16 and e4m3 caches,
group sizes 1 to 8, head_dim 64 and 128, block sizes 16 and 32, sequences
ending exactly at the prefix, sequences whose own blocks span several
block-table windows, batches whose query rows do not fill the last
row block of the prefix pass, prefixes split over several token ranges, work
splits, NaN in unread slots,
the full-size shared-prefix batch on every row, and a broken contract
flagged."""
import pytest
import torch

import oracle
import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # heads, kv heads, head_dim, block size, prefix tokens, suffix range, sequences
    (32, 8, 128, 16, 160, (1, 100), 21),   # G 4: 16 sequences per prefix group, 2 groups
    (16, 2, 64, 32, 64, (0, 70), 9),       # G 8, D 64; some sequences end at the prefix
    (8, 8, 128, 16, 48, (1, 40), 40),      # MHA: 16 per group
    (16, 8, 128, 32, 96, (1, 200), 5),     # G 2
    # own blocks past one 64-entry table window (up to 138), some none
    (32, 8, 128, 16, 128, (0, 2200), 10),
]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("H,Hkv,D,bs,prefix,suffix,S", CASES)
def test_cascade_parity(H, Hkv, D, bs, prefix, suffix, S, fp8):
    base = "long_fp8" if fp8 else "shared_prefix_bf16"
    lo, hi = suffix
    b = workloads.make_batch(base, device=DEV, num_seqs=S, num_heads=H, num_kv_heads=Hkv,
                             head_dim=D, block_size=bs, lens=("prefix", prefix, max(lo, 1), hi),
                             max_len=prefix + hi, pool=("exact",), poison=True, seed=81)
    if lo == 0:                               # a few sequences end exactly at the prefix
        lens = b.seq_lens.clone()
        lens[::3] = prefix
        b.seq_lens.copy_(lens)
    N = prefix // bs
    ref, _, _ = oracle_step(b)        # appends the new rows, then attends over seq_lens
    kc, vc = gpu_caches(b)
    pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, b.k_scale, b.v_scale)
    plain = pa.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, k_scale=b.k_scale,
                      v_scale=b.v_scale)
    # balanced, one-block and 40-block chunks (the last cross table windows
    # and KV heads inside a chunk)
    for P in (0, bs, 40 * bs):
        print("CASE cascade", H, Hkv, D, bs, prefix, suffix, S, "fp8" if fp8 else "bf16", "P", P,
              flush=True)
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = torch.full_like(b.q, float("nan"))
        pa.decode_cascade(b.q, kc, vc, b.block_tables, b.seq_lens, N, b.scale, out=out,
                          k_scale=b.k_scale, v_scale=b.v_scale, partition_tokens=P,
                          err_flag=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        check_close(out, ref, b.cache_dtype, f"cascade P{P}")
        check_close(out, plain.double().cpu().numpy(), b.cache_dtype, f"cascade vs decode P{P}")


def test_cascade_full_size_every_row():
    """The shared-prefix batch at full size, in the benchmark's launch
    configuration: every output row against the oracle."""
    b = workloads.make_batch("shared_prefix_bf16", device=DEV)
    kc, vc = gpu_caches(b)
    pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc)
    print("CASE cascade full size", flush=True)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pa.decode_cascade(b.q, kc, vc, b.block_tables, b.seq_lens, b.shared_prefix_blocks,
                            b.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ref, _, _ = oracle_step(b)
    check_close(out, ref, "bf16", "full-size cascade")


def test_cascade_long_prefix_many_rows():
    """512 sequences x 64 heads (G 8): more (KV head, row block) pairs than
    compute units, and a 68-block prefix: the prefix pass cuts it into
    token ranges of at most 64 blocks.  Every row against the oracle and
    against plain decode."""
    b = workloads.make_batch("shared_prefix_bf16", device=DEV, num_seqs=512, num_heads=64,
                             num_kv_heads=8, lens=("prefix", 68 * 16, 1, 40),
                             max_len=68 * 16 + 48, seed=83)
    kc, vc = gpu_caches(b)
    pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc)
    print("CASE cascade long prefix, 512 x 64 rows", flush=True)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pa.decode_cascade(b.q, kc, vc, b.block_tables, b.seq_lens, 68, b.scale, err_flag=flag)
    plain = pa.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ref, _, _ = oracle_step(b)
    check_close(out, ref, "bf16", "long-prefix cascade")
    check_close(out, plain.double().cpu().numpy(), "bf16", "long-prefix cascade vs decode")


def test_broken_prefix_contract_is_flagged():
    b = workloads.make_batch("shared_prefix_bf16", device=DEV, num_seqs=6,
                             lens=("prefix", 64, 1, 30), max_len=96, seed=82)
    tables = b.block_tables.clone()
    tables[2, 1] = tables[2, 4] if tables[2, 4] >= 0 else tables[3, 4]   # not the shared block
    kc, vc = gpu_caches(b)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("CASE cascade broken contract", flush=True)
    pa.decode_cascade(b.q, kc, vc, tables, b.seq_lens, 4, b.scale, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & pa.DEVERR_PREFIX
