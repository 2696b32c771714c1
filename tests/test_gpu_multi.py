"""GPU parity of pa_decode_multi (several new query tokens per sequence,
causal within them) against the oracle: every new token's K/V row is
appended by pa_kv_append, then the whole step is compared with the oracle's
append + multi-token decode.  Cases cover one, two and four 16-column tiles
of (query token, head) pairs, bf16 and e4m3 caches, head_dim 64 and 128,
block sizes 16 and 32, query counts that differ between sequences (zero
included), sequences made only of new tokens, one-block chunks (many
partials per row), the full-size verify workload on every row, and a
16,384-row batch at head_dim 64 on every row."""
import pytest
import torch

import oracle
import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, gpu_step_multi, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # base, heads, kv heads, head_dim, block_size, query lengths
    ("llama3_8b_bf16_spec8", 32, 8, 128, 16, ("fixed", 8)),        # G 4 x 8: 2 column tiles
    ("llama3_8b_bf16_spec8", 16, 4, 64, 16, ("fixed", 6)),         # G 4 x 6: 2 tiles, D 64
    ("llama3_8b_bf16_spec8", 32, 8, 128, 32, ("uniform", 5, 7)),   # G 4 x 7: 2 tiles, bs 32
    ("llama3_8b_bf16_spec8", 32, 8, 128, 16, ("uniform", 0, 4)),   # 1 tile, some sequences none
    ("llama3_8b_bf16_spec8", 16, 2, 64, 32, ("fixed", 8)),         # G 8 x 8: 4 tiles, D 64
    ("llama3_8b_bf16_spec8", 4, 4, 128, 32, ("uniform", 1, 16)),   # MHA x 16
    ("llama3_8b_bf16_spec8", 8, 4, 128, 16, ("fixed", 3)),         # G 2 x 3: 6 of 16 columns
    ("long_fp8", 16, 4, 128, 32, ("fixed", 5)),                    # e4m3, G 4 x 5: 2 tiles
    ("long_fp8", 8, 8, 64, 16, ("uniform", 1, 12)),                # e4m3, MHA, bs 16
]


@pytest.mark.parametrize("base,H,Hkv,D,bs,qlens", CASES)
def test_multi_token_parity(base, H, Hkv, D, bs, qlens):
    b = workloads.make_batch(base, device=DEV, num_seqs=6, num_heads=H, num_kv_heads=Hkv,
                             head_dim=D, block_size=bs, lens=("uniform", 1, 300), max_len=304,
                             query_lens=qlens, poison=True, seed=51)
    ref, _, _ = oracle_step(b)
    for P in (0, bs, 3 * bs):
        print("CASE", base, H, Hkv, D, bs, qlens, "P", P, flush=True)
        out = torch.full_like(b.q, float("nan"))
        kc, vc = gpu_caches(b)
        gpu_step_multi(b, kc, vc, partition_tokens=P, out=out)
        torch.cuda.synchronize()
        check_close(out, ref, b.cache_dtype, f"{base} H{H}/{Hkv} D{D} bs{bs} {qlens} P{P}")


def test_all_new_tokens_and_single_token_agreement():
    """A sequence made only of new tokens (q_len = L), and q_len = 1 for every
    sequence, which must match pa_decode."""
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=4,
                             lens=("uniform", 1, 12), max_len=16, query_lens=("fixed", 16),
                             seed=52)
    ref, _, _ = oracle_step(b)
    print("CASE all-new", flush=True)
    kc, vc = gpu_caches(b)
    out = gpu_step_multi(b, kc, vc)
    torch.cuda.synchronize()
    check_close(out, ref, "bf16", "q_len = L")

    one = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=5,
                               lens=("uniform", 1, 200), max_len=208, query_lens=("fixed", 1),
                               seed=53)
    print("CASE q_len 1", flush=True)
    kc, vc = gpu_caches(one)
    pa.kv_append(one.k_new, one.v_new, one.slot_mapping, kc, vc)
    multi = pa.decode_multi(one.q, one.query_start_loc, 1, kc, vc, one.block_tables,
                            one.seq_lens, one.scale)
    single = pa.decode(one.q, kc, vc, one.block_tables, one.seq_lens, one.scale)
    torch.cuda.synchronize()
    ref1, _, _ = oracle_step(one)
    check_close(multi, ref1, "bf16", "multi q_len 1")
    check_close(single, ref1, "bf16", "single")


def test_query_layout_violations_are_flagged_and_contained():
    """Sequences claiming more query tokens than max_query_len: each count is
    clamped to the first max_query_len tokens (taken as the sequence's last
    positions), the flag is raised, and nothing else is written."""
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=3,
                             lens=("uniform", 20, 60), max_len=64, query_lens=("fixed", 4),
                             seed=54)
    _, hk, hv = oracle_step(b)
    kc, vc = gpu_caches(b)
    pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full_like(b.q, float("nan"))
    print("CASE max_query_len 3 < 4", flush=True)
    pa.decode_multi(b.q, b.query_start_loc, 3, kc, vc, b.block_tables, b.seq_lens, b.scale,
                    out=out, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) & pa.DEVERR_QUERY
    kept = [4 * s + i for s in range(3) for i in range(3)]
    clamped = oracle.decode_multi(b.q.cpu()[kept], torch.tensor([0, 3, 6, 9], dtype=torch.int32),
                                  hk, hv, b.block_tables.cpu(), b.seq_lens.cpu(), b.scale)
    check_close(out[kept], clamped, "bf16", "clamped rows")
    assert torch.isnan(out[[3, 7, 11]].float()).all(), "rows beyond the clamp were written"


def test_full_size_verify_workload_every_row():
    """The benchmarked verify batch (64 sequences x 8 new tokens, Llama-3-8B
    shape): every output row against the oracle."""
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV)
    kc, vc = gpu_caches(b)
    print("CASE full-size spec8", flush=True)
    out = gpu_step_multi(b, kc, vc)
    torch.cuda.synchronize()
    ref, _, _ = oracle_step(b)
    check_close(out, ref, "bf16", "full-size verify")


def test_many_rows_head_dim_64_every_row():
    """16,384 output rows at head_dim 64 (128 sequences x 8 new tokens x 16
    heads, G 8: four column tiles per KV head): the merge then packs two rows
    into each wavefront, each over 16-lane partial groups; every row against
    the oracle."""
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=128, num_heads=16,
                             num_kv_heads=2, head_dim=64, block_size=16,
                             lens=("uniform", 300, 1200), max_len=1200, seed=41)
    kc, vc = gpu_caches(b)
    print("CASE many-row spec8 D64", flush=True)
    out = gpu_step_multi(b, kc, vc)
    torch.cuda.synchronize()
    assert b.q.shape[0] * b.num_heads >= 8192
    ref, _, _ = oracle_step(b)
    check_close(out, ref, "bf16", "many-row D64 verify")


def test_multi_step_without_new_tokens():
    """A step in which no sequence has a new token: the empty rows, slots and
    query tensors (whatever strides the framework gives them) are accepted,
    nothing is written and the call returns."""
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=1, num_heads=32,
                             num_kv_heads=4, head_dim=64, lens=("uniform", 1, 630), max_len=630,
                             query_lens=("fixed", 0), poison=True, seed=1461281404)
    assert b.q.shape[0] == 0 and b.slot_mapping.shape[0] == 0
    ref, _, _ = oracle_step(b)
    print("CASE multi without new tokens", flush=True)
    kc, vc = gpu_caches(b)
    out = gpu_step_multi(b, kc, vc, partition_tokens=64)
    torch.cuda.synchronize()
    assert out.shape == (0, 32, 64)
    check_close(out, ref, b.cache_dtype, "multi without new tokens")
