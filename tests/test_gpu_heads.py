"""GPU parity of single-query decode of an e4m3 cache with 4 or 8 KV heads
at head_dim 128: the kernel whose workgroups hold one wavefront per KV head
and read each block's K and V rows of every head together.

Its own work split and bookkeeping are what these cases aim at: chunks of
(sequence, block) units that start and end mid-sequence, a segment's
partial slots stepping by the number of KV heads, one workgroup per block
for a small batch, empty sequences between others, group sizes 1-8, block
sizes 16 and 32, fp32 and bf16 partials, and an out-of-range block id or
an over-long length (flagged, not followed).  Every case prints its
parameters before it touches the GPU."""
import pytest
import torch

import oracle
import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, gpu_step, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SHAPES = [
    # kv heads, group, block size
    (8, 8, 32),
    (8, 1, 32),
    (8, 2, 16),
    (8, 4, 16),
    (4, 8, 16),
    (4, 4, 32),
    (4, 1, 16),
    (4, 2, 32),
]


@pytest.mark.parametrize("Hkv,G,bs", SHAPES)
def test_heads_shapes_and_chunkings(Hkv, G, bs):
    b = workloads.make_batch("long_fp8", device=DEV, num_seqs=7, num_heads=Hkv * G,
                             num_kv_heads=Hkv, block_size=bs, lens=("uniform", 1, 420),
                             max_len=448, poison=True, seed=100 + Hkv * 10 + G + bs)
    ref, _, _ = oracle_step(b)
    cap = b.max_blocks_per_seq * bs
    for P in (0, bs, 3 * bs, 5 * bs, cap, b.num_seqs * cap):
        for bf16p in (False, True):
            print("CASE heads Hkv", Hkv, "G", G, "bs", bs, "P", P, "bf16 partials", bf16p,
                  flush=True)
            out = gpu_step(b, *gpu_caches(b), partition_tokens=P, bf16_partials=bf16p)
            torch.cuda.synchronize()
            check_close(out, ref, b.cache_dtype, f"heads Hkv{Hkv} G{G} bs{bs} P{P} bf{bf16p}")


def test_heads_empty_sequences_between_others():
    lens = [0, 37, 0, 1, 500, 0, 32, 33]
    S = len(lens)
    b = workloads.make_batch("long_fp8", device=DEV, num_seqs=S, num_heads=32, num_kv_heads=8,
                             lens=("uniform", 1, 512), max_len=512, poison=False, seed=7)
    tables = torch.full_like(b.block_tables, -1).cpu()
    need = [(L + b.block_size - 1) // b.block_size for L in lens]
    perm = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(3))
    assert sum(need) <= b.num_blocks
    c = 0
    for s in range(S):
        tables[s, :need[s]] = perm[c:c + need[s]]
        c += need[s]
    kc, vc = gpu_caches(b)
    hk, hv = kc.cpu(), vc.cpu()
    lens_t = torch.tensor(lens, dtype=torch.int32)
    ref = oracle.decode(b.q.cpu(), hk, hv, tables, lens_t, b.scale, b.k_scale, b.v_scale)
    for P in (0, 32, 64 * 32):
        print("CASE heads empty sequences P", P, flush=True)
        out = pa.decode(b.q, kc, vc, tables.to(DEV), lens_t.to(DEV), b.scale,
                        k_scale=b.k_scale, v_scale=b.v_scale, partition_tokens=P)
        torch.cuda.synchronize()
        for s, L in enumerate(lens):
            if L == 0:
                assert torch.equal(out[s].float(), torch.zeros_like(out[s].float()))
        check_close(out, ref, b.cache_dtype, f"heads empty sequences P{P}")


def test_heads_small_batch_one_workgroup_per_block():
    """A batch with fewer (sequence, block) units than the device's resident
    workgroups launches one workgroup per unit: the workspace is that of
    one-block chunks of every KV head, and the result matches the oracle."""
    b = workloads.make_batch("long_fp8", device=DEV, num_seqs=3, num_heads=16, num_kv_heads=8,
                             lens=("uniform", 1, 90), max_len=96, poison=True, seed=58)
    kc, vc = gpu_caches(b)
    G = b.num_heads // b.num_kv_heads
    blocks = b.num_seqs * b.block_tables.shape[1]
    slots = blocks * b.num_kv_heads + b.num_seqs * b.num_kv_heads
    want = 4 * slots * G * b.head_dim + 8 * slots * G + 8 * b.num_seqs * b.num_kv_heads
    assert pa.decode_workspace_size(b.q, kc, b.block_tables) == want
    print("CASE heads small batch", flush=True)
    ref, _, _ = oracle_step(b)
    out = gpu_step(b, kc, vc)
    torch.cuda.synchronize()
    check_close(out, ref, b.cache_dtype, "heads small batch")


def test_heads_broken_device_data_is_flagged_not_followed():
    b = workloads.make_batch("long_fp8", device=DEV, num_seqs=3, num_heads=32, num_kv_heads=8,
                             lens=("fixed", 256), max_len=256, seed=9)
    kc, vc = gpu_caches(b)
    tbl = b.block_tables.clone()
    tbl[1, 2] = b.num_blocks + 1000               # block 2 of sequence 1 is out of range
    lens = torch.tensor([200, 200, 10_000], dtype=torch.int32, device=DEV)
    ref = oracle.decode(b.q.cpu(), kc.cpu(), vc.cpu(), b.block_tables.cpu(),
                        torch.tensor([200, 200, 256], dtype=torch.int32), b.scale,
                        b.k_scale, b.v_scale)
    for P in (0, 64):
        print("CASE heads broken device data P", P, flush=True)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = pa.decode(b.q, kc, vc, tbl, lens, b.scale, k_scale=b.k_scale, v_scale=b.v_scale,
                        partition_tokens=P, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == pa.DEVERR_BLOCK_ID | pa.DEVERR_SEQ_LEN
        assert torch.isfinite(out.float()).all()
        check_close(out[[0, 2]], ref[[0, 2]], b.cache_dtype, f"heads clamped rows P{P}")


@pytest.mark.parametrize("bs", [32, 16])
def test_heads_runs_of_partitions(bs):
    """Fixed partitions outnumbering the workgroups the device holds at once:
    each workgroup walks a run of several and carries its softmax state
    across their boundaries, leaving one partial per segment it touches
    (one-block partitions: runs ending inside a block's worth of a
    sequence's start or end)."""
    b = workloads.make_batch("long_fp8", device=DEV, num_seqs=6, num_heads=64, num_kv_heads=8,
                             block_size=bs, lens=("uniform", 1500, 2600), max_len=2624,
                             poison=True, seed=61 + bs)
    ref, _, _ = oracle_step(b)
    for P in (bs, 2 * bs, 3 * bs, 512):
        print("CASE heads partition runs bs", bs, "P", P, flush=True)
        out = gpu_step(b, *gpu_caches(b), partition_tokens=P)
        torch.cuda.synchronize()
        check_close(out, ref, b.cache_dtype, f"heads runs bs{bs} P{P}")
