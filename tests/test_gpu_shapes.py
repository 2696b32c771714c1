"""GPU parity over the shapes and work splits the named workloads do not
reach: head_dim 64 on the matrix-core kernel, bs 32 with bf16 and bs 16 with
e4m3, group sizes 1, 2 and 8, chunk lengths of one block and of odd block
counts (every KV head split between many chunks), one chunk for the whole
batch, and empty sequences between non-empty ones."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import CACHE_TORCH, check_close, gpu_caches, gpu_step, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SHAPES = [
    # base workload, heads, kv heads, head_dim, block_size
    ("llama3_8b_bf16", 8, 8, 64, 16),      # MHA, D 64
    ("llama3_8b_bf16", 16, 2, 64, 32),     # G 8, D 64, bs 32
    ("llama3_8b_bf16", 4, 2, 128, 32),     # G 2, bs 32
    ("long_fp8", 8, 4, 128, 16),           # e4m3, bs 16, G 2
    ("long_fp8", 8, 8, 64, 32),            # e4m3, D 64, MHA
    ("long_fp8", 16, 2, 128, 32),          # e4m3, G 8
    ("tiny_f32", 8, 1, 128, 32),           # f32, MQA, D 128, bs 32
]


def variants_for(b):
    probe = torch.empty((1, b.block_size, b.num_kv_heads, b.head_dim),
                        dtype=CACHE_TORCH[b.cache_dtype], device=DEV)
    out = [pa.VARIANT_VALU]
    try:
        pa.decode_workspace_size(b.q, probe, b.block_tables, variant=pa.VARIANT_MFMA)
        out.append(pa.VARIANT_MFMA)
    except pa.PaError:
        pass
    return out


@pytest.mark.parametrize("base,H,Hkv,D,bs", SHAPES)
def test_shapes_and_chunkings(base, H, Hkv, D, bs):
    b = workloads.make_batch(base, device=DEV, num_seqs=5, num_heads=H, num_kv_heads=Hkv,
                             head_dim=D, block_size=bs, lens=("uniform", 1, 333), max_len=352,
                             poison=True, seed=17)
    ref, _, _ = oracle_step(b)
    total = b.num_seqs * b.num_kv_heads * b.max_blocks_per_seq * bs
    for variant in variants_for(b):
        for P in (0, bs, 3 * bs, total):   # auto, 1 block, 3 blocks, one chunk for everything
            print("CASE", base, H, Hkv, D, bs, "variant", variant, "P", P, flush=True)
            out = gpu_step(b, *gpu_caches(b), variant=variant, partition_tokens=P)
            torch.cuda.synchronize()
            check_close(out, ref, b.cache_dtype, f"{base} H{H}/{Hkv} D{D} bs{bs} v{variant} P{P}")


@pytest.mark.parametrize("lens", [[0, 5, 0, 0, 300, 0], [1], [0, 0, 0], [16, 0, 17, 0, 15]])
def test_empty_and_tiny_sequences(lens):
    S = len(lens)
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=S,
                             lens=("uniform", 1, 300), max_len=304, seed=23)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    bs = b.block_size
    tables = torch.full((S, b.max_blocks_per_seq), -1, dtype=torch.int32)
    perm = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(3))
    c = 0
    for s, L in enumerate(lens):
        nb = -(-L // bs)
        tables[s, :nb] = perm[c:c + nb]
        c += nb
    ref = oracle.decode(b.q.cpu(), b.key_pool.cpu(), b.value_pool.cpu(), tables, lens_t, b.scale)
    for variant in variants_for(b):
        for P in (0, bs, 2 * bs):
            print("CASE lens", lens, "variant", variant, "P", P, flush=True)
            out = torch.full_like(b.q, float("nan"))      # every row must be written
            pa.decode(b.q, b.key_pool, b.value_pool, tables.to(DEV), lens_t.to(DEV), b.scale,
                      out=out, variant=variant, partition_tokens=P)
            torch.cuda.synchronize()
            check_close(out, ref, "bf16", f"lens {lens} v{variant} P{P}")
            for s, L in enumerate(lens):
                if L == 0:
                    assert torch.equal(out[s].float(), torch.zeros_like(out[s].float()))


def test_repeated_calls_reuse_workspace():
    """The workspace carries no state between calls: the same workspace serves
    calls with different batches and chunkings, and results match fresh ones."""
    b1 = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=7, lens=("uniform", 1, 500),
                              max_len=512, seed=31)
    b2 = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=7, lens=("uniform", 1, 500),
                              max_len=512, seed=32)
    need = max(pa.decode_workspace_size(b1.q, b1.key_pool, b1.block_tables, P)
               for P in (0, 16, 48))
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    for b in (b1, b2, b1):
        for P in (48, 0, 16):
            print("CASE workspace reuse P", P, flush=True)
            fresh = pa.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale,
                              partition_tokens=P)
            reused = pa.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale,
                               partition_tokens=P, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(fresh, reused)


@pytest.mark.parametrize("variant", [pa.VARIANT_VALU, pa.VARIANT_MFMA])
def test_segments_split_into_many_parts(variant):
    """One-block chunks over sequences of up to 313 blocks: the merge combines
    more partials per row than it has threads (several passes over its
    weights), next to a short sequence that one chunk covers."""
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=3, num_heads=8,
                             num_kv_heads=2, lens=("fixed", 5000), max_len=5008,
                             poison=True, seed=41)
    lens = torch.tensor([5000, 7, 4113], dtype=torch.int32)    # shortened: tables stay valid
    b.seq_lens.copy_(lens.to(DEV))
    ref = oracle.decode(b.q.cpu(), b.key_pool.cpu(), b.value_pool.cpu(), b.block_tables.cpu(),
                        lens, b.scale)
    for P in (16, 32, 0):
        print("CASE many parts variant", variant, "P", P, flush=True)
        out = torch.full_like(b.q, float("nan"))
        pa.decode(b.q, b.key_pool, b.value_pool, b.block_tables, b.seq_lens, b.scale, out=out,
                  variant=variant, partition_tokens=P)
        torch.cuda.synchronize()
        check_close(out, ref, "bf16", f"many parts v{variant} P{P}")


@pytest.mark.parametrize("variant", [pa.VARIANT_VALU, pa.VARIANT_MFMA])
def test_small_batch_launches_one_wavefront_per_unit(variant):
    """A batch whose largest possible work list (S * Hkv * max_nb blocks) is
    shorter than the device's resident wavefronts gets one wavefront per
    block, not a full device of mostly idle ones: its workspace is that of
    one-block chunks, and the result still matches the oracle."""
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=3, num_heads=8,
                             num_kv_heads=2, head_dim=128, block_size=16,
                             lens=("uniform", 1, 90), max_len=96, seed=57)
    kc, vc = gpu_caches(b)
    units = b.num_seqs * b.num_kv_heads * b.block_tables.shape[1]
    G = b.num_heads // b.num_kv_heads
    slots = units + b.num_seqs * b.num_kv_heads
    acc = 4                                        # fp32 partial accumulators
    want = acc * slots * G * b.head_dim + 8 * slots * G + 8 * b.num_seqs * b.num_kv_heads
    assert pa.decode_workspace_size(b.q, kc, b.block_tables, variant=variant) == want
    print("CASE small batch", variant, flush=True)
    ref, _, _ = oracle_step(b)
    out = gpu_step(b, kc, vc, variant=variant)
    torch.cuda.synchronize()
    check_close(out, ref, b.cache_dtype, f"small batch variant {variant}")
