"""GPU tests of pa_decode_append: the new token's append done inside the
decode kernel (one new bf16 row per sequence on the matrix-core kernels,
batches with at most two (sequence, KV head) pairs per wavefront -- every
batch here), else launched before it.  Its results must be bit for bit those of
pa_kv_append followed by pa_decode -- the output and the whole of both
caches -- on every kernel family (per-wavefront bf16 and e4m3, per-block
e4m3, vector-ALU fallback, f32), with balanced and fixed chunks, and within
the decode tolerance of the oracle; and its contract cases behave as
documented: a slot < 0 appends nothing, a slot outside the pool or away
from position seq_len - 1 raises PA_DEVERR_SLOT, a row for an empty
sequence is flagged and not written.  Every case prints its parameters
before it touches the GPU."""
import pytest
import torch

import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # name, base workload, overrides, variant
    ("llama-bf16", "llama3_8b_bf16", dict(num_seqs=6, lens=("uniform", 1, 700), max_len=704),
     pa.VARIANT_AUTO),
    ("qwen-bf16-G2", "qwen3_0p6b_bf16", dict(num_seqs=9, lens=("lognormal", 120, 1.0, 1, 600),
                                             max_len=608), pa.VARIANT_AUTO),
    ("bf16-bs32-D64-G8", "llama3_8b_bf16", dict(num_seqs=5, num_heads=16, num_kv_heads=2,
                                                head_dim=64, block_size=32,
                                                lens=("uniform", 1, 333), max_len=352),
     pa.VARIANT_AUTO),
    ("e4m3-heads", "long_fp8", dict(num_seqs=3, lens=("uniform", 900, 2500), max_len=2560),
     pa.VARIANT_AUTO),
    ("e4m3-heads-bs16-Hkv4", "long_fp8", dict(num_seqs=7, num_heads=8, num_kv_heads=4,
                                              block_size=16, lens=("uniform", 1, 420),
                                              max_len=448), pa.VARIANT_AUTO),
    ("e4m3-wave-Hkv2", "long_fp8", dict(num_seqs=5, num_heads=16, num_kv_heads=2,
                                        lens=("uniform", 1, 333), max_len=352), pa.VARIANT_AUTO),
    # 1,280 (sequence, KV head) pairs: more than one per wavefront
    ("bf16-many-segments", "llama3_8b_bf16", dict(num_seqs=160, lens=("uniform", 1, 64),
                                                   max_len=64), pa.VARIANT_AUTO),
    ("bf16-valu", "llama3_8b_bf16", dict(num_seqs=6, lens=("uniform", 1, 700), max_len=704),
     pa.VARIANT_VALU),
    ("f32", "tiny_f32", {}, pa.VARIANT_AUTO),
]


def separate(b, kc, vc, slots, **kw):
    """pa_kv_append then pa_decode on copies of the caches."""
    kc, vc = kc.clone(), vc.clone()
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.kv_append(b.k_new, b.v_new, slots, kc, vc, b.k_scale, b.v_scale, err_flag=flag)
    out = pa.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, k_scale=b.k_scale,
                    v_scale=b.v_scale, err_flag=flag, **kw)
    torch.cuda.synchronize()
    return out, kc, vc, int(flag.item())


def fused(b, kc, vc, slots, **kw):
    kc, vc = kc.clone(), vc.clone()
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pa.decode_append(b.k_new, b.v_new, slots, b.q, kc, vc, b.block_tables, b.seq_lens,
                           b.scale, k_scale=b.k_scale, v_scale=b.v_scale, err_flag=flag, **kw)
    torch.cuda.synchronize()
    return out, kc, vc, int(flag.item())


def same_bits(x, y):
    v = torch.int16 if x.element_size() == 2 else (torch.int32 if x.element_size() == 4
                                                      else torch.uint8)
    return torch.equal(x.view(v), y.view(v))


@pytest.mark.parametrize("name,base,over,variant", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_append_then_decode(name, base, over, variant):
    b = workloads.make_batch(base, device=DEV, poison=True, seed=91, **over)
    assert b.k_new.shape[0] == b.num_seqs
    kc, vc = gpu_caches(b)
    ref, _, _ = oracle_step(b)
    for P in (0, 4 * b.block_size):
        print("CASE decode_append", name, "variant", variant, "P", P, flush=True)
        o1, k1, v1, f1 = separate(b, kc, vc, b.slot_mapping, partition_tokens=P, variant=variant)
        o2, k2, v2, f2 = fused(b, kc, vc, b.slot_mapping, partition_tokens=P, variant=variant)
        assert f1 == f2 == 0
        assert same_bits(o1, o2), f"{name} P{P}: output differs from append + decode"
        assert same_bits(k1, k2) and same_bits(v1, v2), f"{name} P{P}: caches differ"
        check_close(o2, ref, b.cache_dtype, f"decode_append {name} P{P}")


@pytest.mark.parametrize("base", ["llama3_8b_bf16", "long_fp8"])
def test_fused_contract_cases(base):
    """Padding (slot -1), a slot in a block no table names (away from
    position L - 1), and a slot past the pool, in one batch: the first
    appends nothing, the other two raise PA_DEVERR_SLOT; the second is
    written where it points, the third nowhere.  None of the three is read
    by any sequence, so output and caches equal append + decode bit for
    bit."""
    over = dict(num_seqs=6, lens=("uniform", 40, 300), max_len=320)
    if base == "long_fp8":
        over["lens"] = ("uniform", 40, 300)
    b = workloads.make_batch(base, device=DEV, pool=("factor", 1.5), seed=93, **over)
    kc, vc = gpu_caches(b)
    used = set(b.block_tables[b.block_tables >= 0].cpu().tolist())
    free = next(i for i in range(b.num_blocks) if i not in used)
    slots = b.slot_mapping.clone()
    slots[1] = -1                                   # padding: nothing appended
    slots[2] = free * b.block_size + 3              # a slot no sequence reads
    slots[4] = b.num_blocks * b.block_size + 5      # past the pool
    for P in (0, 2 * b.block_size):
        print("CASE decode_append contract", base, "P", P, flush=True)
        o1, k1, v1, f1 = separate(b, kc, vc, slots, partition_tokens=P)
        o2, k2, v2, f2 = fused(b, kc, vc, slots, partition_tokens=P)
        assert f1 == pa.DEVERR_SLOT                  # the slot past the pool
        assert f2 == pa.DEVERR_SLOT
        assert same_bits(o1, o2)
        assert same_bits(k1, k2) and same_bits(v1, v2)


def test_fused_row_for_an_empty_sequence_is_flagged():
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=4, lens=("uniform", 20, 200),
                             max_len=208, seed=95)
    kc, vc = gpu_caches(b)
    lens = b.seq_lens.clone()
    lens[2] = 0
    slots = b.slot_mapping.clone()
    slots[2] = -1
    print("CASE decode_append empty sequence", flush=True)
    b.seq_lens = lens
    o1, k1, v1, f1 = separate(b, kc, vc, slots)
    o2, k2, v2, f2 = fused(b, kc, vc, slots)
    assert f1 == f2 == 0 and same_bits(o1, o2) and same_bits(k1, k2) and same_bits(v1, v2)
    assert torch.equal(o2[2].float(), torch.zeros_like(o2[2].float()))
    slots[2] = b.slot_mapping[2]                    # a row for the empty sequence
    o3, k3, v3, f3 = fused(b, kc, vc, slots)
    assert f3 == pa.DEVERR_SLOT
    assert same_bits(o3, o2) and same_bits(k3, k2) and same_bits(v3, v2)   # row not written


def test_more_rows_than_sequences_runs_the_append_first():
    """T != S: the append runs as its own launch, so anything goes that
    append + decode allows (here every sequence's row plus padding rows)."""
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=5, lens=("uniform", 20, 300),
                             max_len=304, seed=97)
    kc, vc = gpu_caches(b)
    k = torch.cat([b.k_new, b.k_new[:2]])
    v = torch.cat([b.v_new, b.v_new[:2]])
    slots = torch.cat([b.slot_mapping, torch.full((2,), -1, dtype=torch.int64, device=DEV)])
    print("CASE decode_append T != S", flush=True)
    kc1, vc1 = kc.clone(), vc.clone()
    pa.kv_append(k, v, slots, kc1, vc1)
    o1 = pa.decode(b.q, kc1, vc1, b.block_tables, b.seq_lens, b.scale)
    kc2, vc2 = kc.clone(), vc.clone()
    o2 = pa.decode_append(k, v, slots, b.q, kc2, vc2, b.block_tables, b.seq_lens, b.scale)
    torch.cuda.synchronize()
    assert same_bits(o1, o2) and same_bits(kc1, kc2) and same_bits(vc1, vc2)


@pytest.mark.parametrize("base", ["llama3_8b_bf16", "long_fp8"])
def test_fused_with_an_out_of_range_last_block(base):
    """The last block of one sequence names a block outside the pool: the
    decode skips it (PA_DEVERR_BLOCK_ID) and the new row is still written to
    its slot, as append + decode do; the fused form also reports that the
    row's position had no slot (PA_DEVERR_SLOT)."""
    b = workloads.make_batch(base, device=DEV, num_seqs=4, lens=("uniform", 40, 300),
                             max_len=320, seed=99)
    kc, vc = gpu_caches(b)
    L = int(b.seq_lens[1].item())
    tbl = b.block_tables.clone()
    tbl[1, (L - 1) // b.block_size] = b.num_blocks + 7
    b.block_tables = tbl
    for P in (0, 2 * b.block_size):
        print("CASE decode_append bad last block", base, "P", P, flush=True)
        o1, k1, v1, f1 = separate(b, kc, vc, b.slot_mapping, partition_tokens=P)
        o2, k2, v2, f2 = fused(b, kc, vc, b.slot_mapping, partition_tokens=P)
        assert f1 == pa.DEVERR_BLOCK_ID
        assert f2 == pa.DEVERR_BLOCK_ID | pa.DEVERR_SLOT
        assert same_bits(o1, o2)
        assert same_bits(k1, k2) and same_bits(v1, v2)
