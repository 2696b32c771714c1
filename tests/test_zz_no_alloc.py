"""pa_decode_noalloc (pa_decode whose split-KV workspace is the library's
static device buffer) through the C ABI, against pa_decode with a caller
workspace on the same inputs: two calls in a row, the second on a smaller
batch, so it runs over the buffer the first one left behind.  The two entry
points share their kernels and plan, so the outputs must agree bit for bit;
each is also checked against the oracle.  A repeated call changes neither
the device's free memory nor torch's allocations."""
import pytest
import torch

import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (workload, overrides of the first call, overrides of the second, smaller call)
CASES = [
    ("llama3_8b_bf16", {}, dict(num_seqs=5, lens=("uniform", 1, 300), max_len=304, seed=92)),
    ("long_fp8", dict(num_seqs=3, lens=("uniform", 900, 4000), max_len=4000, seed=93),
     dict(num_seqs=2, lens=("uniform", 1, 700), max_len=704, seed=94)),
    ("qwen3_0p6b_bf16", dict(num_seqs=40, lens=("lognormal", 300, 1.0, 1, 1500), max_len=1504,
                             seed=95), dict(num_seqs=3, lens=("fixed", 33), max_len=48, seed=96)),
    ("tiny_f32", {}, dict(num_seqs=2, seed=97)),
]


def run_both(b, kc, vc, **kw):
    common = dict(k_scale=b.k_scale, v_scale=b.v_scale, **kw)
    ref = pa.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, **common)
    out = torch.full_like(b.q, float("nan"))
    pa.decode_noalloc(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, out, **common)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_decode_on_two_calls(name, first, second):
    for call, over in (("first", first), ("second, smaller", second)):
        b = workloads.make_batch(name, device=DEV, **over)
        kc, vc = gpu_caches(b)
        pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, b.k_scale, b.v_scale)
        ref_o, _, _ = oracle_step(b)
        for P in (b.partition_tokens or 0, b.block_size * 4):
            for bf16p in ((False, True) if b.q_dtype == "bf16" else (False,)):
                print("CASE noalloc", name, call, "P", P, "bf16 partials", bf16p, flush=True)
                ref, out = run_both(b, kc, vc, partition_tokens=P, bf16_partials=bf16p)
                assert torch.equal(out, ref), f"{name} {call} P{P}: differs from pa_decode"
                check_close(out, ref_o, b.cache_dtype, f"noalloc {name} {call} P{P}")


def test_noalloc_allocates_nothing():
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=16, lens=("uniform", 64, 900),
                             max_len=912, seed=98)
    kc, vc = gpu_caches(b)
    out = torch.empty_like(b.q)
    print("CASE noalloc allocation check", flush=True)
    pa.decode_noalloc(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, out)   # loads the buffer
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    used0 = torch.cuda.memory_allocated()
    for _ in range(3):
        pa.decode_noalloc(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale, out)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.cuda.memory_allocated() == used0
    ref = pa.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
