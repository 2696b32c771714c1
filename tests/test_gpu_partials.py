"""GPU parity of single-query decode with many partial results.  Each case
splits its batch into one-block partitions, so that a large partial volume
arises at a size the oracle finishes quickly: on the bf16 per-wavefront
kernel every partition of a segment leaves its own partial (more than 32 MB
of them, more than the device's L2s hold), and on the per-block e4m3 kernel
each workgroup walks a run of partitions and leaves one partial per segment
the run touches.  fp32 and bf16 partials; with at most 8 query heads per KV
head the lane pairs holding one column write whole lines (both kernels).
The same batch in larger partitions is checked beside them."""
import pytest
import torch

import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import check_close, gpu_caches, gpu_step, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def partial_bytes(b, kc, P, bf16p):
    """Bytes of the accumulator region of the workspace (its first part)."""
    total = pa.decode_workspace_size(b.q, kc, b.block_tables, P, bf16_partials=bf16p)
    G = b.num_heads // b.num_kv_heads
    segs = b.num_seqs * b.num_kv_heads
    # workspace = acc_bytes * slots * G * D + 8 * slots * G + 8 * segs
    per_slot = (2 if bf16p else 4) * G * b.head_dim + 8 * G
    slots = (total - 8 * segs) // per_slot
    return slots * G * b.head_dim * (2 if bf16p else 4)


CASES = [
    # base workload, overrides, partition tokens
    ("long_fp8", dict(num_seqs=4, lens=("uniform", 17000, 19000), max_len=19008), 32),
    ("llama3_8b_bf16", dict(num_seqs=20, lens=("uniform", 2000, 4000), max_len=4000), 16),
]


@pytest.mark.parametrize("base,over,P", CASES, ids=["e4m3-heads", "bf16-wave"])
def test_many_partials(base, over, P):
    b = workloads.make_batch(base, device=DEV, poison=True, seed=77, **over)
    kc, vc = gpu_caches(b)
    ref, _, _ = oracle_step(b)
    if base == "llama3_8b_bf16":
        assert partial_bytes(b, kc, P, False) > 32 << 20       # more than the L2s hold
    for bf16p in (False, True):
        print("CASE many partials", base, "P", P, "bf16 partials", bf16p, flush=True)
        kc, vc = gpu_caches(b)
        out = gpu_step(b, kc, vc, partition_tokens=P, bf16_partials=bf16p)
        torch.cuda.synchronize()
        check_close(out, ref, b.cache_dtype, f"partials {base} P{P} bf{bf16p}")
    P2 = 64 * P
    print("CASE larger partitions", base, "P", P2, flush=True)
    kc, vc = gpu_caches(b)
    out = gpu_step(b, kc, vc, partition_tokens=P2)
    torch.cuda.synchronize()
    check_close(out, ref, b.cache_dtype, f"partials {base} P{P2}")

