"""The comparison the GPU parity tests use, checked on the CPU: the oracle's
own result rounded to the output dtype passes it, and the one-block negative
control at the full Llama-3-8B and Qwen3-0.6B batch shapes makes it fail.
No GPU: the stand-in for the GPU output is the oracle's answer itself."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from pa_cases import check_close, negative_control, oracle_step


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "qwen3_0p6b_bf16"])
def test_negative_control_is_caught_at_full_size(name):
    b = workloads.make_batch(name, device="cpu")
    ref, hk, hv = oracle_step(b)
    out = torch.from_numpy(ref).to(torch.bfloat16)          # a correct result, rounded
    check_close(out, ref, b.cache_dtype, "rounded oracle")
    s, j = negative_control(b, out, hk, hv)
    assert j >= 1 and 0 <= s < b.num_seqs


def test_negative_control_reports_a_miss():
    """When the block the control points at holds the same values as the one
    it replaces, the wrong table cannot be told apart: the helper must then
    fail rather than pass silently."""
    b = workloads.make_batch("llama3_8b_bf16", device="cpu", num_seqs=2, lens=("fixed", 64),
                             max_len=64)
    _, hk, hv = oracle_step(b)
    lens = b.seq_lens.numpy()
    tbl = b.block_tables.numpy()
    s = int(np.argmin(lens))
    j = -(-int(lens[s]) // b.block_size) // 2
    hk[tbl[s, j]] = hk[tbl[s, j - 1]]                    # make the two blocks equal
    hv[tbl[s, j]] = hv[tbl[s, j - 1]]
    out = torch.from_numpy(oracle.decode(b.q, hk, hv, tbl, lens, b.scale)).to(torch.bfloat16)
    with pytest.raises(AssertionError, match="went undetected"):
        negative_control(b, out, hk, hv)
