"""The hot path under HIP graph capture: pa_kv_append + pa_decode (and the
multi-token, block-clearing and cascade calls) queue work on the caller's
stream, allocate nothing and never synchronise, so a step can be captured once
and replayed.  Each replay runs after the program's own eager work (new query
rows written in place, a synchronisation) and must equal the eager result
for the same inputs."""
import pytest
import torch

import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import gpu_caches

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_decode_step_replays_match_eager():
    b = workloads.make_batch("llama3_8b_bf16", device=DEV, num_seqs=16,
                             lens=("uniform", 1, 700), max_len=704, seed=91)
    kc, vc = gpu_caches(b)
    out = torch.empty_like(b.q)
    ws = torch.empty(pa.decode_workspace_size(b.q, kc, b.block_tables), dtype=torch.uint8,
                     device=DEV)
    q = b.q.clone()
    # warm the library's per-device caches (compute-unit count, occupancy) outside capture
    pa.decode(q, kc, vc, b.block_tables, b.seq_lens, b.scale, out=out, workspace=ws)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, stream=s)
            pa.decode(q, kc, vc, b.block_tables, b.seq_lens, b.scale, out=out, workspace=ws,
                      stream=s)
    torch.cuda.synchronize()

    gen = torch.Generator(device=DEV).manual_seed(5)
    for rep in range(4):
        print("CASE graph replay", rep, flush=True)
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))   # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = pa.decode(q, kc, vc, b.block_tables, b.seq_lens, b.scale)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


def test_verify_step_and_block_clear_replay():
    b = workloads.make_batch("llama3_8b_bf16_spec8", device=DEV, num_seqs=8,
                             lens=("uniform", 1, 300), max_len=304, seed=92)
    kc, vc = gpu_caches(b)
    out = torch.empty_like(b.q)
    ws = torch.empty(pa.decode_multi_workspace_size(b.q, b.max_query_len, kc, b.block_tables),
                     dtype=torch.uint8, device=DEV)
    scratch = [torch.randint(1, 256, (32, 4096), dtype=torch.uint8, device=DEV) for _ in range(3)]
    regs = pa.region_table(scratch)
    ids = torch.tensor([3, 9, 30], dtype=torch.int32, device=DEV)
    pa.decode_multi(b.q, b.query_start_loc, b.max_query_len, kc, vc, b.block_tables,
                    b.seq_lens, b.scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, stream=s)
            pa.decode_multi(b.q, b.query_start_loc, b.max_query_len, kc, vc, b.block_tables,
                            b.seq_lens, b.scale, out=out, workspace=ws, stream=s)
            pa.zero_blocks(ids, regs, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        print("CASE graph replay multi", rep, flush=True)
        for t in scratch:
            t.fill_(7)                                   # eager work the replay must undo
        b.q.mul_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = pa.decode_multi(b.q, b.query_start_loc, b.max_query_len, kc, vc, b.block_tables,
                                b.seq_lens, b.scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        for t in scratch:
            assert not t[ids.long()].any() and (t[[0, 1, 2]] == 7).all()


def test_cascade_step_replays_match_eager():
    """Append plus the cascade's kernels (prefix pass, suffix pass, merge)
    captured as one step."""
    b = workloads.make_batch("shared_prefix_bf16", device=DEV, num_seqs=24,
                             lens=("prefix", 320, 1, 90), max_len=320 + 96, seed=93)
    kc, vc = gpu_caches(b)
    N = b.shared_prefix_blocks
    out = torch.empty_like(b.q)
    ws = torch.empty(pa.decode_cascade_workspace_size(b.q, kc, b.block_tables, N),
                     dtype=torch.uint8, device=DEV)
    q = b.q.clone()
    pa.decode_cascade(q, kc, vc, b.block_tables, b.seq_lens, N, b.scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, stream=s)
            pa.decode_cascade(q, kc, vc, b.block_tables, b.seq_lens, N, b.scale, out=out,
                              workspace=ws, stream=s)
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV).manual_seed(6)
    for rep in range(4):
        print("CASE graph replay cascade", rep, flush=True)
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = pa.decode_cascade(q, kc, vc, b.block_tables, b.seq_lens, N, b.scale)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
