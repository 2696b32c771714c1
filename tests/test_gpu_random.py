"""GPU parity on seeded random configurations against the oracle: shapes,
dtypes, length mixes, work splits and kernel families drawn together, so
combinations the hand-picked cases do not name are exercised too.  Every
case is drawn from one fixed seed (the list is the same on every run) and
prints its parameters before it touches the GPU.

decode:  1-40 sequences, 1-8 KV heads, groups 1-8, head_dim 64 or 128,
         block size 16 or 32, f32 / bf16 / e4m3 caches, lengths up to 700
         tokens, balanced or fixed chunks of 1, 4 or 32 blocks, both kernel
         families where the dtypes allow the matrix cores, NaN in every slot
         no sequence may read.
multi:   the same, bf16 query, 0-8 new tokens per sequence.
cascade: 4-40 sequences sharing a prefix of 1-12 blocks plus 1-200 own
         tokens each.
append:  1-69 sequences of up to 4000 tokens, fixed runs of 1-64-block
         partitions or balanced chunks: pa_decode_append bitwise against
         pa_kv_append + pa_decode, and pa_decode_noalloc; 6 of them with
         257-1200 sequences."""
import numpy as np
import pytest
import torch

import paged_kv_cache_54_amd as pa
import workloads
from pa_cases import CACHE_TORCH, check_close, gpu_caches, gpu_step, gpu_step_multi, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

_BASE = {"f32": "tiny_f32", "bf16": "llama3_8b_bf16", "fp8": "long_fp8"}


def _draw(rng, kinds):
    kind = kinds[int(rng.integers(0, len(kinds)))]
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    return dict(kind=kind, S=int(rng.integers(1, 41)), Hkv=Hkv, H=Hkv * G,
                D=int(rng.choice([64, 128])), bs=int(rng.choice([16, 32])),
                max_len=int(rng.integers(1, 701)), chunk=int(rng.choice([0, 0, 1, 4, 32])),
                seed=int(rng.integers(0, 2**31)))


_RNG = np.random.default_rng(20261202)
DECODE = [_draw(_RNG, ["f32", "bf16", "fp8"]) for _ in range(24)]
MULTI = [_draw(_RNG, ["bf16", "fp8"]) for _ in range(12)]
CASCADE = [_draw(_RNG, ["bf16", "fp8"]) for _ in range(12)]


def _ids(cases):
    return [f"{c['kind']}-S{c['S']}-H{c['H']}x{c['Hkv']}-D{c['D']}-bs{c['bs']}-L{c['max_len']}"
            f"-c{c['chunk']}" for c in cases]


def _batch(c, **extra):
    return workloads.make_batch(_BASE[c["kind"]], device=DEV, num_seqs=c["S"],
                                num_heads=c["H"], num_kv_heads=c["Hkv"], head_dim=c["D"],
                                block_size=c["bs"], pool=("factor", 1.2), poison=True,
                                seed=c["seed"], **extra)


def _variants(b):
    probe = torch.empty((1, b.block_size, b.num_kv_heads, b.head_dim),
                        dtype=CACHE_TORCH[b.cache_dtype], device=DEV)
    out = [pa.VARIANT_VALU]
    try:
        pa.decode_workspace_size(b.q, probe, b.block_tables, variant=pa.VARIANT_MFMA)
        out.append(pa.VARIANT_MFMA)
    except pa.PaError:
        pass
    return out


@pytest.mark.parametrize("c", DECODE, ids=_ids(DECODE))
def test_random_decode(c):
    b = _batch(c, lens=("uniform", 1, c["max_len"]), max_len=c["max_len"])
    ref, _, _ = oracle_step(b)
    for variant in _variants(b):
        print("CASE random decode", c, "variant", variant, flush=True)
        kc, vc = gpu_caches(b)
        out = gpu_step(b, kc, vc, variant=variant, partition_tokens=c["chunk"] * c["bs"])
        torch.cuda.synchronize()
        check_close(out, ref, b.cache_dtype, f"random decode {c} variant {variant}")


@pytest.mark.parametrize("c", MULTI, ids=_ids(MULTI))
def test_random_multi(c):
    b = _batch(c, lens=("uniform", 1, c["max_len"]), max_len=c["max_len"],
               query_lens=("uniform", 0, 8))
    ref, _, _ = oracle_step(b)
    print("CASE random multi", c, flush=True)
    kc, vc = gpu_caches(b)
    out = gpu_step_multi(b, kc, vc, partition_tokens=c["chunk"] * c["bs"])
    torch.cuda.synchronize()
    check_close(out, ref, b.cache_dtype, f"random multi {c}")


@pytest.mark.parametrize("c", CASCADE, ids=_ids(CASCADE))
def test_random_cascade(c):
    rng = np.random.default_rng(c["seed"])
    N = int(rng.integers(1, 13))
    S = max(c["S"], 4)
    hi = int(rng.integers(1, 201))
    prefix = N * c["bs"]
    b = workloads.make_batch(_BASE[c["kind"]], device=DEV, num_seqs=S, num_heads=c["H"],
                             num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["bs"],
                             lens=("prefix", prefix, 1, hi), max_len=prefix + hi,
                             pool=("exact",), poison=True, seed=c["seed"])
    ref, _, _ = oracle_step(b)
    print("CASE random cascade", c, "prefix blocks", N, "suffix up to", hi, flush=True)
    kc, vc = gpu_caches(b)
    pa.kv_append(b.k_new, b.v_new, b.slot_mapping, kc, vc, b.k_scale, b.v_scale)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pa.decode_cascade(b.q, kc, vc, b.block_tables, b.seq_lens, N, b.scale,
                            k_scale=b.k_scale, v_scale=b.v_scale,
                            partition_tokens=c["chunk"] * c["bs"], err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    check_close(out, ref, b.cache_dtype, f"random cascade {c}")


def _draw_long(rng):
    kind = ["f32", "bf16", "bf16", "fp8"][int(rng.integers(0, 4))]
    Hkv = int(rng.choice([1, 2, 4, 8]))
    return dict(kind=kind, S=int(rng.integers(1, 70)), Hkv=Hkv, H=Hkv * int(rng.choice([1, 2, 4, 8])),
                D=int(rng.choice([64, 128])), bs=int(rng.choice([16, 32])),
                max_len=int(rng.integers(1, 4001)), chunk=int(rng.choice([0, 0, 1, 3, 16, 64])),
                seed=int(rng.integers(0, 2**31)))


_RNG_LONG = np.random.default_rng(20261203)
APPEND = [_draw_long(_RNG_LONG) for _ in range(16)]


def _bits_dtype(t):
    """Integer dtype of a cache's bit patterns, so NaN-poisoned slots compare equal."""
    return {torch.float32: torch.int32, torch.bfloat16: torch.int16}.get(t.dtype, t.dtype)


@pytest.mark.parametrize("c", APPEND, ids=_ids(APPEND))
def test_random_decode_append(c):
    """Longer sequences (up to 4000 tokens, 1-69 of them) and fixed runs of
    partitions: pa_decode_append bit for bit equal to pa_kv_append then
    pa_decode (output and both whole caches), that within tolerance of the
    oracle, and pa_decode_noalloc equal to pa_decode where its static
    workspace suffices."""
    b = _batch(c, lens=("uniform", 1, c["max_len"]), max_len=c["max_len"])
    ref, _, _ = oracle_step(b)
    P = c["chunk"] * c["bs"]
    print("CASE random decode_append", c, flush=True)
    kc, vc = gpu_caches(b)
    sep = gpu_step(b, kc, vc, partition_tokens=P)
    kc2, vc2 = gpu_caches(b)
    fused = pa.decode_append(b.k_new, b.v_new, b.slot_mapping, b.q, kc2, vc2, b.block_tables,
                             b.seq_lens, b.scale, k_scale=b.k_scale, v_scale=b.v_scale,
                             partition_tokens=P)
    torch.cuda.synchronize()
    check_close(sep, ref, b.cache_dtype, f"random decode_append {c}")
    assert torch.equal(fused, sep)
    for x, y in ((kc, kc2), (vc, vc2)):
        assert torch.equal(x.view(_bits_dtype(x)), y.view(_bits_dtype(x)))
    if pa.decode_workspace_size(b.q, kc2, b.block_tables, P) <= pa.NOALLOC_MAX_WORKSPACE:
        out = torch.empty_like(b.q)
        pa.decode_noalloc(b.q, kc2, vc2, b.block_tables, b.seq_lens, b.scale, out,
                          k_scale=b.k_scale, v_scale=b.v_scale, partition_tokens=P)
        torch.cuda.synchronize()
        assert torch.equal(out, sep)


def _draw_wide(rng):
    c = _draw_long(rng)
    c.update(S=int(rng.integers(257, 1201)), max_len=int(rng.integers(1, 601)))
    return c


_RNG_WIDE = np.random.default_rng(20261204)
WIDE = [_draw_wide(_RNG_WIDE) for _ in range(6)]


@pytest.mark.parametrize("c", WIDE, ids=_ids(WIDE))
def test_random_wide_batches(c):
    """257-1200 sequences: the chunk location for batches beyond one
    256-sequence register pass (two passes over the lengths), balanced
    chunks and runs of partitions, the fused append bit for bit against the
    two calls."""
    test_random_decode_append(c)
