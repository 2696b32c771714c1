"""Seeded synthetic decode batches for paged attention.

This module only *draws* inputs: sequence lengths, a physical placement of
the KV blocks in a shared pool, the per-sequence block tables that record that
placement, random query/key/value values and the slot each new token is
written to.  It holds none of the attention or quantisation arithmetic, so the
CPU oracle and the GPU library can both be fed from it without sharing any of
the computation they are checked on.

Shapes and layouts (the vLLM concept page, "Technical principles" section and
its PagedAttention pseudocode; the vLLM-internals blog, section 1.1):

  q, out                  [num_seqs, num_heads, head_dim]
  key/value pool          [num_blocks, block_size, num_kv_heads, head_dim]
  block_tables   int32    [num_seqs, max_blocks_per_seq]  (entry j = physical
                          block holding logical block j; unused entries = -1)
  seq_lens       int32    [num_seqs]  tokens to attend over, the token being
                          appended in this step included
  slot_mapping   int64    [num_seqs]  physical slot (block * block_size +
                          offset) of that new token

Workloads (sizes as named): see ``CONFIGS``.  Everything is reproducible from
``seed``; random draws happen in a fixed order (lengths, placement, q, K pool,
V pool, new K rows, new V rows).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# --------------------------------------------------------------------------
# Named decode workloads.
#   lens: ("uniform", lo, hi)              L ~ U{lo..hi}
#         ("lognormal", median, sigma, lo, hi)  L = clip(round(median*e^{sigma N(0,1)}), lo, hi)
#         ("prefix", prefix, lo, hi)       L = prefix + U{lo..hi}; the prefix blocks
#                                          are one physical copy shared by all sequences
#         ("fixed", n)                     L = n
#   pool: ("fixed", n)    n blocks; the sequences' blocks are a random choice without
#                         replacement, the rest stay unused
#         ("factor", f)   ceil(f * blocks needed) blocks, shuffled placement
#         ("exact",)      exactly the blocks needed (shared prefix counted once), shuffled
# --------------------------------------------------------------------------
CONFIGS = {
    "tiny_f32": dict(
        num_seqs=4, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
        q_dtype="f32", cache_dtype="f32", lens=("uniform", 1, 200), pool=("fixed", 128),
        max_len=200, partition_tokens=None),
    "llama3_8b_bf16": dict(
        num_seqs=64, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype="bf16", cache_dtype="bf16", lens=("uniform", 512, 4096), pool=("factor", 1.2),
        max_len=4096, partition_tokens=None),
    "qwen3_0p6b_bf16": dict(
        num_seqs=256, num_heads=16, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype="bf16", cache_dtype="bf16", lens=("lognormal", 512, 1.0, 128, 2048),
        pool=("factor", 1.2), max_len=2048, partition_tokens=None),
    "shared_prefix_bf16": dict(
        num_seqs=128, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype="bf16", cache_dtype="bf16", lens=("prefix", 2048, 1, 512), pool=("exact",),
        max_len=2048 + 512, partition_tokens=None),
    "long_fp8": dict(
        num_seqs=8, num_heads=64, num_kv_heads=8, head_dim=128, block_size=32,
        q_dtype="bf16", cache_dtype="fp8_e4m3", lens=("fixed", 131072), pool=("exact",),
        max_len=131072, partition_tokens=512),
    # Speculative-decoding verify step on the Llama-3-8B-shaped batch: each
    # sequence checks 7 drafted tokens plus the last accepted one (8 new query
    # tokens; the P-EAGLE page reports its best speed-up at 7 drafts).
    "llama3_8b_bf16_spec8": dict(
        num_seqs=64, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype="bf16", cache_dtype="bf16", lens=("uniform", 512, 4096), pool=("factor", 1.2),
        max_len=4096, partition_tokens=None, query_lens=("fixed", 8)),
}

# Seeds, one per workload (block workloads below take 6 to 8).
SEEDS = {"tiny_f32": 1, "llama3_8b_bf16": 2, "qwen3_0p6b_bf16": 3, "shared_prefix_bf16": 4,
         "long_fp8": 5, "llama3_8b_bf16_spec8": 9}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
# Largest finite magnitude of the OCP E4M3FN format (exponent 1111, mantissa 110).
E4M3_MAX = 448.0


@dataclasses.dataclass
class DecodeBatch:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    q_dtype: str
    cache_dtype: str
    scale: float
    seq_lens: torch.Tensor        # int32 [S]            (on `device`)
    block_tables: torch.Tensor    # int32 [S, max_nb]    (-1 beyond each sequence's blocks)
    q: torch.Tensor               # [S, H, D]            q_dtype
    key_pool: torch.Tensor        # [NB, bs, Hkv, D]     values (bf16/f32) -- for an fp8
    value_pool: torch.Tensor      #                      cache these are the bf16 values
                                  #                      that get quantised into it
    k_new: torch.Tensor           # [S, Hkv, D]
    v_new: torch.Tensor           # [S, Hkv, D]
    slot_mapping: torch.Tensor    # int64 [S]
    k_scale: float = 1.0          # per-tensor fp32 scales of an fp8 cache (1.0 otherwise)
    v_scale: float = 1.0
    partition_tokens: Optional[int] = None
    poisoned: bool = False
    # Several new tokens per sequence (None: one): sequence s owns rows
    # query_start_loc[s] .. query_start_loc[s+1]-1 of q, k_new, v_new and
    # slot_mapping, its last q_len positions in order.
    query_start_loc: Optional[torch.Tensor] = None   # int32 [S + 1]
    max_query_len: int = 1
    # leading logical blocks every sequence shares (the same physical blocks)
    shared_prefix_blocks: int = 0

    @property
    def num_query_tokens(self) -> int:
        return self.q.shape[0]

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[self.cache_dtype]

    @property
    def q_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2}[self.q_dtype]

    def pool_slots(self) -> torch.Tensor:
        """Every slot of the pool in order: appending ``key_pool`` reshaped to
        [NB*bs, Hkv, D] at these slots fills the whole cache."""
        return torch.arange(self.num_blocks * self.block_size, dtype=torch.int64,
                            device=self.key_pool.device)


def _draw_lens(rng: np.random.Generator, spec, S: int) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        return rng.integers(spec[1], spec[2] + 1, size=S)
    if kind == "lognormal":
        median, sigma, lo, hi = spec[1:]
        raw = np.rint(median * np.exp(sigma * rng.standard_normal(S)))
        return np.clip(raw, lo, hi).astype(np.int64)
    if kind == "prefix":
        return spec[1] + rng.integers(spec[2], spec[3] + 1, size=S)
    if kind == "fixed":
        return np.full(S, spec[1], dtype=np.int64)
    raise ValueError(f"unknown length spec {spec!r}")


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def make_batch(name: str = "tiny_f32", seed: Optional[int] = None, device="cpu",
               poison: bool = False, **overrides) -> DecodeBatch:
    """Draw one decode batch of workload ``name``.

    ``overrides`` replaces any field of the workload (e.g. ``num_seqs=8``,
    ``lens=("uniform", 1, 300)``, ``max_len=300``) to make reduced-size cases.
    With ``poison=True`` every pool slot that no sequence may read (blocks no
    table names, and the slots at positions >= L in each sequence's last
    block) holds NaN, so a kernel that lets them reach the result is caught.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = SEEDS.get(name, 0) if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    S, H, Hkv = cfg["num_seqs"], cfg["num_heads"], cfg["num_kv_heads"]
    D, bs = cfg["head_dim"], cfg["block_size"]
    if H % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    max_nb = _cdiv(cfg["max_len"], bs)

    # 1. lengths
    lens = _draw_lens(rng, cfg["lens"], S).astype(np.int64)
    if lens.min() < 1 or lens.max() > max_nb * bs:
        raise ValueError("drawn length outside [1, capacity]")
    nblk = (lens + bs - 1) // bs
    # 1b. new query tokens per sequence (multi-token workloads only)
    qspec = cfg.get("query_lens")
    if qspec is None:
        qlens = np.ones(S, dtype=np.int64)
    else:
        qlens = np.minimum(_draw_lens(rng, qspec, S).astype(np.int64), lens)
        if qlens.min() < 0:
            raise ValueError("negative query length")
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])

    # 2. placement of logical blocks in the physical pool
    pool = cfg["pool"]
    tables = np.full((S, max_nb), -1, dtype=np.int32)
    if cfg["lens"][0] == "prefix":
        prefix = cfg["lens"][1]
        if prefix % bs:
            raise ValueError("shared prefix must be a whole number of blocks")
        n_shared = prefix // bs
        private = nblk - n_shared
        needed = n_shared + int(private.sum())
        NB = needed if pool[0] == "exact" else (
            math.ceil(pool[1] * needed) if pool[0] == "factor" else pool[1])
        perm = rng.permutation(NB)
        shared_ids = perm[:n_shared]
        cursor = n_shared
        for s in range(S):
            tables[s, :n_shared] = shared_ids
            tables[s, n_shared:nblk[s]] = perm[cursor:cursor + private[s]]
            cursor += private[s]
    else:
        needed = int(nblk.sum())
        if pool[0] == "fixed":
            NB = pool[1]
        elif pool[0] == "factor":
            NB = math.ceil(pool[1] * needed)
        else:
            NB = needed
        if needed > NB:
            raise ValueError("pool too small for the drawn lengths")
        perm = rng.permutation(NB)
        cursor = 0
        for s in range(S):
            tables[s, :nblk[s]] = perm[cursor:cursor + nblk[s]]
            cursor += nblk[s]

    # 3. values: q, pool K, pool V, new K rows, new V rows -- all N(0, 1)
    val_dtype = torch.float32 if cfg["cache_dtype"] == "f32" else torch.bfloat16
    q = _randn((T, H, D), gen, device).to(_TORCH_DTYPE[cfg["q_dtype"]])
    key_pool = _randn((NB, bs, Hkv, D), gen, device, out_dtype=val_dtype)
    value_pool = _randn((NB, bs, Hkv, D), gen, device, out_dtype=val_dtype)
    k_new = _randn((T, Hkv, D), gen, device).to(val_dtype)
    v_new = _randn((T, Hkv, D), gen, device).to(val_dtype)

    # 4. the slots of each sequence's new tokens (positions L-q_len .. L-1)
    seq_of = np.repeat(np.arange(S), qlens)
    pos = lens[seq_of] - qlens[seq_of] + (np.arange(T) - qsl[:-1][seq_of])
    slots = tables[seq_of, pos // bs].astype(np.int64) * bs + (pos % bs)

    # 5. per-tensor fp8 scales: largest magnitude maps to the format's largest value
    k_scale = v_scale = 1.0
    if cfg["cache_dtype"] == "fp8_e4m3":
        k_amax = max(float(key_pool.abs().max()), float(k_new.abs().max()))
        v_amax = max(float(value_pool.abs().max()), float(v_new.abs().max()))
        k_scale = float(np.float32(k_amax) / np.float32(E4M3_MAX))
        v_scale = float(np.float32(v_amax) / np.float32(E4M3_MAX))

    seq_lens_t = torch.from_numpy(lens.astype(np.int32)).to(device)
    tables_t = torch.from_numpy(tables).to(device)
    if poison:
        _poison(key_pool, value_pool, tables, lens, bs)

    return DecodeBatch(
        name=name, num_seqs=S, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=bs,
        num_blocks=NB, max_blocks_per_seq=max_nb, q_dtype=cfg["q_dtype"],
        cache_dtype=cfg["cache_dtype"], scale=1.0 / math.sqrt(D),
        seq_lens=seq_lens_t, block_tables=tables_t, q=q, key_pool=key_pool,
        value_pool=value_pool, k_new=k_new, v_new=v_new,
        slot_mapping=torch.from_numpy(slots).to(device), k_scale=k_scale, v_scale=v_scale,
        partition_tokens=cfg.get("partition_tokens"), poisoned=poison,
        query_start_loc=None if qspec is None else torch.from_numpy(qsl).to(device),
        max_query_len=1 if qspec is None else max(1, int(qlens.max())),
        shared_prefix_blocks=cfg["lens"][1] // bs if cfg["lens"][0] == "prefix" else 0)


def _randn(shape, gen, device, out_dtype=torch.float32, chunk=1 << 26):
    """N(0,1) draws, generated in float32 in chunks of the leading dim so that
    a multi-GiB pool never needs a float32 copy of itself."""
    n_lead = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = torch.empty(shape, dtype=out_dtype, device=device)
    flat = out.view(n_lead, inner)
    step = max(1, chunk // max(inner, 1))
    for i in range(0, n_lead, step):
        j = min(n_lead, i + step)
        flat[i:j] = torch.randn((j - i, inner), generator=gen, device=device,
                                dtype=torch.float32).to(out_dtype)
    return out


def unread_slot_mask(block_tables, seq_lens, num_blocks: int, block_size: int) -> np.ndarray:
    """Bool [NB, bs]: True where no sequence may read the slot (blocks no table
    names, and slots at positions >= L in a sequence's last block)."""
    tables = np.asarray(block_tables.cpu() if torch.is_tensor(block_tables) else block_tables)
    lens = np.asarray(seq_lens.cpu() if torch.is_tensor(seq_lens) else seq_lens)
    readable = np.zeros((num_blocks, block_size), dtype=bool)
    for s in range(tables.shape[0]):
        nb = -(-int(lens[s]) // block_size)
        for j in range(nb):
            n_valid = min(block_size, int(lens[s]) - j * block_size)
            readable[tables[s, j], :n_valid] = True
    return ~readable


def _poison(key_pool, value_pool, tables, lens, bs):
    mask = torch.from_numpy(unread_slot_mask(tables, lens, key_pool.shape[0], bs))
    mask = mask.to(key_pool.device)
    key_pool[mask] = float("nan")
    value_pool[mask] = float("nan")


# --------------------------------------------------------------------------
# Block-maintenance workloads: clearing newly allocated blocks and copying
# blocks.  A workload is a set of regions (caches) that share one block
# geometry -- ``layers`` layers x {K, V}, each a pool of ``num_blocks`` blocks of
# block_size x kv_heads x head_dim elements -- and a list of block ids (clear)
# or (src, dst) pairs (copy).
#
# The clearing sizes follow the vLLM v0.17.1 notes (fix #35219), which give
# only totals: ~515 blocks (~920 MiB) cleared for a prefill step, ~30 for a
# decode step.  The geometry is a reading chosen to match ~1.8 MiB per block:
# 15 attention layers x {K, V} x 64 tokens x 2 KV heads x 256 dims in bf16
# (64 KiB per cache block, 1.875 MiB per block over all caches).
# Copy-on-write uses the Llama-3-8B-shaped cache (32 layers x {K, V}, 16 tokens
# x 8 KV heads x 128 dims, bf16: 32 KiB per cache block), one copied block per
# sequence of a 256-sequence batch.
# --------------------------------------------------------------------------
BLOCK_CONFIGS = {
    "block_zero_prefill": dict(op="zero", layers=15, block_size=64, kv_heads=2, head_dim=256,
                               elem_bytes=2, num_blocks=2048, items=515),
    "block_zero_decode": dict(op="zero", layers=15, block_size=64, kv_heads=2, head_dim=256,
                              elem_bytes=2, num_blocks=2048, items=30),
    "block_copy_cow": dict(op="copy", layers=32, block_size=16, kv_heads=8, head_dim=128,
                           elem_bytes=2, num_blocks=4096, items=256),
}
BLOCK_SEEDS = {name: 6 + i for i, name in enumerate(BLOCK_CONFIGS)}


@dataclasses.dataclass
class BlockCase:
    name: str
    op: str                       # "zero" or "copy"
    regions: list                 # uint8 tensors [num_blocks, block_bytes], one per cache
    items: torch.Tensor           # int32 [n] block ids, or [n, 2] (src, dst) pairs
    block_bytes: int
    num_blocks: int

    @property
    def region_count(self) -> int:
        return len(self.regions)


def make_block_case(name: str, seed: Optional[int] = None, device="cpu",
                    **overrides) -> BlockCase:
    """Draw the regions (random bytes, no zero byte, so a cleared byte is
    always visible) and the items of block workload ``name``.  Clear: distinct
    random ids.  Copy: distinct sources and distinct destinations, disjoint
    from each other."""
    cfg = dict(BLOCK_CONFIGS[name])
    cfg.update(overrides)
    seed = BLOCK_SEEDS.get(name, 0) if seed is None else seed
    gen = torch.Generator(device="cpu").manual_seed(seed)
    NB, n = cfg["num_blocks"], cfg["items"]
    block_bytes = cfg["block_size"] * cfg["kv_heads"] * cfg["head_dim"] * cfg["elem_bytes"]
    perm = torch.randperm(NB, generator=gen)
    if cfg["op"] == "zero":
        if n > NB:
            raise ValueError("more ids than blocks")
        items = perm[:n].to(torch.int32)
    else:
        if 2 * n > NB:
            raise ValueError("more pairs than fit the pool")
        items = torch.stack([perm[:n], perm[n:2 * n]], dim=1).to(torch.int32).contiguous()
    regions = []
    dev_gen = torch.Generator(device=device).manual_seed(seed + 1000)
    for _ in range(2 * cfg["layers"]):
        regions.append(torch.randint(1, 256, (NB, block_bytes), dtype=torch.uint8,
                                     device=device, generator=dev_gen))
    return BlockCase(name, cfg["op"], regions, items, block_bytes, NB)


# --------------------------------------------------------------------------
# Step-metadata workloads: a persistent state table of `rows` requests
# (block tables of max_blocks entries over a pool of num_blocks, token ids up
# to max_blocks * block_size) and one step's batch: `reqs` requests in a
# random order, each with U{lo..hi} new tokens, outputs sized `max_tokens`.
# "prep_decode" is the Llama-3-8B-shaped decode batch (64 requests, one token
# each); "prep_mixed" a chunked-prefill-sized step (256 requests, up to 32
# new tokens each, 8192 token rows).
# --------------------------------------------------------------------------
PREP_CONFIGS = {
    "prep_decode": dict(rows=256, reqs=64, new=(1, 1), max_tokens=64, block_size=16,
                        max_blocks=256, num_blocks=16384),
    "prep_mixed": dict(rows=1024, reqs=256, new=(0, 32), max_tokens=8192, block_size=16,
                       max_blocks=256, num_blocks=65536),
}
PREP_SEEDS = {"prep_decode": 10, "prep_mixed": 11}


def make_prep_case(name: str, seed: Optional[int] = None, device="cpu", **overrides) -> dict:
    """State table and step batch (int32 tensors on ``device``) of workload
    ``name``: idx_mapping, num_scheduled, num_computed, block_table, token_ids,
    plus block_size, num_blocks, max_tokens.  Every request has room in its
    table for its computed and new tokens."""
    cfg = dict(PREP_CONFIGS[name])
    cfg.update(overrides)
    rng = np.random.default_rng(PREP_SEEDS.get(name, 0) if seed is None else seed)
    R, S, bs, max_nb = cfg["rows"], cfg["reqs"], cfg["block_size"], cfg["max_blocks"]
    max_len = max_nb * bs
    lo, hi = cfg["new"]
    n = rng.integers(lo, hi + 1, S)
    computed = rng.integers(0, max_len - hi, R)
    block_table = rng.integers(0, cfg["num_blocks"], size=(R, max_nb))
    token_ids = rng.integers(0, 150000, size=(R, max_len))
    idx = rng.permutation(R)[:S]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x).astype(np.int32)).to(device)
    return dict(idx_mapping=t(idx), num_scheduled=t(n), num_computed=t(computed),
                block_table=t(block_table), token_ids=t(token_ids), block_size=bs,
                num_blocks=cfg["num_blocks"], max_tokens=cfg["max_tokens"])
