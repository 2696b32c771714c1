"""paged_kv_cache_54_amd -- paged KV-cache append and paged decode attention
for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libpa.so`` (include/pa.h): argument
marshalling only.  Every step of the computation runs in the library's HIP
kernels; PyTorch supplies device memory and the current stream.  If the
library has not been built, every call raises ``RuntimeError`` -- there is no
fallback implementation.

    kv_append(k, v, slot_mapping, key_cache, value_cache, k_scale=1, v_scale=1)
    decode(q, key_cache, value_cache, block_tables, seq_lens, scale, out=None, ...)
    decode_workspace_size(q, key_cache, block_tables, ...)
    decode_multi(q, query_start_loc, max_query_len, key_cache, value_cache, ...)
    decode_cascade(q, key_cache, value_cache, block_tables, seq_lens, prefix_blocks, scale, ...)
    decode_multi_workspace_size(q, max_query_len, key_cache, block_tables, ...)
    zero_blocks(block_ids, regions)
    copy_blocks(block_pairs, src_regions, dst_regions)
    region_table(caches, device)
    prepare_step(idx_mapping, num_scheduled, num_computed, block_table, token_ids, ...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = ["kv_append", "decode", "decode_append", "decode_workspace_size", "decode_noalloc", "decode_multi",
           "decode_cascade", "NOALLOC_MAX_WORKSPACE",
           "decode_cascade_workspace_size",
           "decode_multi_workspace_size", "zero_blocks", "copy_blocks",
           "region_table", "Regions", "prepare_step", "PaError", "status_string", "version", "library_path",
           "VARIANT_AUTO", "VARIANT_VALU", "VARIANT_MFMA", "PARTIALS_F32", "PARTIALS_BF16",
           "DEVERR_BLOCK_ID", "DEVERR_SEQ_LEN",
           "DEVERR_SLOT", "DEVERR_REGION", "DEVERR_QUERY", "DEVERR_STEP", "DEVERR_PREFIX"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3, PA_I32, PA_I64 = 0, 1, 2, 3, 4
VARIANT_AUTO, VARIANT_VALU, VARIANT_MFMA = 0, 1, 2
PARTIALS_F32, PARTIALS_BF16 = 0, 1
NOALLOC_MAX_WORKSPACE = 96 << 20           # PA_NOALLOC_MAX_WORKSPACE
DEVERR_BLOCK_ID, DEVERR_SEQ_LEN, DEVERR_SLOT, DEVERR_REGION, DEVERR_QUERY = 0x1, 0x2, 0x4, 0x8, 0x10
DEVERR_STEP, DEVERR_PREFIX = 0x20, 0x40

_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3,
           torch.float8_e4m3fn: PA_FP8_E4M3, torch.int32: PA_I32, torch.int64: PA_I64}


class PaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class PaOpts(ctypes.Structure):
    _fields_ = [("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("partition_tokens", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("err_flag", ctypes.c_void_p), ("kernel_events", ctypes.c_void_p * 2),
                ("partials", ctypes.c_int32)]


class PaStepState(ctypes.Structure):
    _fields_ = [("num_computed", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("token_ids", ctypes.c_void_p), ("num_rows", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("max_len", ctypes.c_int32)]


class PaStepInputs(ctypes.Structure):
    _fields_ = [("query_start_loc", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("positions", ctypes.c_void_p), ("input_ids", ctypes.c_void_p),
                ("slot_mapping", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
                ("max_tokens", ctypes.c_int32)]


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python paged_kv_cache_54_amd/build.py")
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        lib.pa_kv_append.restype = ctypes.c_int
        lib.pa_kv_append.argtypes = [P(PaTensor), P(PaTensor), P(PaTensor), P(PaTensor),
                                     P(PaTensor), P(PaOpts), ctypes.c_void_p]
        lib.pa_decode.restype = ctypes.c_int
        lib.pa_decode.argtypes = [P(PaTensor), P(PaTensor), P(PaTensor), P(PaTensor),
                                  P(PaTensor), ctypes.c_float, P(PaTensor), P(PaOpts),
                                  ctypes.c_void_p]
        lib.pa_decode_append.restype = ctypes.c_int
        lib.pa_decode_append.argtypes = [P(PaTensor)] * 8 + [ctypes.c_float, P(PaTensor),
                                                             P(PaOpts), ctypes.c_void_p]
        lib.pa_decode_cascade.restype = ctypes.c_int
        lib.pa_decode_cascade.argtypes = [P(PaTensor), P(PaTensor), P(PaTensor), P(PaTensor),
                                          P(PaTensor), ctypes.c_int32, ctypes.c_float,
                                          P(PaTensor), P(PaOpts), ctypes.c_void_p]
        lib.pa_decode_cascade_workspace_size.restype = ctypes.c_int
        lib.pa_decode_cascade_workspace_size.argtypes = [P(PaTensor), P(PaTensor), P(PaTensor),
                                                         ctypes.c_int32, P(PaOpts),
                                                         P(ctypes.c_size_t)]
        lib.pa_decode_multi.restype = ctypes.c_int
        lib.pa_decode_multi.argtypes = [P(PaTensor), P(PaTensor), ctypes.c_int32, P(PaTensor),
                                        P(PaTensor), P(PaTensor), P(PaTensor), ctypes.c_float,
                                        P(PaTensor), P(PaOpts), ctypes.c_void_p]
        lib.pa_decode_multi_workspace_size.restype = ctypes.c_int
        lib.pa_decode_multi_workspace_size.argtypes = [P(PaTensor), ctypes.c_int32, P(PaTensor),
                                                       P(PaTensor), P(PaOpts),
                                                       P(ctypes.c_size_t)]
        lib.pa_decode_noalloc.restype = ctypes.c_int
        lib.pa_decode_noalloc.argtypes = [P(PaTensor), P(PaTensor), P(PaTensor), P(PaTensor),
                                          P(PaTensor), ctypes.c_float, P(PaTensor), P(PaOpts),
                                          ctypes.c_void_p]
        lib.pa_decode_workspace_size.restype = ctypes.c_int
        lib.pa_decode_workspace_size.argtypes = [P(PaTensor), P(PaTensor), P(PaTensor),
                                                 P(PaOpts), P(ctypes.c_size_t)]
        lib.pa_opts_init.restype = None
        lib.pa_opts_init.argtypes = [P(PaOpts)]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_version.restype = ctypes.c_int
        lib.pa_version.argtypes = []
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.pa_prepare_step.restype = ctypes.c_int
        lib.pa_prepare_step.argtypes = [vp, vp, i32, P(PaStepState), i32, i32, P(PaStepInputs),
                                        P(PaOpts), vp]
        lib.pa_zero_blocks.restype = ctypes.c_int
        lib.pa_zero_blocks.argtypes = [vp, i64, vp, i32, i64, i64, i64, P(PaOpts), vp]
        lib.pa_copy_blocks.restype = ctypes.c_int
        lib.pa_copy_blocks.argtypes = [vp, i64, vp, vp, i32, i64, i64, i64, i64, P(PaOpts), vp]
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return _load().pa_status_string(status).decode()


def version() -> int:
    return _load().pa_version()


def describe(t: torch.Tensor) -> PaTensor:
    """pa_tensor descriptor of a torch tensor (no copy)."""
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d = PaTensor()
    d.data = t.data_ptr() if t.numel() else 0
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _opts(k_scale=1.0, v_scale=1.0, partition_tokens=0, variant=VARIANT_AUTO, workspace=None,
          err_flag=None, events: Optional[Sequence[int]] = None,
          bf16_partials=False) -> PaOpts:
    o = PaOpts()
    _load().pa_opts_init(ctypes.byref(o))
    o.k_scale = float(k_scale)
    o.v_scale = float(v_scale)
    o.partition_tokens = int(partition_tokens)
    o.variant = int(variant)
    o.partials = PARTIALS_BF16 if bf16_partials else PARTIALS_F32
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    if err_flag is not None:
        if err_flag.dtype != torch.int32 or err_flag.numel() < 1 or not err_flag.is_cuda:
            raise TypeError("err_flag must be a device int32 tensor")
        o.err_flag = err_flag.data_ptr()
    if events is not None:
        o.kernel_events[0] = events[0]
        o.kernel_events[1] = events[1]
    return o


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(stream):
    """The torch stream object of a call's ``stream`` argument (None: the
    current stream; a raw hipStream_t handle is wrapped).  Outputs and
    workspaces a call allocates are allocated on it, so the caching allocator
    reuses a freed workspace only for work queued after the call's kernels on
    that stream, not while they still run."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(_stream(stream))


def _check(fn: str, rc: int):
    if rc != 0:
        raise PaError(fn, rc)


def kv_append(k, v, slot_mapping, key_cache, value_cache, k_scale=1.0, v_scale=1.0,
              err_flag=None, stream=None):
    """Write rows k, v [T, Hkv, D] into key_cache / value_cache [NB, bs, Hkv, D]
    at slot_mapping[t] (int64; negative = skip).  fp8 caches (uint8 or
    float8_e4m3fn tensors) store nearest-e4m3(x * (1/scale))."""
    lib = _load()
    o = _opts(k_scale, v_scale, err_flag=err_flag)
    args = [describe(x) for x in (k, v, slot_mapping, key_cache, value_cache)]
    _check("pa_kv_append", lib.pa_kv_append(*[ctypes.byref(x) for x in args], ctypes.byref(o),
                                            _stream(stream)))


def decode_workspace_size(q, key_cache, block_tables, partition_tokens=0,
                          variant=VARIANT_AUTO, bf16_partials=False) -> int:
    lib = _load()
    o = _opts(partition_tokens=partition_tokens, variant=variant, bf16_partials=bf16_partials)
    n = ctypes.c_size_t(0)
    _check("pa_decode_workspace_size",
           lib.pa_decode_workspace_size(ctypes.byref(describe(q)), ctypes.byref(describe(key_cache)),
                                        ctypes.byref(describe(block_tables)), ctypes.byref(o),
                                        ctypes.byref(n)))
    return n.value


def decode(q, key_cache, value_cache, block_tables, seq_lens, scale, out=None, k_scale=1.0,
           v_scale=1.0, partition_tokens=0, variant=VARIANT_AUTO, workspace=None,
           err_flag=None, events=None, stream=None, bf16_partials=False):
    """Paged decode attention; returns ``out`` [S, H, D] (same dtype as q).

    ``workspace``: optional uint8 device tensor of at least
    ``decode_workspace_size(...)`` bytes; allocated here (torch caching
    allocator) when needed and not given.  ``events``: optional pair of raw
    hipEvent_t handles recorded around the attention kernel.
    ``bf16_partials``: store split-KV partial accumulators as bf16 instead of
    fp32 (bf16 outputs only)."""
    lib = _load()
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            need = decode_workspace_size(q, key_cache, block_tables, partition_tokens, variant,
                                         bf16_partials)
            if need:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = _opts(k_scale, v_scale, partition_tokens, variant, workspace, err_flag, events,
              bf16_partials)
    args = [describe(x) for x in (q, key_cache, value_cache, block_tables, seq_lens)]
    _check("pa_decode", lib.pa_decode(*[ctypes.byref(x) for x in args], float(scale),
                                      ctypes.byref(describe(out)), ctypes.byref(o),
                                      ts.cuda_stream))
    return out


def decode_append(k, v, slot_mapping, q, key_cache, value_cache, block_tables, seq_lens, scale,
                  out=None, k_scale=1.0, v_scale=1.0, partition_tokens=0, variant=VARIANT_AUTO,
                  workspace=None, err_flag=None, events=None, stream=None, bf16_partials=False):
    """pa_decode_append: kv_append(k, v, slot_mapping, caches) then decode(q,
    caches, ...), the append done inside the decode kernel where it takes
    one (one new bf16 row per sequence on the matrix-core kernels).  Same
    arguments and workspace as ``decode``; returns ``out``."""
    lib = _load()
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            need = decode_workspace_size(q, key_cache, block_tables, partition_tokens, variant,
                                         bf16_partials)
            if need:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = _opts(k_scale, v_scale, partition_tokens, variant, workspace, err_flag, events,
              bf16_partials)
    args = [describe(x) for x in (k, v, slot_mapping, q, key_cache, value_cache, block_tables,
                                  seq_lens)]
    _check("pa_decode_append",
           lib.pa_decode_append(*[ctypes.byref(x) for x in args], float(scale),
                                ctypes.byref(describe(out)), ctypes.byref(o), ts.cuda_stream))
    return out


def decode_noalloc(q, key_cache, value_cache, block_tables, seq_lens, scale, out, k_scale=1.0,
                   v_scale=1.0, partition_tokens=0, variant=VARIANT_AUTO, err_flag=None,
                   stream=None, bf16_partials=False):
    """pa_decode_noalloc: pa_decode with the library's static device
    workspace (NOALLOC_MAX_WORKSPACE bytes per device, shared by every call
    on that device: calls that may overlap on one device race).  ``out``
    [S, H, D] is required; nothing is allocated, here or in the library."""
    lib = _load()
    o = _opts(k_scale, v_scale, partition_tokens, variant, None, err_flag, None, bf16_partials)
    args = [describe(x) for x in (q, key_cache, value_cache, block_tables, seq_lens)]
    _check("pa_decode_noalloc",
           lib.pa_decode_noalloc(*[ctypes.byref(x) for x in args], float(scale),
                                 ctypes.byref(describe(out)), ctypes.byref(o), _stream(stream)))
    return out


def decode_cascade_workspace_size(q, key_cache, block_tables, prefix_blocks, partition_tokens=0,
                                  variant=VARIANT_AUTO, bf16_partials=False) -> int:
    lib = _load()
    o = _opts(partition_tokens=partition_tokens, variant=variant, bf16_partials=bf16_partials)
    n = ctypes.c_size_t(0)
    _check("pa_decode_cascade_workspace_size",
           lib.pa_decode_cascade_workspace_size(ctypes.byref(describe(q)),
                                                ctypes.byref(describe(key_cache)),
                                                ctypes.byref(describe(block_tables)),
                                                int(prefix_blocks), ctypes.byref(o),
                                                ctypes.byref(n)))
    return n.value


def decode_cascade(q, key_cache, value_cache, block_tables, seq_lens, prefix_blocks, scale,
                   out=None, k_scale=1.0, v_scale=1.0, partition_tokens=0, variant=VARIANT_AUTO,
                   workspace=None, err_flag=None, events=None, stream=None, bf16_partials=False):
    """pa_decode for a batch whose sequences share their first prefix_blocks
    blocks: the shared blocks are read once per group of sequences."""
    lib = _load()
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            need = decode_cascade_workspace_size(q, key_cache, block_tables, prefix_blocks,
                                                 partition_tokens, variant, bf16_partials)
            if need:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = _opts(k_scale, v_scale, partition_tokens, variant, workspace, err_flag, events,
              bf16_partials)
    args = [describe(x) for x in (q, key_cache, value_cache, block_tables, seq_lens)]
    _check("pa_decode_cascade",
           lib.pa_decode_cascade(*[ctypes.byref(x) for x in args], int(prefix_blocks),
                                 float(scale), ctypes.byref(describe(out)), ctypes.byref(o),
                                 ts.cuda_stream))
    return out


def decode_multi_workspace_size(q, max_query_len, key_cache, block_tables, partition_tokens=0,
                                variant=VARIANT_AUTO, bf16_partials=False) -> int:
    lib = _load()
    o = _opts(partition_tokens=partition_tokens, variant=variant, bf16_partials=bf16_partials)
    n = ctypes.c_size_t(0)
    _check("pa_decode_multi_workspace_size",
           lib.pa_decode_multi_workspace_size(ctypes.byref(describe(q)), int(max_query_len),
                                              ctypes.byref(describe(key_cache)),
                                              ctypes.byref(describe(block_tables)),
                                              ctypes.byref(o), ctypes.byref(n)))
    return n.value


def decode_multi(q, query_start_loc, max_query_len, key_cache, value_cache, block_tables,
                 seq_lens, scale, out=None, k_scale=1.0, v_scale=1.0, partition_tokens=0,
                 variant=VARIANT_AUTO, workspace=None, err_flag=None, events=None, stream=None,
                 bf16_partials=False):
    """Paged attention of several new query tokens per sequence (causal within
    them); q, out [T, H, D] bf16, query_start_loc int32 [S+1]."""
    lib = _load()
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            need = decode_multi_workspace_size(q, max_query_len, key_cache, block_tables,
                                               partition_tokens, variant, bf16_partials)
            if need:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = _opts(k_scale, v_scale, partition_tokens, variant, workspace, err_flag, events,
              bf16_partials)
    d_q, d_qsl = describe(q), describe(query_start_loc)
    args = [describe(x) for x in (key_cache, value_cache, block_tables, seq_lens)]
    _check("pa_decode_multi",
           lib.pa_decode_multi(ctypes.byref(d_q), ctypes.byref(d_qsl), int(max_query_len),
                               *[ctypes.byref(x) for x in args], float(scale),
                               ctypes.byref(describe(out)), ctypes.byref(o), ts.cuda_stream))
    return out


class Regions:
    """A set of caches with one block geometry, as the block operations see
    it: ``bases`` is an int64 tensor of the caches' block-0 addresses (on the
    device, or in pinned host memory), ``block_stride`` and ``block_bytes`` in
    bytes, ``num_blocks`` blocks per cache.  Keeps the caches alive."""

    def __init__(self, bases, block_stride, block_bytes, num_blocks, caches=()):
        self.bases = bases
        self.block_stride = int(block_stride)
        self.block_bytes = int(block_bytes)
        self.num_blocks = int(num_blocks)
        self.caches = tuple(caches)


def region_table(caches, device=None, pin=False) -> Regions:
    """Regions of cache tensors [NB, ...] that share a shape and dtype (block b
    = index b of dim 0, contiguous).  The address table goes to ``device``
    (default: the caches' device) or, with ``pin=True``, to pinned host
    memory."""
    caches = list(caches)
    if not caches:
        raise ValueError("no caches")
    c0 = caches[0]
    for c in caches:
        if c.shape != c0.shape or c.dtype != c0.dtype or not c.is_contiguous():
            raise ValueError("caches must be contiguous and share shape and dtype")
    stride = c0[0].numel() * c0.element_size()
    addrs = torch.tensor([c.data_ptr() for c in caches], dtype=torch.int64)
    if pin:
        bases = addrs.pin_memory()
    else:
        bases = addrs.to(device if device is not None else c0.device)
    return Regions(bases, stride, stride, c0.shape[0], caches)


def _dev_ptr(t: torch.Tensor, what: str) -> int:
    if t.numel() == 0:
        return 0                        # nothing is read; the library takes no pointer
    if not (t.is_cuda or t.is_pinned()):
        raise TypeError(f"{what} must be device memory or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def zero_blocks(block_ids: torch.Tensor, regions: Regions, err_flag=None, stream=None):
    """Clear blocks ``block_ids`` (int32, device or pinned host) in every region."""
    if block_ids.dtype != torch.int32:
        raise TypeError("block_ids must be int32")
    lib = _load()
    o = _opts(err_flag=err_flag)
    _check("pa_zero_blocks",
           lib.pa_zero_blocks(_dev_ptr(block_ids, "block_ids"), block_ids.numel(),
                              _dev_ptr(regions.bases, "region bases"), regions.bases.numel(),
                              regions.block_stride, regions.block_bytes, regions.num_blocks,
                              ctypes.byref(o), _stream(stream)))


def copy_blocks(block_pairs: torch.Tensor, src: Regions, dst: Regions, err_flag=None,
                stream=None):
    """Copy block pairs[i, 0] of ``src`` over block pairs[i, 1] of ``dst``, in
    every region (``src`` and ``dst`` share the geometry)."""
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise TypeError("block_pairs must be int32 [n, 2]")
    if (src.block_stride, src.block_bytes) != (dst.block_stride, dst.block_bytes) or \
            src.bases.numel() != dst.bases.numel():
        raise ValueError("src and dst regions differ in geometry")
    lib = _load()
    o = _opts(err_flag=err_flag)
    _check("pa_copy_blocks",
           lib.pa_copy_blocks(_dev_ptr(block_pairs, "block_pairs"), block_pairs.shape[0],
                              _dev_ptr(src.bases, "src bases"), _dev_ptr(dst.bases, "dst bases"),
                              dst.bases.numel(), dst.block_stride, dst.block_bytes,
                              src.num_blocks, dst.num_blocks, ctypes.byref(o), _stream(stream)))


def prepare_step(idx_mapping, num_scheduled, num_computed, block_table, token_ids, block_size,
                 num_blocks, max_tokens, err_flag=None, stream=None):
    """One step's inputs from the per-request state table (all int32 device
    tensors: idx_mapping [S], num_scheduled [S], num_computed [R],
    block_table [R, max_blocks], token_ids [R, max_len]).  Returns a dict of
    device tensors: query_start_loc [S+1], seq_lens [S], positions int64
    [max_tokens], input_ids [max_tokens], slot_mapping int64 [max_tokens],
    block_tables [S, max_blocks]."""
    for name, t in (("idx_mapping", idx_mapping), ("num_scheduled", num_scheduled),
                    ("num_computed", num_computed), ("block_table", block_table),
                    ("token_ids", token_ids)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int32 tensor")
    S = idx_mapping.numel()
    if num_scheduled.numel() != S or block_table.dim() != 2 or token_ids.dim() != 2 or \
            block_table.shape[0] != num_computed.numel() or token_ids.shape[0] != num_computed.numel():
        raise ValueError("inconsistent state shapes")
    dev = idx_mapping.device
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        out = dict(query_start_loc=torch.empty(S + 1, dtype=torch.int32, device=dev),
                   seq_lens=torch.empty(S, dtype=torch.int32, device=dev),
                   positions=torch.empty(max_tokens, dtype=torch.int64, device=dev),
                   input_ids=torch.empty(max_tokens, dtype=torch.int32, device=dev),
                   slot_mapping=torch.empty(max_tokens, dtype=torch.int64, device=dev),
                   block_tables=torch.empty((S, block_table.shape[1]), dtype=torch.int32,
                                            device=dev))
    st = PaStepState(num_computed.data_ptr(), block_table.data_ptr(), token_ids.data_ptr(),
                     num_computed.numel(), block_table.shape[1], token_ids.shape[1])
    io = PaStepInputs(out["query_start_loc"].data_ptr(), out["seq_lens"].data_ptr(),
                      out["positions"].data_ptr(), out["input_ids"].data_ptr(),
                      out["slot_mapping"].data_ptr(), out["block_tables"].data_ptr(),
                      int(max_tokens))
    o = _opts(err_flag=err_flag)
    _check("pa_prepare_step",
           _load().pa_prepare_step(idx_mapping.data_ptr(), num_scheduled.data_ptr(), S,
                                   ctypes.byref(st), int(block_size), int(num_blocks),
                                   ctypes.byref(io), ctypes.byref(o), ts.cuda_stream))
    return out
