"""Benchmark of one paged decode step on one MI355X.

A step is the whole hot path for one batch: pa_kv_append of each sequence's
new K/V row into its slot, then pa_decode (block-table walk, gather, QK,
online softmax, PV, split-KV merge).  Inputs are generated on the GPU and are
resident in HBM before timing starts.  W untimed warm-up steps, then exactly
K timed steps between device synchronisations.  Before every step a kernel
reads and writes a 1 GiB scratch buffer, so no cache (the 4 MB L2 of each
XCD, the 256 MB Infinity Cache) still holds the batch from the step before;
HIP events bracket each step (the flush is outside them); on every second
step the library records a second pair around its attention kernel, and the
step times come from the other steps, which have no event records inside.
``--warm`` runs the steps back to back instead, with no flush.

Prints one JSON line.  ``value`` is the step's algorithmic HBM bytes divided
by the median step time, in GB/s; the roofline fraction comes from the
attention kernel's median time.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak, 8 TB/s
FLUSH_BYTES = 1 << 30      # scratch read and written before every timed step
METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + decode seqs/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "valu": ["paged_kv_cache_54_amd/csrc/decode_valu.hip", "paged_kv_cache_54_amd/csrc/pa_device.h"],
    "mfma": ["paged_kv_cache_54_amd/csrc/decode_mfma.hip",
             "paged_kv_cache_54_amd/csrc/decode_mfma_wave.h",
             "paged_kv_cache_54_amd/csrc/mfma_common.h", "paged_kv_cache_54_amd/csrc/pa_device.h",
             "paged_kv_cache_54_amd/csrc/decode_mfma_kernel.h",
             "paged_kv_cache_54_amd/csrc/decode_mfma_append.hip"],
    "mfma_multi": ["paged_kv_cache_54_amd/csrc/decode_mfma_multi.hip",
                   "paged_kv_cache_54_amd/csrc/mfma_common.h",
                   "paged_kv_cache_54_amd/csrc/pa_device.h"],
}
KERNEL_SOURCES["blocks"] = ["paged_kv_cache_54_amd/csrc/blocks.hip",
                            "paged_kv_cache_54_amd/csrc/pa_device.h"]
KERNEL_SOURCES["cascade"] = KERNEL_SOURCES["mfma"][1:4] + ["paged_kv_cache_54_amd/csrc/cascade.hip"]
KERNEL_SOURCES["mfma_heads"] = ["paged_kv_cache_54_amd/csrc/decode_mfma_heads.hip",
                                "paged_kv_cache_54_amd/csrc/decode_mfma_heads_kernel.h",
                                "paged_kv_cache_54_amd/csrc/decode_mfma_heads_append.hip"] + \
    KERNEL_SOURCES["mfma"][1:4]
KERNEL_NAMES = {"valu": "decode_valu_kernel", "mfma": "decode_mfma_kernel",
                "mfma_multi": "decode_mfma_multi_kernel",
                "cascade": "cascade_kernel", "mfma_heads": "decode_mfma_heads_kernel"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_bf16")
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--no-cascade", action="store_true",
                    help="for a batch with a shared prefix, use plain pa_decode instead of "
                         "pa_decode_cascade")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--warm", action="store_true",
                    help="run the timed steps back to back with no cache flush between them")
    ap.add_argument("--separate-append", action="store_true",
                    help="one-query steps: pa_kv_append then pa_decode (two launches) "
                         "instead of pa_decode_append")
    ap.add_argument("--bf16-partials", action="store_true",
                    help="store split-KV partial accumulators as bf16 instead of fp32")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB "
                         "(3 launches) so hardware byte counters can be scaled against a known size")
    return ap.parse_args()


def cdiv(a, b):
    return -(-a // b)


def quantiles(ms):
    """Median, p10 and p90 of a list of times in ms."""
    import numpy as np
    p10, med, p90 = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return {"median": round(float(med), 5), "p10": round(float(p10), 5),
            "p90": round(float(p90), 5)}


def algorithmic_bytes(b):
    """Bytes a step must move at least once: decode reads each sequence's L
    K and V rows of every KV head (a shared physical block counted once),
    q, the block-table entries it walks and seq_lens, and writes out; append
    reads the new rows and slot_mapping and writes them into the cache."""
    import numpy as np
    lens = b.seq_lens.cpu().numpy().astype(np.int64)
    tables = b.block_tables.cpu().numpy()
    bs, Hkv, D = b.block_size, b.num_kv_heads, b.head_dim
    kv_tok = Hkv * D * b.kv_elem_bytes * 2                  # K and V of one token
    logical_tokens = int(lens.sum())
    # unique (block, offset) slots read
    seen = {}
    for s in range(b.num_seqs):
        nb = cdiv(int(lens[s]), bs)
        for j in range(nb):
            n = min(bs, int(lens[s]) - j * bs)
            blk = int(tables[s, j])
            seen[blk] = max(seen.get(blk, 0), n)
    unique_tokens = sum(seen.values())
    T = b.q.shape[0]                                        # query tokens (S, or more)
    qo = 2 * T * b.num_heads * D * b.q_elem_bytes
    meta = 4 * int(sum(cdiv(int(x), bs) for x in lens)) + 4 * b.num_seqs
    if b.query_start_loc is not None:
        meta += 4 * (b.num_seqs + 1)
    decode = unique_tokens * kv_tok + qo + meta
    in_elt = 4 if b.cache_dtype == "f32" else 2
    append = T * Hkv * D * 2 * (in_elt + b.kv_elem_bytes) + 8 * T
    return dict(decode=decode, append=append, step=decode + append,
                logical_decode=logical_tokens * kv_tok + qo + meta,
                unique_tokens=unique_tokens, logical_tokens=logical_tokens)


def source_sha(variant):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[variant]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def traffic_for(variant, workload, kernel=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel source as it stands now; else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(f"{kernel or KERNEL_NAMES[variant]}:{workload}")
    if not rec or rec.get("source_sha256") != source_sha(variant):
        return None
    return rec.get("traffic_bytes_per_launch")


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self, n):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def record(self, k, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(self.ev[k]), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def close(self):
        for e in self.ev:
            self.lib.hipEventDestroy(e)


def cpu_model():
    """The host CPU's model name and the number of CPUs this process may use."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return name, len(os.sched_getaffinity(0))


def cpu_baseline(b, budget_s):
    """The oracle, as it stands, on the host cores: one call over the whole
    batch (every query row; OpenMP over rows), the median of 3 runs -- fewer
    when one run already takes more than budget_s -- after the host caches are
    filled (not timed).  Reported in the step's unit: algorithmic GB/s of the
    decode, plus seconds per batch and decode sequences per second."""
    import statistics

    import oracle
    NB, bs, Hkv, D = b.num_blocks, b.block_size, b.num_kv_heads, b.head_dim
    kc, vc = oracle.fill_cache(b, b.key_pool.cpu().view(NB * bs, Hkv, D),
                               b.value_pool.cpu().view(NB * bs, Hkv, D))
    oracle.kv_append(b.k_new.cpu(), b.v_new.cpu(), b.slot_mapping.cpu(), kc, vc, b.k_scale,
                     b.v_scale)
    q, tables, lens = b.q.cpu(), b.block_tables.cpu(), b.seq_lens.cpu()
    rows = q.shape[0] * b.num_heads
    times = []
    while len(times) < 3 and (not times or sum(times) < budget_s):
        t0 = time.perf_counter()
        if b.query_start_loc is None:
            oracle.decode(q, kc, vc, tables, lens, b.scale, b.k_scale, b.v_scale)
        else:
            oracle.decode_multi(q, b.query_start_loc.cpu(), kc, vc, tables, lens, b.scale,
                                b.k_scale, b.v_scale)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    nbytes = algorithmic_bytes(b)["decode"]
    threads = min(oracle.num_threads(), rows)
    model, ncpu = cpu_model()
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_batch": round(t, 3),
            "decode_seqs_per_s": round(b.num_seqs / t, 2),
            "sample": f"the whole batch ({rows} query rows) in one call, median of "
                      f"{len(times)} run(s): {t:.2f} s; fp64 C oracle, OpenMP over query rows on "
                      f"{threads} threads; host {model}, {ncpu} CPUs available"}


def block_cpu_baseline(case, budget_s):
    """The block oracle, as it stands, on a bounded sample: whole calls over a
    prefix of the regions, repeated until about budget_s seconds; GB/s of the
    bytes the GPU kernel moves for the same work."""
    import oracle.blocks as ob
    R = min(len(case.regions), 4)
    regs = [r.cpu().numpy().reshape(-1) for r in case.regions[:R]]
    items = case.items.numpy()
    per_region = len(items) * case.block_bytes * (1 if case.op == "zero" else 2)
    done, t_total = 0, 0.0
    while t_total < budget_s and done < 1000:
        t0 = time.perf_counter()
        if case.op == "zero":
            ob.zero_blocks(regs, items, case.block_bytes, case.block_bytes, case.num_blocks)
        else:
            ob.copy_blocks(regs, regs, items, case.block_bytes, case.block_bytes,
                           case.num_blocks, case.num_blocks)
        t_total += time.perf_counter() - t0
        done += 1
    return {"value": round(done * R * per_region / t_total / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} whole calls over {R} of the {len(case.regions)} regions in "
                      f"{t_total:.1f} s; numpy slicing, one thread"}


def bench_blocks(args):
    """One launch of pa_zero_blocks / pa_copy_blocks per step over the block
    workload; value = bytes the op must move (written, plus read for a copy)
    per second of wall time."""
    import torch

    import paged_kv_cache_54_amd as pa
    import workloads

    dev = "cuda:0"
    case = workloads.make_block_case(args.workload, device=dev)
    regs = pa.region_table(case.regions)
    items = case.items.to(dev)
    lib = pa._load()
    stream = torch.cuda.current_stream().cuda_stream
    n = case.items.shape[0]
    R = len(case.regions)
    nbytes = n * R * case.block_bytes * (1 if case.op == "zero" else 2)
    ev = HipEvents(2 * args.steps)
    o = pa._opts()
    by = ctypes.byref

    def step(k=None):
        if k is not None:
            ev.record(2 * k, stream)
        if case.op == "zero":
            rc = lib.pa_zero_blocks(items.data_ptr(), n, regs.bases.data_ptr(), R,
                                    regs.block_stride, regs.block_bytes, regs.num_blocks, by(o),
                                    stream)
        else:
            rc = lib.pa_copy_blocks(items.data_ptr(), n, regs.bases.data_ptr(),
                                    regs.bases.data_ptr(), R, regs.block_stride,
                                    regs.block_bytes, regs.num_blocks, regs.num_blocks, by(o),
                                    stream)
        if rc:
            raise pa.PaError("block op", rc)
        if k is not None:
            ev.record(2 * k + 1, stream)

    flush = None if args.warm else torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        if flush is not None:
            flush.add_(1)
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.add_(1)                      # read + write 1 GiB, outside the events
        step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_q = quantiles([ev.elapsed_ms(2 * k, 2 * k + 1) for k in range(args.steps)])
    ev.close()
    kernel_ms = ms = kern_q["median"]          # a step is the one launch
    value = nbytes / (ms * 1e-3) / 1e9
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    # the library's choice: one workgroup per 4 KiB piece for operations of
    # 128 MiB and more (tables here are in device memory), else grouped
    kind = "block_piece_kernel" if n * R * case.block_bytes >= (128 << 20) else "block_op_kernel"
    kname = f"{kind}<{'true' if case.op == 'copy' else 'false'}>"
    traffic = traffic_for("blocks", args.workload, kernel=kname)
    res = {
        "metric": f"block {'clear' if case.op == 'zero' else 'copy'}: achieved HBM GB/s "
                  f"({'bytes written' if case.op == 'zero' else 'bytes read + written'})",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": args.workload, "op": case.op, "items": n, "regions": R,
                   "block_bytes": case.block_bytes, "num_blocks": case.num_blocks},
        "timing": {"protocol": "back to back, no flush" if args.warm else
                   "1 GiB read+write flush before each step, outside the events",
                   "kernel_ms": kern_q, "wall_ms_per_step": round(wall / args.steps * 1e3, 5)},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel_ms": round(kernel_ms, 5),
                     "kernel_ms_from": f"median of HIP events around each of the {args.steps} "
                                       f"launches" + ("" if args.warm else
                                                      ", caches flushed before each"),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    res["cpu_baseline"] = None if args.no_cpu_baseline else block_cpu_baseline(
        case, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


def bench_prep(args):
    """One pa_prepare_step launch per step over a step-metadata workload;
    value = microseconds per call (the work is a few hundred KB: latency)."""
    import torch

    import paged_kv_cache_54_amd as pa
    import workloads

    c = workloads.make_prep_case(args.workload, device="cuda:0")
    S, R = c["idx_mapping"].numel(), c["num_computed"].numel()
    max_nb, max_len = c["block_table"].shape[1], c["token_ids"].shape[1]
    T = int(c["num_scheduled"].sum())
    mt = c["max_tokens"]
    nbytes = (12 * S + 4 * S * max_nb) + 8 * T + (8 * S + 4 + 20 * mt + 4 * S * max_nb)
    ev = HipEvents(2 * args.steps)
    stream = torch.cuda.current_stream().cuda_stream
    outs = pa.prepare_step(c["idx_mapping"], c["num_scheduled"], c["num_computed"],
                           c["block_table"], c["token_ids"], c["block_size"], c["num_blocks"], mt)
    st = pa.PaStepState(c["num_computed"].data_ptr(), c["block_table"].data_ptr(),
                        c["token_ids"].data_ptr(), R, max_nb, max_len)
    io = pa.PaStepInputs(*[outs[k].data_ptr() for k in ("query_start_loc", "seq_lens",
                                                          "positions", "input_ids",
                                                          "slot_mapping", "block_tables")], mt)
    lib = pa._load()
    o = pa._opts()
    by = ctypes.byref

    def step(k=None):
        if k is not None:
            ev.record(2 * k, stream)
        rc = lib.pa_prepare_step(c["idx_mapping"].data_ptr(), c["num_scheduled"].data_ptr(), S,
                                 by(st), c["block_size"], c["num_blocks"], by(io), by(o), stream)
        if rc:
            raise pa.PaError("pa_prepare_step", rc)
        if k is not None:
            ev.record(2 * k + 1, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sum(ev.elapsed_ms(2 * k, 2 * k + 1) for k in range(args.steps)) / args.steps
    ev.close()
    ms = wall / args.steps * 1e3
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    res = {
        "metric": "step metadata prep: microseconds per call", "value": round(ms * 1e3, 3),
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": args.workload, "reqs": S, "state_rows": R, "new_tokens": T,
                   "max_tokens": mt, "max_blocks": max_nb},
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "step_prep_kernel", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 6), "traffic": None,
                     "kernel_ms": round(kernel_ms, 5),
                     "kernel_ms_from": f"HIP events around each of the {args.steps} launches",
                     "algorithmic_bytes_per_launch": nbytes,
                     "note": "a few hundred KB per call: bound by launch latency, not HBM"},
    }
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
    else:
        import oracle.step_prep as osp
        h = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in c.items()}
        done, t_cpu = 0, 0.0
        while t_cpu < args.cpu_budget_s and done < 200:
            t1 = time.perf_counter()
            osp.prepare_step(h["idx_mapping"], h["num_scheduled"], h["num_computed"],
                             h["block_table"], h["token_ids"], h["block_size"], mt,
                             h["num_blocks"])
            t_cpu += time.perf_counter() - t1
            done += 1
        res["cpu_baseline"] = {"value": round(t_cpu / done * 1e6, 1), "unit": "us", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{done} whole calls in {t_cpu:.1f} s; python loops"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_54_amd as pa
    import workloads
    from paged_kv_cache_54_amd import PaOpts, describe

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))
        return
    if args.workload in workloads.BLOCK_CONFIGS:
        bench_blocks(args)
        return
    if args.workload in workloads.PREP_CONFIGS:
        bench_prep(args)
        return
    b = workloads.make_batch(args.workload, device=dev)
    P = args.partition_tokens if args.partition_tokens is not None else (b.partition_tokens or 0)
    variant = {"auto": pa.VARIANT_AUTO, "valu": pa.VARIANT_VALU, "mfma": pa.VARIANT_MFMA}[args.variant]

    # caches resident in HBM (an fp8 cache is quantised by the library's append)
    if b.cache_dtype == "fp8_e4m3":
        kc = torch.zeros(b.key_pool.shape, dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        NB, bs, Hkv, D = b.key_pool.shape
        pa.kv_append(b.key_pool.view(NB * bs, Hkv, D), b.value_pool.view(NB * bs, Hkv, D),
                     b.pool_slots(), kc, vc, b.k_scale, b.v_scale)
    else:
        kc, vc = b.key_pool.clone(), b.value_pool.clone()
    out = torch.empty_like(b.q)
    multi = b.query_start_loc is not None
    cascade = (b.shared_prefix_blocks > 0 and not args.no_cascade and b.q_dtype == "bf16"
               and variant != pa.VARIANT_VALU)
    bf16p = args.bf16_partials
    if cascade:
        ws_bytes = pa.decode_cascade_workspace_size(b.q, kc, b.block_tables,
                                                    b.shared_prefix_blocks, P, variant, bf16p)
    elif multi:
        ws_bytes = pa.decode_multi_workspace_size(b.q, b.max_query_len, kc, b.block_tables, P,
                                                  variant, bf16p)
    else:
        ws_bytes = pa.decode_workspace_size(b.q, kc, b.block_tables, P, variant, bf16p)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    # One-query steps call pa_decode_append: the append is done by the decode
    # kernel (matrix-core variants) and its bytes are then that kernel's too.
    fused = not (cascade or multi or args.separate_append)

    # descriptors built once; each step is one or two C calls
    lib = pa._load()
    d_k, d_v, d_slot = describe(b.k_new), describe(b.v_new), describe(b.slot_mapping)
    d_q, d_kc, d_vc = describe(b.q), describe(kc), describe(vc)
    d_bt, d_len, d_out = describe(b.block_tables), describe(b.seq_lens), describe(out)
    d_qsl = describe(b.query_start_loc) if multi else None
    o = PaOpts()
    lib.pa_opts_init(ctypes.byref(o))
    o.k_scale, o.v_scale = b.k_scale, b.v_scale
    o.partition_tokens, o.variant = P, variant
    o.workspace, o.workspace_bytes = ws.data_ptr(), ws.numel()
    o.partials = pa.PARTIALS_BF16 if bf16p else pa.PARTIALS_F32
    stream = torch.cuda.current_stream().cuda_stream
    # per timed step: step start, kernel start, kernel end, step end
    ev = HipEvents(4 * args.steps)
    flush = None if args.warm else torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    by = ctypes.byref

    # Even timed steps also record the attention kernel's events (the kernel's
    # median comes from them); odd steps run without those two records inside
    # the step (the step's median comes from them).
    def step(i=None):
        if i is None or i % 2:
            o.kernel_events[0] = o.kernel_events[1] = None
        else:
            o.kernel_events[0], o.kernel_events[1] = ev.ev[4 * i + 1], ev.ev[4 * i + 2]
        if i is not None:
            ev.record(4 * i, stream)
        if fused:
            rc = lib.pa_decode_append(by(d_k), by(d_v), by(d_slot), by(d_q), by(d_kc), by(d_vc),
                                      by(d_bt), by(d_len), ctypes.c_float(b.scale), by(d_out),
                                      by(o), stream)
            if rc:
                raise pa.PaError("step", rc)
            if i is not None:
                ev.record(4 * i + 3, stream)
            return
        rc = lib.pa_kv_append(by(d_k), by(d_v), by(d_slot), by(d_kc), by(d_vc), by(o), stream)
        if cascade:
            rc = rc or lib.pa_decode_cascade(by(d_q), by(d_kc), by(d_vc), by(d_bt), by(d_len),
                                             b.shared_prefix_blocks, ctypes.c_float(b.scale),
                                             by(d_out), by(o), stream)
        elif multi:
            rc = rc or lib.pa_decode_multi(by(d_q), by(d_qsl), b.max_query_len, by(d_kc),
                                           by(d_vc), by(d_bt), by(d_len), ctypes.c_float(b.scale),
                                           by(d_out), by(o), stream)
        else:
            rc = rc or lib.pa_decode(by(d_q), by(d_kc), by(d_vc), by(d_bt), by(d_len),
                                     ctypes.c_float(b.scale), by(d_out), by(o), stream)
        if rc:
            raise pa.PaError("step", rc)
        if i is not None:
            ev.record(4 * i + 3, stream)

    for _ in range(args.warmup):
        if flush is not None:
            flush.add_(1)
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.add_(1)                      # read + write 1 GiB, outside the events
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_t = [ev.elapsed_ms(4 * i, 4 * i + 3) for i in range(1, args.steps, 2)] or \
        [ev.elapsed_ms(0, 3)]
    kern_t = [ev.elapsed_ms(4 * i + 1, 4 * i + 2) for i in range(0, args.steps, 2)]
    ev.close()
    step_q, kern_q = quantiles(step_t), quantiles(kern_t)
    kernel_ms = kern_q["median"]

    nbytes = algorithmic_bytes(b)
    ms_per_step = step_q["median"]
    value = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    used = "mfma_multi" if multi else "mfma" if (variant == pa.VARIANT_MFMA or (
        variant == pa.VARIANT_AUTO and _mfma_ok(pa, b, kc))) else "valu"
    if cascade:
        used = "cascade"
    if used == "mfma" and not multi and _heads_kernel(b):
        used = "mfma_heads"
    # The library fuses the append into the matrix-core one-query kernels
    # when the batch has at most two (sequence, KV head) segments per
    # wavefront; the wavefronts follow from the workspace size, whose slots
    # are wavefronts + segments.
    in_kernel = (fused and used in ("mfma", "mfma_heads") and b.k_new.shape[0] == b.num_seqs
                 and b.num_seqs * b.num_kv_heads <= 2 * _waves(b, ws_bytes, bf16p))
    kernel_bytes = nbytes["decode"] + (nbytes["append"] if in_kernel else 0)
    achieved = kernel_bytes / (kernel_ms * 1e-3) / 1e9
    kname = KERNEL_NAMES[used]
    cols = b.group_size * b.max_query_len if multi else 0
    if cols > 32 or (cols > 16 and b.cache_dtype != "bf16"):
        kname = "decode_mfma_multi_coop_kernel"     # two wavefronts per chunk
    traffic = traffic_for(used, args.workload, kname)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3"}[b.cache_dtype],
        "timing": {"protocol": "back to back, no flush" if args.warm else
                   "1 GiB read+write flush before each step, outside the events",
                   "step_ms_from": f"median of HIP events around the {len(step_t)} odd-numbered "
                                   f"timed steps (no event records inside them)",
                   "step_ms": step_q, "kernel_ms": kern_q,
                   "wall_ms_per_step": round(wall / args.steps * 1e3, 5)},
        "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": b.num_seqs, "num_heads": b.num_heads,
                   "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "block_size": b.block_size, "num_blocks": b.num_blocks,
                   "mean_seq_len": round(nbytes["logical_tokens"] / b.num_seqs, 1),
                   "q_dtype": b.q_dtype, "cache_dtype": b.cache_dtype,
                   "partition_tokens": P or "auto", "variant": used,
                   "partials": "bf16" if bf16p and b.q_dtype == "bf16" else "f32",
                   "append": "in the decode kernel" if in_kernel else
                             ("pa_decode_append, own launch" if fused else "pa_kv_append"),
                   **({"shared_prefix_blocks": b.shared_prefix_blocks} if cascade else {}),
                   **({"query_tokens": b.q.shape[0], "max_query_len": b.max_query_len}
                      if multi else {})},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_seqs_per_s": round(b.num_seqs / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": nbytes["step"],
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel_ms": round(kernel_ms, 5),
                     "kernel_ms_from": f"median of HIP events around the attention kernel on "
                                       f"the {len(kern_t)} even-numbered of the {args.steps} timed "
                                       f"steps" + ("" if args.warm else
                                                   ", caches flushed before each step"),
                     "algorithmic_bytes_per_launch": kernel_bytes},
    }
    if nbytes["logical_decode"] != nbytes["decode"]:
        res["logical_decode_bytes"] = nbytes["logical_decode"]
        res["effective_logical_gbs"] = round(nbytes["logical_decode"] / (kernel_ms * 1e-3) / 1e9, 2)
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(b, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


def _waves(b, ws_bytes, bf16p):
    """Wavefronts of a one-query decode plan, from its workspace bytes:
    acc [slots, G, D] (2 or 4 bytes) | ml [slots, G, 2] f32 | seg [S*Hkv, 2] i32,
    slots = wavefronts + S*Hkv."""
    G = b.num_heads // b.num_kv_heads
    segs = b.num_seqs * b.num_kv_heads
    per_slot = G * b.head_dim * (2 if bf16p and b.q_dtype == "bf16" else 4) + 8 * G
    return (ws_bytes - 8 * segs) // per_slot - segs


def _heads_kernel(b):
    """Whether the library runs this one-query batch on its per-block e4m3
    kernel (workgroups of one wavefront per KV head)."""
    G = b.num_heads // b.num_kv_heads
    return (b.cache_dtype == "fp8_e4m3" and b.head_dim == 128 and b.block_size in (16, 32)
            and b.num_kv_heads in (4, 8) and G in (1, 2, 4, 8))


def _mfma_ok(pa, b, kc):
    try:
        pa.decode_workspace_size(b.q, kc, b.block_tables, 0, pa.VARIANT_MFMA)
        return True
    except pa.PaError:
        return False


if __name__ == "__main__":
    main()
