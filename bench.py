#!/usr/bin/env python3
"""Benchmark of the per-layer n-gram embedding (PLE) hot path on one MI355X.

Default workload: 8192-token prefill over ragged requests (geometric lengths,
mean 512, clipped to [1, 4096]) with Zipf(1.1) token ids, 8 hash heads (orders
2 and 3) over an 8.39M-row x 512 bf16 table in HBM, hidden 4096, kv_proj
4096 -> 2x4096, gate, and conv (kernel 4, dilation 3).  One step is one pass of
the whole path for one layer: fused ids+gather, kv_proj, gate, conv.  Steps
rotate over 16 layers' hash multipliers (and 4 kv weights) so consecutive
lookups touch different rows (about 1 GB of distinct rows per 16 steps, more
than the 256 MB last-level cache).

Prints one JSON line (rank 0): tokens/s of the whole path, per-stage times
from HIP events on the launch stream, the dominant kernel's roofline, the
fused lookup's gathered GB/s, and the single-threaded CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s + gathered GB/s (% HBM peak), fused PLE lookup, 8k-token prefill"
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: past the chip's power-controller transient (after setup the clock "
                         "boosts, then throttles below its steady value for about the first 50 prefill steps) and "
                         "more than one rotation of the layers, so clocks and caches are settled")
    ap.add_argument("--layers", type=int, default=16, help="hash layers rotated over the steps")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--prefetch-cus", type=int, default=32, help="CUs of the host-table prefetch stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="prefill-8k-bf16-hbm",
                    choices=["prefill-8k-bf16-hbm", "prefill-16k-fp8-hbm", "prefill-16k-fp8global-hbm",
                             "prefill-8k-nvfp4-hbm", "prefill-8k-bf16-host", "select-rows-8k",
                             "spec-decode-256x4", "decode-256"],
                    help="the default is the benchmark line; the others report the fp8-table (per-row or "
                         "one global scale), NVFP4-table and host-resident-table variants, the row select of a "
                         "sharded table, and the decode and speculative-decode steps of the decode-shaped model")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import layer_embedding_lookup_amd as ple
    import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload == "prefill-8k-bf16-host":
        return bench_host_table(args)
    if args.workload == "select-rows-8k":
        return bench_select_rows(args)
    if args.workload == "spec-decode-256x4":
        return bench_spec_decode(args)
    if args.workload == "decode-256":
        return bench_decode(args)
    # table format of the workload; the batch, projection and conv are those of
    # the 8k prefill (bf16, NVFP4) or the 16k prefill (fp8 tables)
    fmt = {"prefill-8k-bf16-hbm": "bf16", "prefill-16k-fp8-hbm": "fp8", "prefill-16k-fp8global-hbm": "fp8-global",
           "prefill-8k-nvfp4-hbm": "nvfp4"}[args.workload]
    cfg = wl.CONFIGS[3] if fmt in ("bf16", "nvfp4") else wl.CONFIGS[4]
    L = args.layers
    log(f"workload {args.workload}: T={cfg.T} H={cfg.H} rows={cfg.num_rows} D={cfg.D} N={cfg.N}")
    b = wl.make_batch(cfg, layers=L)
    log("generating the table on the host")
    t0 = time.time()
    if fmt == "nvfp4":
        codes_h, bs_h, tscale = wl.make_nvfp4_table(cfg.num_rows, cfg.D, cfg.seed)
        table_h, scales_h = codes_h, (bs_h, tscale)
    else:
        table_h, scales_h = wl.make_table(cfg)
        if fmt == "fp8-global":
            # the same codes with one scale for the table: the largest per-row scale
            scales_h = np.asarray([scales_h.max()], dtype=np.float32)
    log(f"table ready in {time.time() - t0:.1f}s; copying to HBM")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def it(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if fmt == "bf16":
        table = bf(table_h)
        tb = ple.Table.from_tensor(table)
    elif fmt == "nvfp4":
        table = it(table_h)
        tb = ple.Table.nvfp4(table, it(scales_h[0]), it(np.asarray([scales_h[1]], dtype=np.float32)))
    else:
        table, scales = it(table_h), it(scales_h)
        tb = ple.Table.from_tensor(table, scales)
    kv_ws_h = [wl.make_kv_weight(cfg, layer=i) for i in range(4)]
    kv_ws = [bf(w) for w in kv_ws_h]
    conv_w_h = wl.make_conv_weight(cfg)
    conv_w = bf(conv_w_h)
    hidden_h = wl.make_hidden(cfg)
    hidden = bf(hidden_h)
    toks, qsl = it(b.input_ids), it(b.qsl)
    hashes = [ple.HashParams(b.multipliers[l], b.vocab_sizes, b.offsets, heads_per_ngram=cfg.heads_per_ngram,
                             context_len=cfg.context_len, eos_token_id=wl.EOS) for l in range(L)]
    layers = [ple.Layer(hashes[l], tb, kv_ws[l % 4], conv_w, conv_dilation=cfg.conv_dilation, eps=cfg.eps)
              for l in range(L)]
    T, H, D, N = cfg.T, cfg.H, cfg.D, cfg.N
    rows = torch.empty((T, H * D), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty_like(rows) for _ in range(8)]
    kv = torch.empty((T, 2 * N), dtype=torch.bfloat16, device=dev)
    gated = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((ple.ple_prefill_workspace_bytes(layers[0], T),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def timed(fn, n):
        """Average duration of n back-to-back launches, HIP events on the launch stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def step(s):
        lay = layers[s % L]
        ple.ple_prefill_fused(lay, toks, qsl, hidden, out=out, workspace=ws)

    log(f"warmup {args.warmup} steps")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    K = args.steps
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(K):
        step(args.warmup + s)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / K

    # per-kernel durations: the same kernels, shapes and launch configurations
    # as inside the fused step, each launched back to back
    log("timing each kernel")
    reps = max(K, L)
    # Every timed kernel reads real data: rows from a lookup here, kv and gated
    # from the loops before theirs.  (The matrix cores run measurably faster on
    # zero operands: kv_proj on a zero-filled x takes ~10% less time.)
    ple.ple_lookup(hashes[0], tb, toks, qsl, rows=rows)
    stage_ms = {
        # the lookup writes into 8 rotating output buffers (512 MiB, twice the
        # last-level cache) so neither its row reads nor its row writes can
        # stay cached between launches
        "lookup": timed(lambda i: ple.ple_lookup(hashes[i % L], tb, toks, qsl, rows=outs[i % len(outs)]), 4 * L),
        "kv_proj": timed(lambda i: ple.ple_kv_proj(rows, kv_ws[i % 4], kv=kv), reps),
        "gate": timed(lambda i: ple.ple_gate(hidden, kv, eps=cfg.eps, out=gated, want_gate=False), reps),
        "conv": timed(lambda i: ple.ple_conv(gated, qsl, conv_w, dilation=cfg.conv_dilation, y=out), reps),
    }
    lookup_ms = stage_ms["lookup"]
    # reference point for kv_proj: the vendor GEMM (torch.matmul, which calls
    # hipBLASLt) on the same rows and weights, then ours again, so that the
    # chip's clock drift under sustained MFMA load shows in the pair
    torch.matmul(rows, kv_ws[0].t(), out=kv)  # first call loads the kernel
    vendor_kv_ms = timed(lambda i: torch.matmul(rows, kv_ws[i % 4].t(), out=kv), reps)
    kv_again_ms = timed(lambda i: ple.ple_kv_proj(rows, kv_ws[i % 4], kv=kv), reps)
    # the same launches into one output buffer, as inside the fused step (its
    # workspace rows are rewritten every layer)
    lookup_same_ms = timed(lambda i: ple.ple_lookup(hashes[i % L], tb, toks, qsl, rows=rows), 4 * L)
    # Reference points for the lookup, same bytes and buffers: the row output
    # written alone (torch fill, no reads), and, for a bf16 table, torch's own
    # embedding gather on the same IDs (an index_select into the same output).
    rows.fill_(1.0)  # first launch loads the kernel: keep it out of the timing
    write_only_ms = timed(lambda i: outs[i % len(outs)].fill_(1.0), 4 * L)
    torch_gather_ms = None
    if fmt == "bf16":
        ids_l = [ple.ple_ngram_ids(hashes[l], toks, qsl).view(-1).long() for l in range(L)]
        rows_flat = rows.view(T * H, D)
        torch.index_select(table, 0, ids_l[0], out=rows_flat)
        torch_gather_ms = timed(lambda i: torch.index_select(table, 0, ids_l[i % L],
                                                            out=outs[i % len(outs)].view(T * H, D)), 4 * L)
        del ids_l
    # Streaming-copy ceilings (libple_bench, hand-written 16-byte copies, one
    # pass per wave): the lookup's 64 MiB of output copied contiguously from
    # rotating 64 MiB windows of the table, and the same random rows the
    # lookup reads (this layer's IDs) gathered into the same rotating outputs
    blib = bench_library()
    out_bytes = T * H * D * 2
    row_bytes_in = {"bf16": D * 2, "fp8": D, "fp8-global": D, "nvfp4": D // 2}[fmt]
    n_windows = max(1, min(16, (cfg.num_rows * row_bytes_in) // out_bytes))

    def bench_copy(i):
        src = table.data_ptr() + (i % n_windows) * out_bytes
        check_bench(blib.ple_bench_copy(src, outs[i % len(outs)].data_ptr(), out_bytes,
                                        torch.cuda.current_stream().cuda_stream), blib)
    bench_copy(0)
    contig_ms = timed(bench_copy, 4 * L)
    contig_gbps = 2 * out_bytes / (contig_ms * 1e-3) / 1e9
    ids_rows = [ple.ple_ngram_ids(hashes[l], toks, qsl).view(-1) for l in range(L)]
    rows_of_table = table.numel() * table.element_size() // row_bytes_in

    # the random-row ceiling moves the lookup's own bytes: a bf16 table's rows
    # copied as they are; a quantized table's codes widened to the 1 KiB
    # output row, with its scale reads (per-row word, or NVFP4 block bytes)
    expand = {"bf16": 1, "fp8": 2, "fp8-global": 2, "nvfp4": 4}[fmt]
    aux_mode, aux_ptr = {"fp8": (1, tb.row_scales_ptr), "nvfp4": (2, tb.block_scales_ptr)}.get(fmt, (0, None))

    def bench_rows(i):
        ids_p, out_p = ids_rows[i % L].data_ptr(), outs[i % len(outs)].data_ptr()
        stream = torch.cuda.current_stream().cuda_stream
        if fmt == "bf16":
            check_bench(blib.ple_bench_copy_rows(table.data_ptr(), rows_of_table, row_bytes_in, ids_p, T * H, out_p,
                                                 stream), blib)
        else:
            check_bench(blib.ple_bench_gather_expand(table.data_ptr(), rows_of_table, expand, aux_ptr, aux_mode,
                                                     ids_p, T * H, D * 2, out_p, stream), blib)
    bench_rows(0)
    rows_ms = timed(bench_rows, 4 * L)
    rows_gbps = lookup_bytes_of(fmt, T, H, D, b.R) / (rows_ms * 1e-3) / 1e9
    # rows that repeat within a batch are served by the caches: the distinct
    # rows per layer, and the lookup's bytes counted with each row read once
    distinct = float(np.mean([torch.unique(ids_rows[l]).numel() for l in range(L)]))
    del ids_rows

    R = b.R
    lookup_bytes = lookup_bytes_of(fmt, T, H, D, R)
    lookup_gbps = lookup_bytes / (lookup_ms * 1e-3) / 1e9
    kv_flops = 2.0 * T * (H * D) * (2 * N)
    kv_tflops = kv_flops / (stage_ms["kv_proj"] * 1e-3) / 1e12
    gate_bytes = T * N * 2 * 4   # hidden + key + value read, gated value written
    conv_bytes = T * N * 2 * 2   # x read once, y written
    tokens_per_s = T / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, b, table_h, scales_h, kv_ws_h[0], conv_w_h, hidden_h, args.cpu_sample_tokens,
                           args.workload)

    line = {
        "metric": METRIC if args.workload == "prefill-8k-bf16-hbm"
        else METRIC.replace("8k-token prefill", f"{T // 1024}k-token prefill, {fmt} table"),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "requests": R, "heads": H, "orders": [2, 3],
                   "table_rows": cfg.num_rows, "dim": D, "table_dtype": fmt, "table_location": "hbm",
                   "hidden": N, "kv_proj": [H * D, 2 * N], "conv": [cfg.conv_kernel, cfg.conv_dilation],
                   "layers_rotated": L},
        "roofline": {"kernel": "kv_proj (MFMA bf16 GEMM)", "bound": "mfma",
                     "achieved": round(kv_tflops, 1), "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kv_tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(cfg.name), "traffic_unit": "bytes per launch",
                     "traffic_source": "profiles/kv_proj_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE passes "
                                       "scaled by a contiguous copy's, recorded with the kernel source's hash "
                                       "(null when the source has changed since)"},
        "lookup": {"kernel": "fused ids+gather" + ("" if fmt == "bf16" else f"+{fmt} dequant"),
                   "ms": round(lookup_ms, 5), "bytes": lookup_bytes,
                   "gathered_GBps": round(lookup_gbps, 1), "frac_hbm_peak": round(lookup_gbps / HBM_PEAK_GBPS, 4),
                   "frac_copy_ceiling": round(lookup_gbps / rows_gbps, 4),
                   "frac_contiguous_copy": round(lookup_gbps / contig_gbps, 4),
                   "tokens_per_s": round(T / (lookup_ms * 1e-3), 1),
                   "outputs_rotated": 8,
                   "same_output_ms": round(lookup_same_ms, 5),
                   "same_output_frac_hbm_peak": round(lookup_bytes / (lookup_same_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "write_only_ms": round(write_only_ms, 5),
                   "torch_index_select_ms": None if torch_gather_ms is None else round(torch_gather_ms, 5),
                   "distinct_rows": round(distinct, 1), "distinct_row_frac": round(distinct / (T * H), 4),
                   "distinct_bytes": int(lookup_bytes - (T * H - distinct) * row_in_bytes(fmt, D)),
                   "distinct_GBps": round((lookup_bytes - (T * H - distinct) * row_in_bytes(fmt, D))
                                          / (lookup_ms * 1e-3) / 1e9, 1)},
        "kv_proj": {"ms": round(stage_ms["kv_proj"], 5), "ms_after_vendor": round(kv_again_ms, 5),
                    "torch_matmul_ms": round(vendor_kv_ms, 5), "flops": kv_flops},
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stages_GBps": {"gate": round(gate_bytes / (stage_ms["gate"] * 1e-3) / 1e9, 1),
                        "conv": round(conv_bytes / (stage_ms["conv"] * 1e-3) / 1e9, 1)},
        "copy_ceiling": {"kernel": "hand-written 16-byte streaming copy (libple_bench), one pass per wave",
                         "random_rows_ms": round(rows_ms, 5), "random_rows_GBps": round(rows_gbps, 1),
                         "random_rows": "the lookup's own rows and bytes (this batch's IDs, "
                                        + f"{row_bytes_in}-byte table rows"
                                        + ("" if fmt == "bf16" else " widened to 1 KiB, with the scale reads")
                                        + "), no arithmetic",
                         "contiguous_ms": round(contig_ms, 5), "contiguous_GBps": round(contig_gbps, 1),
                         "bytes": out_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def row_in_bytes(fmt, D):
    """Bytes read per looked-up row: the bf16 row; fp8 codes and the row's
    scale; NVFP4 codes and block scales."""
    return {"bf16": D * 2, "fp8": D + 4, "fp8-global": D, "nvfp4": D // 2 + D // 16}[fmt]


def lookup_bytes_of(fmt, T, H, D, R):
    """Algorithmic bytes of one lookup: per (token, head) row the table row read
    and the bf16 row written, plus the tokens and query_start_loc."""
    return T * H * (row_in_bytes(fmt, D) + D * 2) + T * 4 + (R + 1) * 4


def bench_library():
    """libple_bench: the streaming-copy ceilings (include/ple_bench.h)."""
    import ctypes
    path = os.path.join(ROOT, "layer_embedding_lookup_amd", "libple_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -m layer_embedding_lookup_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.ple_bench_copy.argtypes = [P, P, ctypes.c_size_t, P]
    lib.ple_bench_copy_rows.argtypes = [P, I64, I32, P, I64, P, P]
    lib.ple_bench_gather_expand.argtypes = [P, I64, I32, P, I32, P, I64, I32, P, P]
    lib.ple_bench_error_message.restype = ctypes.c_char_p
    return lib


def check_bench(rc, lib):
    if rc != 0:
        raise RuntimeError(f"libple_bench call failed ({rc}): {lib.ple_bench_error_message().decode()}")


def host_cpu():
    """nproc, the CPUs this process may run on, and the CPU model name."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)), "cpu_model": model}


def recorded_traffic(workload):
    """HBM bytes per kv_proj launch from the committed counter summary, or None
    when the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "kv_proj_traffic.json")
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("workload") != workload or hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec.get("traffic_bytes")


def bench_host_table(args):
    """Host-resident table: the 8192-token prefill batch over a 67.1M-row
    (64 GiB) bf16 table in pinned host memory that the lookup kernel reads
    directly.  Reports the synchronous lookup (host-link GB/s) and, with the
    next layer's rows prefetched on a CU-masked side stream while the main
    stream runs a 4096x4096 projection stand-in, the lookup time left exposed
    per layer."""
    import numpy as np
    import torch

    import layer_embedding_lookup_amd as ple
    import workloads as wl

    dev = "cuda:0"
    cfg = wl.CONFIGS[5]
    L = 4
    T, H, D, N = cfg.T, cfg.H, cfg.D, cfg.N
    nbytes = cfg.num_rows * D * 2
    log(f"workload {cfg.name}: allocating {nbytes / 2**30:.1f} GiB of pinned host memory")
    t0 = time.time()
    hb = ple.ple_host_alloc(nbytes)
    log(f"pinned in {time.time() - t0:.1f}s; filling")
    table_h = hb.numpy(np.uint16, (cfg.num_rows, D))
    wl.fill_table(cfg, table_h)
    log(f"table ready after {time.time() - t0:.1f}s")
    b = wl.make_batch(cfg, layers=L)
    toks = torch.from_numpy(b.input_ids).to(dev)
    qsl = torch.from_numpy(b.qsl).to(dev)
    tb = ple.Table(hb.device, cfg.num_rows, D, ple.PLE_DTYPE_BF16)
    hashes = [ple.HashParams(b.multipliers[l], b.vocab_sizes, b.offsets, heads_per_ngram=cfg.heads_per_ngram,
                             context_len=cfg.context_len, eos_token_id=wl.EOS) for l in range(L)]
    # projection stand-in for the rest of the layer: [8192, 4096] x [4096, 4096]
    x_std = torch.from_numpy(wl.normal_bf16((T, 4096), 77, 0.02).view(np.int16)).to(dev).view(torch.bfloat16)
    w_std = torch.from_numpy(wl.normal_bf16((4096, 4096), 78, 0.2).view(np.int16)).to(dev).view(torch.bfloat16)
    y_std = torch.empty((T, 4096), dtype=torch.bfloat16, device=dev)
    staging = [torch.empty((T, H * D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    # the distinct-rows prefetch: layers (only hash and table are read), workspace, distinct-row count
    conv_dummy = torch.zeros((N, 4), dtype=torch.bfloat16, device=dev)
    kv_dummy = torch.zeros((2 * N, H * D), dtype=torch.bfloat16, device=dev)
    layers = [ple.Layer(hashes[l], tb, kv_dummy, conv_dummy, conv_dilation=3) for l in range(L)]
    ws_dd = [torch.empty((ple.ple_prefetch_dedup_workspace_bytes(T, H),), dtype=torch.uint8, device=dev)
             for _ in range(2)]
    n_unique = torch.zeros((L,), dtype=torch.int32, device=dev)
    side = ple.ple_stream_create_cu_masked(args.prefetch_cus)
    # the dedup plan's stream takes any CU: it starts once the layer's work is done, when the
    # CUs outside the prefetch stream's mask are idle
    plan_side = torch.cuda.Stream()
    # the layer's work runs on a non-blocking stream: the legacy null stream
    # would serialise with the (blocking) side stream and hide the overlap
    main = torch.cuda.Stream()
    torch.cuda.set_stream(main)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    reps = max(2, args.steps // L)
    try:
        for _ in range(2):
            ple.ple_lookup(hashes[0], tb, toks, qsl, rows=staging[0])
            ple.ple_kv_proj(x_std, w_std, kv=y_std)
        torch.cuda.synchronize()
        lookup_ms = timed(lambda i: ple.ple_lookup(hashes[i % L], tb, toks, qsl, rows=staging[0]), 2 * L)
        gemm_ms = timed(lambda i: ple.ple_kv_proj(x_std, w_std, kv=y_std), 2 * L)

        def sync_layer(i):  # lookup on the critical path, then the layer's work
            ple.ple_lookup(hashes[i % L], tb, toks, qsl, rows=staging[0])
            ple.ple_kv_proj(x_std, w_std, kv=y_std)
        sync_ms = timed(sync_layer, reps * L)

        def fetch_plain(l, buf, stream):
            ple.ple_lookup(hashes[l % L], tb, toks, qsl, rows=staging[buf], stream=stream)

        def fetch_dedup(l, buf, stream):
            ple.ple_prefetch_dedup(layers[l % L], toks, qsl, staging[buf], workspace=ws_dd[buf],
                                   num_unique=n_unique[l % L:l % L + 1], stream=stream)

        for buf in range(2):  # first calls load the kernels
            fetch_dedup(0, buf, None)
        torch.cuda.synchronize()
        dedup_ms = timed(lambda i: fetch_dedup(i, 0, None), 2 * L)

        def sync_layer_dedup(i):
            fetch_dedup(i, 0, None)
            ple.ple_kv_proj(x_std, w_std, kv=y_std)
        sync_dd_ms = timed(sync_layer_dedup, reps * L)
        torch.cuda.synchronize()
        unique_frac = float(n_unique.float().mean().item()) / (T * H)

        def pipelined(n_layers, fetch=fetch_plain):
            ready = [torch.cuda.Event() for _ in range(2)]
            free = [torch.cuda.Event() for _ in range(2)]
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            side.wait_event(e0)
            fetch(0, 0, side)
            ready[0].record(side)
            for l in range(n_layers):
                cur, nxt = l % 2, (l + 1) % 2
                if l + 1 < n_layers:  # prefetch layer l+1 beside layer l
                    if l >= 1:
                        side.wait_event(free[nxt])
                    fetch(l + 1, nxt, side)
                    ready[nxt].record(side)
                main.wait_event(ready[cur])
                ple.ple_kv_proj(x_std, w_std, kv=y_std)   # the layer's work (uses staging[cur] in a real model)
                free[cur].record(main)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        def plan(l, buf, stream):
            ple.ple_prefetch_dedup_plan(layers[l % L], toks, qsl, ws_dd[buf], stream=stream)

        def fetch_planned(l, buf, stream):
            ple.ple_prefetch_dedup_fetch(layers[l % L], T, ws_dd[buf], staging[buf],
                                         num_unique=n_unique[l % L:l % L + 1], stream=stream)

        def pipelined_split(n_layers):
            """The dedup prefetch in two halves: the plan of layer l+2 runs on its own stream once
            layer l's work is done, beside the fetch of layer l+1, so that no short launch of the
            prefetch starts while the layer's work holds the CUs."""
            ready = [torch.cuda.Event() for _ in range(2)]
            free = [torch.cuda.Event() for _ in range(2)]
            planned = [torch.cuda.Event() for _ in range(2)]
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(min(2, n_layers)):
                plan_side.wait_event(e0)
                plan(k, k, plan_side)
                planned[k].record(plan_side)
            side.wait_event(planned[0])
            fetch_planned(0, 0, side)
            ready[0].record(side)
            for l in range(n_layers):
                cur, nxt = l % 2, (l + 1) % 2
                if l + 1 < n_layers:
                    if l >= 1:
                        side.wait_event(free[nxt])
                    side.wait_event(planned[nxt])
                    fetch_planned(l + 1, nxt, side)
                    ready[nxt].record(side)
                main.wait_event(ready[cur])
                ple.ple_kv_proj(x_std, w_std, kv=y_std)
                free[cur].record(main)
                if l + 2 < n_layers:  # workspace cur is free once fetch l is done (before the layer's work)
                    plan_side.wait_event(free[cur])
                    plan(l + 2, cur, plan_side)
                    planned[cur].record(plan_side)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        def staged(n_layers):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(n_layers):
                ple.ple_kv_proj(x_std, w_std, kv=y_std)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        n_layers = reps * L
        pipelined(L)
        pipe_ms = min(pipelined(n_layers) for _ in range(3))
        pipelined(L, fetch_dedup)
        pipe_dd_ms = min(pipelined(n_layers, fetch_dedup) for _ in range(3))
        pipelined_split(L)
        pipe_split_ms = min(pipelined_split(n_layers) for _ in range(3))
        staged_ms = min(staged(n_layers) for _ in range(3))
    finally:
        torch.cuda.synchronize()
        ple.ple_stream_destroy(side)
    rows_bytes = T * H * D * 2
    line = {
        "metric": "host-link GB/s and exposed lookup ms per layer, host-resident PLE table, 8k-token prefill",
        "value": round(rows_bytes / (lookup_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_layers,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "requests": b.R, "heads": H, "table_rows": cfg.num_rows,
                   "dim": D, "table_location": "pinned host, mapped", "layers": L,
                   "stand_in": "ple_kv_proj [8192,4096]x[4096,4096]", "prefetch_cus": args.prefetch_cus},
        "lookup_ms_sync": round(lookup_ms, 4),
        "host_link_GBps": round(rows_bytes / (lookup_ms * 1e-3) / 1e9, 2),
        "stand_in_ms": round(gemm_ms, 4),
        "sync_ms_per_layer": round(sync_ms, 4),
        "pipelined_ms_per_layer": round(pipe_ms / n_layers, 4),
        "staged_ms_per_layer": round(staged_ms / n_layers, 4),
        "exposed_lookup_ms_per_layer": round((pipe_ms - staged_ms) / n_layers, 4),
        "exposed_floor_ms_per_layer": round(max(0.0, lookup_ms - gemm_ms), 4),
        "dedup": {"entry_point": "ple_prefetch_dedup", "distinct_rows_frac": round(unique_frac, 4),
                  "host_bytes_per_layer": int(round(unique_frac * rows_bytes)),
                  "lookup_ms_sync": round(dedup_ms, 4),
                  "host_link_GBps": round(unique_frac * rows_bytes / (dedup_ms * 1e-3) / 1e9, 2),
                  "sync_ms_per_layer": round(sync_dd_ms, 4),
                  "pipelined_ms_per_layer": round(pipe_dd_ms / n_layers, 4),
                  "exposed_lookup_ms_per_layer": round((pipe_dd_ms - staged_ms) / n_layers, 4),
                  "split": {"entry_points": "ple_prefetch_dedup_plan on a second stream, ple_prefetch_dedup_fetch",
                            "pipelined_ms_per_layer": round(pipe_split_ms / n_layers, 4),
                            "exposed_lookup_ms_per_layer": round((pipe_split_ms - staged_ms) / n_layers, 4)}},
    }
    print(json.dumps(line), flush=True)
    hb.close()
    return 0


def bench_select_rows(args):
    """One-GPU part of a table sharded over 8 data-parallel replicas at the 8k
    prefill's width: the rank-major gathered buffer [8][8 x 8192][512] bf16
    (each shard's 1 of 8 heads for every replica's 8192-token slot), and one
    replica selecting its 8192 tokens x 4096 (all heads)."""
    import torch

    import layer_embedding_lookup_amd as ple

    dev = "cuda:0"
    E, S, W = 8, 8192, 512
    gathered = torch.randn((E, E * S, W), device=dev).to(torch.bfloat16)
    out = torch.empty((S, E * W), dtype=torch.bfloat16, device=dev)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for r in range(E):
        ple.ple_select_rows(gathered, r, S, out=out)
    ms = min(timed(lambda i: ple.ple_select_rows(gathered, i % E, S, out=out), 64) for _ in range(3))
    nbytes = 2 * S * E * W * 2
    line = {"metric": "GB/s, rank-major row select (one-GPU part of a DP-sharded table), 8k-token prefill width",
            "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": 64,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "select-rows-8k", "shards": E, "slot_tokens": S, "shard_width": W},
            "ms": round(ms, 5), "bytes": nbytes, "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    print(json.dumps(line), flush=True)
    return 0


def bench_decode(args):
    """Decode on the decode-shaped model: 256 requests of one new token each
    with a 2-token n-gram context and a 9-row conv state, 8 heads over a
    ~1M x 256 bf16 table, hidden 2048, kv_proj 2048 -> 2x2048, conv 4 /
    dilation 3.  A step is one layer's fused path that also writes the next
    context and conv state, timed eagerly; the same step replayed as a HIP
    graph per layer is reported beside it."""
    import numpy as np
    import torch

    import layer_embedding_lookup_amd as ple
    import workloads as wl

    dev = "cuda:0"
    cfg = wl.CONFIGS[2]
    L = args.layers
    T = R = cfg.T
    b = wl.make_batch(cfg, layers=L)
    log(f"decode: R={R} T={T} rows={cfg.num_rows} D={cfg.D} N={cfg.N}")
    table_h, _ = wl.make_table(cfg)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def it(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    tb = ple.Table.from_tensor(bf(table_h))
    kv_ws = [bf(wl.make_kv_weight(cfg, layer=i)) for i in range(4)]
    conv_w = bf(wl.make_conv_weight(cfg))
    hidden = bf(wl.make_hidden(cfg))
    toks, qsl = it(b.input_ids), it(b.qsl)
    hashes = [ple.HashParams(b.multipliers[l], b.vocab_sizes, b.offsets, heads_per_ngram=cfg.heads_per_ngram,
                             context_len=cfg.context_len, eos_token_id=wl.EOS) for l in range(L)]
    layers = [ple.Layer(hashes[l], tb, kv_ws[l % 4], conv_w, conv_dilation=cfg.conv_dilation, eps=cfg.eps)
              for l in range(L)]
    ws = torch.empty((ple.ple_prefill_workspace_bytes(layers[0], T),), dtype=torch.uint8, device=dev)
    st = [[bf(b.conv_state), torch.empty((R, cfg.S, cfg.N), dtype=torch.bfloat16, device=dev)] for _ in range(L)]
    ctx = [[it(b.ngram_context), torch.empty((R, cfg.context_len), dtype=torch.int32, device=dev)]
           for _ in range(L)]
    out = torch.empty((T, cfg.N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(s, swap=True, hint=1):
        # one token per request: the fused entry point's one-kernel decode tail
        l = s % L
        ple.ple_prefill_fused(layers[l], toks, qsl, hidden, ngram_context=ctx[l][0], ngram_context_out=ctx[l][1],
                              conv_state=st[l][0], conv_state_out=st[l][1], out=out, workspace=ws,
                              max_request_tokens=hint)
        if swap:
            st[l].reverse()
            ctx[l].reverse()

    for s in range(max(args.warmup, L)):
        step(s)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for s in range(K):
        step(s)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K
    # the same steps without the hint (separate gate, conv and state kernels)
    for s in range(L):
        step(s, hint=0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(s, hint=0)
    torch.cuda.synchronize()
    unhinted_ms = (time.perf_counter() - t0) * 1e3 / K
    graphs = []
    for l in range(L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(l, swap=False)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        graphs[s % L].replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    H, D, N, S = cfg.H, cfg.D, cfg.N, cfg.S
    # HBM bytes of one step at one pass per array: table rows, rows out and
    # back in, kv weight, kv out and back in, hidden, gated out and back in,
    # output, conv state in and out, tokens, contexts
    step_bytes = (3 * T * H * D * 2 + 2 * N * H * D * 2 + 2 * T * 2 * N * 2 + T * N * 2 + 2 * T * N * 2 + T * N * 2
                  + 2 * R * S * N * 2 + T * 4 + 2 * R * cfg.context_len * 4)
    line = {"metric": "tokens/s, decode step (one new token per request), decode-shaped model (one layer)",
            "value": round(T / (eager_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
            "warmup": args.warmup, "ms_per_step": round(eager_ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "decode-256", "requests": R, "tokens": T, "heads": H, "table_rows": cfg.num_rows,
                       "dim": D, "hidden": N, "kv_proj": [H * D, 2 * N], "conv": [cfg.conv_kernel, cfg.conv_dilation],
                       "context_len": cfg.context_len, "layers_rotated": L},
            "graph_ms_per_step": round(ms_per_step, 4),
            "separate_kernels_ms_per_step": round(unhinted_ms, 4),
            "step_bytes": step_bytes,
            "step_GBps": round(step_bytes / (eager_ms * 1e-3) / 1e9, 1)}
    print(json.dumps(line), flush=True)
    return 0


def bench_spec_decode(args):
    """Speculative decode on the decode-shaped model (256 requests, 8 heads over
    a ~1M x 256 bf16 table, hidden 2048, conv 4 / dilation 3): each request
    verifies a 4-token window (its last token and 3 drafts) through the fused
    path, then the carried conv state and n-gram context are committed for the
    1..4 accepted tokens (uniform).  A step is one layer's verify + commit,
    timed eagerly (the same step replayed as a HIP graph per layer is reported
    beside it); verify and commit are each timed as graphs of back-to-back
    calls."""
    import numpy as np
    import torch

    import layer_embedding_lookup_amd as ple
    import workloads as wl

    dev = "cuda:0"
    cfg = wl.CONFIGS[2]
    W, L = 4, args.layers
    R = cfg.T
    T = R * W
    b = wl.make_batch(cfg, layers=L)
    toks_h = wl.make_tokens(cfg, T=T)
    qsl_h = np.arange(0, T + 1, W, dtype=np.int32)
    acc_h = wl.uniform_ints(wl.stream_seed(cfg.seed, 99), R, 1, W + 1)
    log(f"spec decode: R={R} window={W} T={T} rows={cfg.num_rows} D={cfg.D} N={cfg.N}")
    table_h, _ = wl.make_table(cfg)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def it(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    tb = ple.Table.from_tensor(bf(table_h))
    kv_ws = [bf(wl.make_kv_weight(cfg, layer=i)) for i in range(4)]
    conv_w = bf(wl.make_conv_weight(cfg))
    hidden = bf(wl.make_hidden(cfg, T=T))
    toks, qsl, acc = it(toks_h), it(qsl_h), it(acc_h)
    hashes = [ple.HashParams(b.multipliers[l], b.vocab_sizes, b.offsets, heads_per_ngram=cfg.heads_per_ngram,
                             context_len=cfg.context_len, eos_token_id=wl.EOS) for l in range(L)]
    layers = [ple.Layer(hashes[l], tb, kv_ws[l % 4], conv_w, conv_dilation=cfg.conv_dilation, eps=cfg.eps)
              for l in range(L)]
    nbytes = ple.ple_prefill_workspace_bytes(layers[0], T)
    ws = [torch.empty((nbytes,), dtype=torch.uint8, device=dev) for _ in range(L)]
    xs = [ple.prefill_conv_input(layers[l], ws[l], T) for l in range(L)]
    # per layer: the state and context the step starts from, and the committed ones
    st = [[bf(b.conv_state), torch.empty((R, cfg.S, cfg.N), dtype=torch.bfloat16, device=dev)] for _ in range(L)]
    ctx = [[it(b.ngram_context), torch.empty((R, cfg.context_len), dtype=torch.int32, device=dev)]
           for _ in range(L)]
    out = torch.empty((T, cfg.N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def verify(s, hint=W):
        # windows of W <= 4 tokens: the fused entry point's one-kernel tail for gate and conv
        l = s % L
        ple.ple_prefill_fused(layers[l], toks, qsl, hidden, ngram_context=ctx[l][0], conv_state=st[l][0], out=out,
                              workspace=ws[l], max_request_tokens=hint)

    def commit(s):
        l = s % L
        ple.ple_spec_commit(toks, qsl, acc, hash=hashes[l], ngram_context=ctx[l][0], ngram_context_out=ctx[l][1],
                            x=xs[l], conv_kernel=cfg.conv_kernel, conv_dilation=cfg.conv_dilation,
                            conv_state=st[l][0], conv_state_out=st[l][1])

    def step(s, hint=W):
        verify(s, hint)
        commit(s)
        l = s % L
        st[l].reverse()
        ctx[l].reverse()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for s in range(max(args.warmup, L)):
        step(s)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for s in range(K):
        step(s)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K
    # the same steps with separate gate and conv kernels (no window hint)
    for s in range(L):
        step(s, hint=0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(s, hint=0)
    torch.cuda.synchronize()
    unhinted_ms = (time.perf_counter() - t0) * 1e3 / K
    # The same step as a HIP graph per layer (verify + commit; the library
    # allocates nothing and clears nothing with memset, so the calls capture
    # as plain kernel nodes), replayed the way a serving loop would.
    graphs = []
    for l in range(L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            verify(l)
            commit(l)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        graphs[s % L].replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K

    def graph_of(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        return g

    reps = 4 * L
    g_verify, g_commit = graph_of(verify, reps), graph_of(commit, reps)
    verify_ms = min(timed(lambda i: g_verify.replay(), 4) for _ in range(3)) / reps
    commit_ms = min(timed(lambda i: g_commit.replay(), 4) for _ in range(3)) / reps
    S, N, C = cfg.S, cfg.N, cfg.context_len
    # each committed state row is read once (from the old state or the window) and written once
    commit_bytes = 2 * R * S * N * 2 + 2 * R * C * 4 + R * 4 + (R + 1) * 4
    line = {"metric": "tokens/s, speculative verify + state commit, decode-shaped model (one layer)",
            "value": round(T / (eager_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
            "warmup": args.warmup, "ms_per_step": round(eager_ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "spec-decode-256x4", "requests": R, "window": W, "tokens": T,
                       "accepted_mean": round(float(acc_h.mean()), 3), "heads": cfg.H, "table_rows": cfg.num_rows,
                       "dim": cfg.D, "hidden": N, "conv": [cfg.conv_kernel, cfg.conv_dilation],
                       "context_len": C, "layers_rotated": L},
            "committed_tokens_per_s": round(float(acc_h.sum()) / (eager_ms * 1e-3), 1),
            "graph_ms_per_step": round(ms_per_step, 4),
            "separate_kernels_ms_per_step": round(unhinted_ms, 4),
            "verify_ms": round(verify_ms, 5),
            "commit": {"ms": round(commit_ms, 5), "bytes": commit_bytes,
                       "GBps": round(commit_bytes / (commit_ms * 1e-3) / 1e9, 1),
                       "frac_hbm_peak": round(commit_bytes / (commit_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}}
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(cfg, b, table_h, scales_h, kvw_h, conv_w_h, hidden_h, n_tokens, workload):
    """The oracle, single-threaded and pinned to one core of the host: its IDs and
    row gather (+ dequant) over every token of the batch, and the whole path
    (ids, gather, kv_proj, gate, conv) on a bounded sample, the first n_tokens
    of the batch (whole requests, the last one cut to a prefix chunk; by
    causality their outputs equal the full batch's)."""
    import numpy as np

    import oracle
    import workloads as wl

    host = host_cpu()
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        T, H, D = cfg.T, cfg.H, cfg.D
        ids_args_all = dict(input_ids=b.input_ids, qsl=b.qsl, multipliers=b.multipliers[0],
                            vocab_sizes=b.vocab_sizes, offsets=b.offsets, context_len=cfg.context_len,
                            heads_per_ngram=cfg.heads_per_ngram, eos_token_id=wl.EOS)
        log(f"cpu baseline: oracle pinned to core {core}: ids + gather over all {T} tokens")
        t0 = time.perf_counter()
        ids = oracle.ngram_ids(**ids_args_all)
        if scales_h is None:
            oracle.gather_bf16(table_h, ids)
        elif isinstance(scales_h, tuple):
            oracle.gather_nvfp4(table_h, scales_h[0], scales_h[1], ids)
        elif np.size(scales_h) == 1:
            oracle.gather_fp8_global(table_h, np.asarray(scales_h).reshape(-1)[0], ids)
        else:
            oracle.gather_fp8(table_h, scales_h, ids)
        dt_ig = time.perf_counter() - t0
        if scales_h is None:
            row_read = D * 2
        elif isinstance(scales_h, tuple):
            row_read = D // 2 + D // 16
        else:
            row_read = D if np.size(scales_h) == 1 else D + 4
        ig_bytes = T * H * (row_read + D * 2) + T * 4 + (b.R + 1) * 4

        n = int(min(n_tokens, cfg.T))
        q = b.qsl.astype(np.int64)
        R = int(np.searchsorted(q, n, side="left"))  # requests 0..R-1 cover [0, n)
        qsl = np.minimum(q[:R + 1], n).astype(np.int32)
        qsl[-1] = n
        log(f"cpu baseline: oracle on the first {n} tokens ({R} requests), whole path")
        ids_args = dict(ids_args_all, input_ids=b.input_ids[:n], qsl=qsl)
        t0 = time.perf_counter()
        oracle.prefill(ids_args, table_h, scales_h, hidden_h[:n], kvw_h, conv_w_h, cfg.conv_dilation, qsl=qsl,
                       eps=cfg.eps)
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, allowed)
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} tokens ({R} requests) of the {workload} batch, whole path "
                      f"(ids, gather, kv_proj, gate, conv), single-threaded C pinned to one core, {dt:.1f} s",
            "ids_gather": {"tokens": T, "s": round(dt_ig, 3), "tokens_per_s": round(T / dt_ig, 1),
                           "GBps": round(ig_bytes / dt_ig / 1e9, 3),
                           "what": "ids + row gather (+ dequant) over every token, same algorithmic bytes as "
                                   "the GPU lookup"},
            "host": host}


if __name__ == "__main__":
    sys.exit(main())
