#!/usr/bin/env python3
"""Benchmark of MLA paged latent decode on one MI355X.

One step = one decode of the whole batch (stage 1 split-KV attention, then
the stage-2 log-sum-exp merge) on synthetic seeded inputs already resident in
HBM.  Default workload: B=64 sequences, H=128 heads, D=576 (kv_lora_rank 512
+ rope 64), bf16 q and cache, page 64, pool of 8192 pages, lengths uniform in
[1024, 8192], shuffled block table, scale 192^-0.5.

Two copies of the cache (the second with every page moved to another
physical slot) alternate step by step, so consecutive steps never find the
previous step's rows in the 256 MB Infinity Cache.

Prints ONE JSON line: value = algorithmic HBM GB/s of the whole decode
(bytes the method must move / time per step), plus TFLOP/s, the roofline of
the stage-1 kernel timed with HIP events on its own stream, and the float64
CPU oracle timed on the host as a baseline.

Extra modes:
  --copy-calibration   also runs a plain 1 GiB device copy (for scaling
                       rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
  --ingest-pmc F W [M] turn rocprofv3 --pmc counter CSVs (FETCH_SIZE,
                       WRITE_SIZE runs of this script with --copy-calibration,
                       optionally an MFMA pass: SQ_VALU_MFMA_BUSY_CYCLES,
                       SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE) into
                       profiles/<kernel>_<workload>_traffic.json
  --peaks              measured peaks next to the spec ones: a 1 GiB device
                       copy and read-only sums (HBM), a bf16 8192^3 GEMM
                       (hipBLASLt, MFMA), and the in-tree probes of
                       libmla_peaks.so: HBM -> LDS streaming in the decode's
                       load pattern, a v_mfma_f32_32x32x16_bf16 loop and
                       ds_read_b128 LDS reads
  --dcp G              time the cross-shard merge of G page shards
  --zero-data          power study: the same batch, plan and pages with the
                       query and the cache zeroed (same instructions and
                       bytes, less switching power); the line says so in
                       "data" and carries no counter traffic or CPU baseline
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode HBM GB/s + MFMA TFLOP/s (% of peak), B=64 H=128 D=576 ctx 1k-8k"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, public spec
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, public spec
# the sources the stage-1 kernel is compiled from: counters read on one
# version are reported only while all of them are unchanged
KERNEL_SRCS = [os.path.join(ROOT, "mla_paged_latent_decode_amd", "csrc", f)
               for f in ("mla_kernels.hip", "mla_device.h", "mla_internal.h")]
COPY_BYTES = 1 << 30
EVENT_EVERY = 4           # per-kernel events on every 4th timed step (see the timed loop)


def kernel_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(inp):
    """Bytes and FLOPs the method itself must move / compute (no workspace,
    no padding): the cache rows read once, q, o, lse, the table entries and
    seq_lens; FLOPs = 2 H (D + D_v) times the keys each query token sees
    (sum(n) for single-token decode; multi-token decode: query token i sees
    n - q_len + 1 + i keys)."""
    import numpy as np
    w = inp.workload
    n = np.asarray(inp.seq_lens, dtype=np.int64)
    B, H, D, DV, P = w.batch, w.num_heads, w.head_size, w.kv_lora_rank, w.page_size
    # bytes of one cache row the method needs: bf16 values, fp8 codes, or the
    # per-token codes (fp8, int8: D bytes; int4: D/2) and the token's fp32 scale
    # (the rest of the per-token pad is unused)
    row = {"bf16": 2 * D, "fp8_per_token": D + 4, "int8_per_token": D + 4,
           "int4_per_token": D // 2 + 4}.get(w.kv_dtype, D)
    ql = w.q_len
    if w.topk:
        # sparse decode: the selected rows, the index lists and one table entry each
        k = int(np.asarray(inp.topk_lens, dtype=np.int64).sum())
        kv = k * row
        stage1 = kv + B * H * D * 2 + k * 4 + k * 4 + 4 * B
        total = stage1 + B * H * DV * 2 + B * H * 4
        flops = 2 * H * k * (D + DV)
        return {"kv_bytes": kv, "stage1_bytes": stage1, "total_bytes": total, "flops": flops,
                "tokens": k}
    kv = int(n.sum()) * row
    table = int(((n + P - 1) // P).sum()) * 4
    stage1 = kv + B * ql * H * D * 2 + table + 4 * B
    total = stage1 + B * ql * H * DV * 2 + B * ql * H * 4
    seen = sum(int(np.clip(n - ql + 1 + i, 0, n).sum()) for i in range(ql))
    flops = 2 * H * seen * (D + DV)
    return {"kv_bytes": kv, "stage1_bytes": stage1, "total_bytes": total, "flops": flops,
            "tokens": int(n.sum())}


def host_facts():
    """Cores this process may run on (sched_getaffinity), the CPU model name
    (lscpu), and the thread count of the BLAS numpy uses."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().lower().startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        pass
    return cores, model, threads


def cpu_baseline(inp, alg, budget_s=25.0):
    """The float64 oracle on the host cores, over whole sequences of the same
    batch until the batch is done or the time budget is spent.  The oracle
    processes one sequence at a time; its two products per sequence (scores,
    then weights times V) run in the host BLAS with `blas_threads` threads."""
    import numpy as np
    import oracle
    w = inp.workload
    cores, model, threads = host_facts()
    done, tok = 0, 0
    t0 = time.perf_counter()
    fn = oracle.decode if w.q_len == 1 else oracle.decode_mtp
    for b in range(w.batch):
        if w.topk:
            oracle.decode_sparse(inp.q_bits, inp.kv_bits, inp.block_table, inp.topk_indices,
                                 inp.topk_lens, scale=w.scale, k_scale=w.k_scale,
                                 kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank, batches=[b])
            tok += int(inp.topk_lens[b])
        else:
            fn(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens, scale=w.scale,
               k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank,
               batches=[b])
            tok += int(inp.seq_lens[b])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    per_token = alg["total_bytes"] / alg["tokens"]
    return {"value": round(tok * per_token / dt / 1e9, 4), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.batch} sequences ({tok} tokens) of the same batch, "
                      f"{dt:.1f} s, numpy float64 with BLAS on the host",
            "cpu_model": model, "blas_threads": threads,
            "tokens_heads_per_s": round(tok * w.num_heads / dt, 1)}


def load_counters(workload):
    """The stage-1 counter figures of profiles/mla_stage1_<workload>_traffic.json,
    or None when they were taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"mla_stage1_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha256_16") != kernel_hash():
        return None  # counters were taken on another version of the kernel
    return t


def load_traffic(workload):
    t = load_counters(workload)
    return t.get("bytes_per_launch") if t else None


def ingest_pmc(fetch_csv, write_csv, workload, mfma_csv=None):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the stage-1
    kernel, scaled by what the same counters read for the 1 GiB copy."""
    def per_kernel(path, counter):
        acc = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                acc.setdefault(name, []).append(float(row["Counter_Value"]))
        return acc
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, key):
        ks = [k for k in d if key in k]
        vals = [v for k in ks for v in d[k]]
        return sum(vals) / len(vals) if vals else None

    def copy_of(d):
        ks = [k for k in d if "copy" in k.lower() or "elementwise" in k.lower()]
        vals = [v for k in ks for v in d[k]]
        return max(vals) if vals else None
    f1, w1 = pick(fetch, "mla_stage1"), pick(write, "mla_stage1")
    fc, wc = copy_of(fetch), copy_of(write)
    ffac = COPY_BYTES / (fc * 1024) if fc else 1.0
    wfac = COPY_BYTES / (wc * 1024) if wc else 1.0
    out = {"workload": workload, "kernel_sha256_16": kernel_hash(),
           "fetch_kib_per_dispatch": f1, "write_kib_per_dispatch": w1,
           "copy_fetch_kib": fc, "copy_write_kib": wc, "fetch_scale": ffac, "write_scale": wfac,
           "bytes_per_launch": (f1 * 1024 * ffac + w1 * 1024 * wfac) if f1 and w1 else None,
           "sources": [os.path.basename(fetch_csv), os.path.basename(write_csv)]}
    if mfma_csv:
        # the MFMA work the hardware counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 is
        # in units of 512 FLOP), per dispatch; the raw busy-cycle and GPU-busy
        # counters are kept as read
        mops = pick(per_kernel(mfma_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), "mla_stage1")
        out["mfma_flops_counted"] = mops * 512 if mops else None
        out["sq_valu_mfma_busy_cycles"] = pick(per_kernel(mfma_csv, "SQ_VALU_MFMA_BUSY_CYCLES"),
                                               "mla_stage1")
        out["grbm_gui_active"] = pick(per_kernel(mfma_csv, "GRBM_GUI_ACTIVE"), "mla_stage1")
        out["sources"].append(os.path.basename(mfma_csv))
    path = os.path.join(ROOT, "profiles", f"mla_stage1_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def run_peaks(args):
    """Measured peaks next to the spec ones: HBM from a 1 GiB device-to-device
    copy (2 GiB moved per copy) and from read-only fp32 sums (torch's
    reduction over 1 GiB and over the 356 MB the dsv3 batch's cache rows
    take), MFMA from a bf16 8192^3 GEMM (hipBLASLt), each the median of 20
    timed runs after 5 warm-ups."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def timed(fn, n=20):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e-3

    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del dst
    t_sum = timed(lambda: src.sum())
    small = src[:309371 * 1152 // 4]
    t_sum_small = timed(lambda: small.sum())
    del src, small
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    t_mm = timed(lambda: torch.mm(a, b))
    copy_gbs = 2 * COPY_BYTES / t_copy / 1e9
    mm_tflops = 2 * n ** 3 / t_mm / 1e12
    del a, b
    probes = run_probes(timed)
    print(json.dumps({
        "metric": "measured peaks (one MI355X)",
        "copy_GBps": round(copy_gbs, 1), "copy_frac_of_spec": round(copy_gbs / HBM_PEAK_GBS, 4),
        "read_sum_GBps": round(COPY_BYTES / t_sum / 1e9, 1),
        "read_sum_356MB_GBps": round(309371 * 1152 / t_sum_small / 1e9, 1),
        "gemm_bf16_TFLOPs": round(mm_tflops, 1),
        "gemm_frac_of_spec": round(mm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "spec": {"hbm_GBps": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS},
        "probes": probes,
        "how": "median of 20 HIP-event-timed runs: torch copy_ of 1 GiB (read + write), "
               "torch sum of 1 GiB and of 356 MB fp32 (read only), "
               "torch.mm bf16 8192x8192x8192; probes: libmla_peaks.so kernels, GB/s or "
               "TFLOP/s from the events, cycles from each workgroup's s_memtime and the "
               "shader clock from s_memtime over s_memrealtime (100 MHz)"}), flush=True)
    return 0


def run_probes(timed):
    """The in-tree probes of libmla_peaks.so (see mla_peaks.hip):
    - stream: HBM -> LDS copies of 36 KB tiles (halves of 64-row pages of
      1152-byte rows, pages in a seeded random order) through a ring of LDS
      tiles, one workgroup per CU, about the dsv3 cache's bytes per launch;
      the decode's configuration is 4 waves, ring 3, 16-row loads;
    - mfma: v_mfma_f32_32x32x16_bf16 on every SIMD, on 8 independent
      accumulator chains and on 1, 2 and 4 (cycles per MFMA);
    - lds: ds_read_b128 by 4 and 8 waves per CU;
    - tileloop: the stage-1 tile loop stripped to its copies, MFMAs, LDS
      operand reads and softmax-like VALU work, with and without the copies,
      on pages of N(0,1) bf16 values and on zeroed pages (same instructions
      and bytes): the time per tile and the shader clock it ran at."""
    import ctypes
    import numpy as np
    import torch
    from mla_paged_latent_decode_amd import _build
    lib = ctypes.CDLL(_build.PEAKS_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.mla_peak_stream.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.mla_peak_mfma.argtypes = [i32, i32, vp, vp, vp]
    lib.mla_peak_mfma_chain.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.mla_peak_lds.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    lib.mla_peak_tileloop.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid = cus
    cyc = torch.zeros((4 * grid, 2), dtype=torch.int64, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    out = {}

    def clock(g):
        c = cyc[:g].cpu().numpy().astype(np.float64)
        return c[:, 0], float(np.median(c[:, 0] / np.maximum(c[:, 1], 1) * 100.0))

    pool_pages = 8192
    pool = torch.empty(pool_pages * 64 * 1152, dtype=torch.uint8, device=dev).fill_(1)
    per_wg = 38
    g = np.random.default_rng(1234)
    pages = torch.from_numpy(g.permutation(pool_pages)[: grid * per_wg // 2].astype(np.int32)).to(dev)
    nbytes = grid * per_wg * 36 * 1024
    for waves, ring, rows, read in ((4, 3, 1, 0), (4, 2, 1, 0), (4, 4, 1, 0), (4, 3, 0, 0),
                                    (4, 3, 1, 1), (8, 3, 1, 0), (8, 4, 1, 0), (8, 3, 1, 1)):
        def go():
            rc = lib.mla_peak_stream(pool.data_ptr(), pages.data_ptr(), grid, per_wg, waves, ring,
                                     rows, read, cyc.data_ptr(), sink.data_ptr(), stream)
            if rc:
                raise RuntimeError(f"mla_peak_stream failed: {rc}")
        t = timed(go)
        cycles, mhz = clock(grid)
        key = f"stream_w{waves}_ring{ring}_{'rows' if rows else 'contig'}{'_read' if read else ''}"
        out[key] = {"GBps": round(nbytes / t / 1e9, 1), "frac_of_spec": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                    "us_per_tile": round(t * 1e6 / per_wg, 3),
                    "cycles_per_tile": round(float(np.median(cycles)) / per_wg, 1),
                    "mhz": round(mhz)}
    # the tile loop on pages of N(0,1) bf16 values and on zeroed pages, in two
    # alternating passes (the clock follows the recent load with some lag)
    normal = torch.empty(pool.numel() // 2, dtype=torch.bfloat16, device=dev)
    normal.normal_(generator=torch.Generator(device=dev).manual_seed(1234))
    for pas, data in ((1, "normal"), (1, "zero"), (2, "normal"), (2, "zero")):
        if data == "zero":
            pool.zero_()
        else:
            pool.view(torch.bfloat16).copy_(normal)
        for copy in (1, 0):
            def go_loop():
                rc = lib.mla_peak_tileloop(pool.data_ptr(), pages.data_ptr(), grid, per_wg, copy,
                                           cyc.data_ptr(), sink.data_ptr(), stream)
                if rc:
                    raise RuntimeError(f"mla_peak_tileloop failed: {rc}")
            t = timed(go_loop)
            cycles, mhz = clock(grid)
            key = f"tileloop_{'copies_compute' if copy else 'compute_only'}_{data}_pass{pas}"
            out[key] = {"us_per_tile": round(t * 1e6 / per_wg, 3),
                        "cycles_per_tile": round(float(np.median(cycles)) / per_wg, 1),
                        "mhz": round(mhz)}
    del pool, normal
    iters = 2000

    def go_mfma():
        if lib.mla_peak_mfma(grid, iters, cyc.data_ptr(), sink.data_ptr(), stream):
            raise RuntimeError("mla_peak_mfma failed")
    t = timed(go_mfma)
    cycles, mhz = clock(grid)
    flops = grid * 4 * iters * 8 * 32 * 32 * 16 * 2
    out["mfma_bf16_32x32x16"] = {"TFLOPs": round(flops / t / 1e12, 1),
                                 "frac_of_spec": round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                 "cycles_per_mfma": round(float(np.median(cycles)) / (iters * 8), 2),
                                 "mhz": round(mhz)}
    for chains in (1, 2, 4):
        def go_chain():
            if lib.mla_peak_mfma_chain(grid, iters, chains, cyc.data_ptr(), sink.data_ptr(), stream):
                raise RuntimeError("mla_peak_mfma_chain failed")
        timed(go_chain)
        cycles, mhz = clock(grid)
        out[f"mfma_bf16_32x32x16_{chains}_chains"] = {
            "cycles_per_mfma": round(float(np.median(cycles)) / (iters * 8), 2), "mhz": round(mhz)}
    for tr in (0, 1):
        for waves in (4, 8):
            lit = 200

            def go_lds():
                if lib.mla_peak_lds(grid, waves, lit, tr, cyc.data_ptr(), sink.data_ptr(), stream):
                    raise RuntimeError("mla_peak_lds failed")
            t = timed(go_lds)
            cycles, mhz = clock(grid)
            per_wg_bytes = waves * lit * (32 if tr else 64) * 1024
            name = "lds_read_b64_tr_b16" if tr else "lds_read_b128"
            out[f"{name}_w{waves}"] = {"bytes_per_clk_per_cu":
                                       round(per_wg_bytes / float(np.median(cycles)), 1),
                                       "mhz": round(mhz)}
    return out


def run_dcp(args, G):
    """Context-parallel decode on one GPU: the workload's batch is cut into G
    round-robin page shards, each decoded by the library (untimed, bf16 o and
    fp32 lse, as a serving stack would exchange them), and the timed step is
    the merge of the G shard results into the final (o, lse).  On G GPUs each
    would decode its own shard; the merge is the one step the context split
    adds (after the exchange of the shard results, which one GPU cannot show)."""
    import numpy as np
    import torch

    import mla_paged_latent_decode_amd as mla
    import workloads as W

    dev = torch.device("cuda:0")
    inp = W.generate(args.workload)
    w = inp.workload
    if w.kv_dtype != "bf16" or w.q_len != 1 or w.topk:
        print("--dcp runs on the bf16 single-token workloads", file=sys.stderr)
        return 2
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    o_parts, l_parts = [], []
    for r in range(G):
        sh = W.shard_pages(inp, G, r)
        bt = torch.from_numpy(sh.block_table).to(dev)
        sl = torch.from_numpy(sh.seq_lens).to(dev)
        o, lse = mla.mla_decode(q, kv, bt, sl, w.scale, w.page_size, w.k_scale, num_cus=cus)
        o_parts.append(o)
        l_parts.append(lse)
    o_p = torch.stack(o_parts).contiguous()
    l_p = torch.stack(l_parts).contiguous()
    del kv
    o = torch.empty((w.batch, w.num_heads, w.kv_lora_rank), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.num_heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        mla.mla_merge_shards(o_p, l_p, "ln", o, lse, stream=stream)
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        evs[i][0].record(stream)
        mla.mla_merge_shards(o_p, l_p, "ln", o, lse, stream=stream)
        evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    rows = w.batch * w.num_heads
    # every shard row (bf16) and lse read once, the merged row and lse written once
    nbytes = G * rows * (w.kv_lora_rank * 2 + 4) + rows * (w.kv_lora_rank * 2 + 4)
    ach = nbytes / (launch_ms * 1e-3) / 1e9
    out = {
        "metric": "MLA context-parallel shard merge GB/s (% of HBM peak)",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} merge of {G} round-robin page shards: {w.description}",
                   "batch": w.batch, "heads": w.num_heads, "kv_lora_rank": w.kv_lora_rank,
                   "shards": G, "seed": w.seed},
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "mla_merge_shards_kernel", "avg_launch_ms": round(launch_ms, 5)},
    }
    if not args.no_cpu_baseline:
        import oracle
        op = o_p.float().cpu().numpy().astype(np.float64)
        lp = l_p.cpu().numpy().astype(np.float64)
        done = 0
        t1 = time.perf_counter()
        for b in range(w.batch):
            oracle.merge_shards(op[:, b], lp[:, b])
            done += 1
            if time.perf_counter() - t1 > 20.0:
                break
        dt = time.perf_counter() - t1
        out["cpu_baseline"] = {
            "value": round(done * w.num_heads * (G + 1) * (w.kv_lora_rank * 2 + 4) / dt / 1e9, 4),
            "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {w.batch} sequences' rows merged by oracle.merge_shards "
                      f"(python loop per row, float64), {dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the first ~200 steps run up to 10 % slower while the GPU settles into
    # its steady clocks, so the default warm-up is that long (≈ 30 ms)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--split", default="plan", choices=["plan", "pages", "single"])
    ap.add_argument("--fixed-splits", type=int, default=0, metavar="S",
                    help="per-sequence split mode with S splits of every sequence (a fixed S "
                         "is batch-invariant); overrides --split")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--zero-data", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ingest-pmc", nargs="+", metavar="CSV")
    ap.add_argument("--peaks", action="store_true")
    ap.add_argument("--dcp", type=int, default=0, metavar="G",
                    help="time the cross-shard merge of G round-robin page shards of the "
                         "workload instead of the decode (the shards are decoded untimed)")
    args = ap.parse_args()

    if args.ingest_pmc:
        if len(args.ingest_pmc) not in (2, 3):
            ap.error("--ingest-pmc takes FETCH_CSV WRITE_CSV [MFMA_CSV]")
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload,
                   args.ingest_pmc[2] if len(args.ingest_pmc) == 3 else None)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world}): this "
              "library has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mla_paged_latent_decode_amd as mla
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.dcp:
        return run_dcp(args, args.dcp)
    if args.peaks:
        return run_peaks(args)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp = W.generate(args.workload)
    w = inp.workload
    alg = algorithmic(inp)
    print(f"[bench] generated {args.workload} in {time.perf_counter() - t_gen:.1f}s: "
          f"{alg['tokens']} tokens", file=sys.stderr, flush=True)

    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if w.kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    elif w.kv_dtype in ("fp8_per_token", "int8_per_token", "int4_per_token"):
        kv = torch.from_numpy(inp.kv_bits).to(dev)  # uint8 rows: codes | fp32 scale | pad
    else:
        kv = torch.from_numpy(inp.kv_bits).view(torch.float8_e4m3fn).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    if args.zero_data:
        q.zero_()
        kv.view(torch.uint8).zero_()  # any cache dtype (fp8 has no fill)
    # second copy of the cache with its pages moved (input preparation only)
    g = torch.Generator(device="cpu").manual_seed(1234)
    new_of_old = torch.randperm(kv.shape[0], generator=g).to(dev)
    kv2 = torch.empty_like(kv)
    kv2[new_of_old] = kv
    bt2 = new_of_old.to(torch.int32)[bt.long()].contiguous()
    sets = [(kv, bt), (kv2, bt2)]

    shape = mla.shape_of(q, kv, bt, kv_dtype=w.kv_dtype)
    max_len, tot = int(inp.seq_lens.max()), int(inp.seq_lens.sum())
    topk_dev = None
    if w.topk:  # sparse decode: the plan counts list entries
        max_len, tot = w.topk, int(inp.topk_lens.sum())
        topk_dev = torch.from_numpy(inp.topk_indices).to(dev)
        sl = torch.from_numpy(inp.topk_lens).to(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ql = w.q_len
    if args.fixed_splits > 0:
        mode, splits = mla.SPLIT_PER_SEQUENCE, args.fixed_splits
        ws_bytes = mla.mla_workspace_size(shape, mode, splits, ql)
    elif args.split == "plan":
        mode, splits, ws_bytes = mla.mla_plan(shape, max_len, tot, cus, q_len=ql)
    elif args.split == "pages":
        mode, splits = mla.SPLIT_PER_SEQUENCE, mla.mla_pages_split_count(max_len, cus)
        ws_bytes = mla.mla_workspace_size(shape, mode, splits, ql)
    else:
        mode, splits, ws_bytes = mla.SPLIT_PER_SEQUENCE, 1, 0
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    rows = (w.batch, w.num_heads) if ql == 1 else (w.batch, ql, w.num_heads)
    o = torch.empty(rows + (w.kv_lora_rank,), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    calls = [mla.PreparedDecode(q, k, b, sl, w.scale, w.page_size, w.k_scale, splits, mode, o,
                                lse, ws, stream=stream.cuda_stream, topk_indices=topk_dev,
                                kv_dtype=w.kv_dtype)
             for (k, b) in sets]

    for i in range(args.warmup):
        calls[i % 2]("stage1")
        calls[i % 2]("stage2")
    torch.cuda.synchronize()

    K = args.steps
    # Per-kernel HIP events on every EVENT_EVERY-th step, recorded by the two
    # kernel launches themselves (mla_time_next_launch): they bracket each
    # kernel alone, as a profiler's kernel trace does, and add no marker
    # between the launches.  torch creates an event at its first record, so
    # each is recorded once here before the timed loop.
    sampled = [i for i in range(K) if i % EVENT_EVERY == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in sampled}
    for e in evs.values():
        for x in e:
            x.record(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        c = calls[i % 2]
        e = evs.get(i)
        if e:
            mla.mla_time_next_launch(1, e[0], e[1])
            if mode == mla.SPLIT_BALANCED or splits > 1:
                mla.mla_time_next_launch(2, e[2], e[3])
        c("stage1")
        c("stage2")
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K
    s1 = np.array([e[0].elapsed_time(e[1]) for e in evs.values()])
    s2 = (np.array([e[2].elapsed_time(e[3]) for e in evs.values()])
          if mode == mla.SPLIT_BALANCED or splits > 1 else np.zeros(len(evs)))

    if args.copy_calibration:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()

    gbs = alg["total_bytes"] / (ms_step * 1e-3) / 1e9
    tflops = alg["flops"] / (ms_step * 1e-3) / 1e12
    s1_ms = float(s1.mean())
    t_hbm = alg["stage1_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        ach = alg["stage1_bytes"] / (s1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = alg["flops"] / (s1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    # the stored counters were read on the planner's launch configuration;
    # another split moves other partial bytes
    stored = args.split == "plan" and not args.fixed_splits and not args.zero_data
    roof["traffic"] = load_traffic(args.workload) if stored else None
    counters = load_counters(args.workload) if stored else None
    if counters and counters.get("mfma_flops_counted"):
        # MFMA work counted by the hardware for one launch, over the measured
        # launch time: the MFMA rate from counters rather than from the method
        rate = counters["mfma_flops_counted"] / (s1_ms * 1e-3) / 1e12
        roof["mfma_tflops_counted"] = round(rate, 1)
        roof["mfma_frac_counted"] = round(rate / MFMA_BF16_PEAK_TFLOPS, 4)
    roof["kernel"] = "mla_stage1"
    roof["avg_launch_ms"] = round(s1_ms, 5)
    roof["mfma_tflops"] = round(alg["flops"] / (s1_ms * 1e-3) / 1e12, 1)
    roof["mfma_frac"] = round(roof["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    roof["hbm_gbs"] = round(alg["stage1_bytes"] / (s1_ms * 1e-3) / 1e9, 1)
    roof["hbm_frac"] = round(roof["hbm_gbs"] / HBM_PEAK_GBS, 4)
    roof["roofline_frac"] = round(max(t_hbm, t_mfma) / (s1_ms * 1e-3), 4)

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.kv_dtype,
        "data": "synthetic, query and cache zeroed (power study)" if args.zero_data else "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.batch,
                   "heads": w.num_heads, "head_size": w.head_size,
                   "kv_lora_rank": w.kv_lora_rank, "page_size": w.page_size,
                   "total_tokens": alg["tokens"], "q_len": ql, "topk": w.topk,
                   "split_mode": int(mode),
                   "num_kv_splits": int(splits), "seed": w.seed},
        "tflops": round(tflops, 1),
        "tokens_heads_per_s": round(alg["tokens"] * w.num_heads / (ms_step * 1e-3), 1),
        "roofline_frac_total": round(max(alg["total_bytes"] / (HBM_PEAK_GBS * 1e9), t_mfma)
                                     / (ms_step * 1e-3), 4),
        "stage2_avg_ms": round(float(s2.mean()), 5),
        "stage1_ms_p10_p50_p90": [round(float(np.percentile(s1, q)), 5) for q in (10, 50, 90)],
        "sampled_step_ms_p10_p50_p90": [round(float(np.percentile(s1 + s2, q)), 5)
                                        for q in (10, 50, 90)],
        "wall_s": round(wall, 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline and not args.zero_data:
        out["cpu_baseline"] = cpu_baseline(inp, alg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
