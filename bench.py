"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one pass of the whole path over one batch: kv_store of the step's new rows, EXTEND
of the prefill chunk, DECODE of the running requests, all on one stream, inputs resident in
HBM. Default workload: the mixed chunked-prefill batch (one 2,048-token chunk on a
14,336-token cached prefix plus 128 decode requests with 1,024..8,192 tokens of context,
32 q / 8 kv heads, head_dim 128, bf16, a 1,048,576-slot pool), which exercises every call.
``--kv fp8`` runs the same step over FP8 E4M3 pools (kv_store_fp8, extend_attention_fp8,
decode_attention_fp8; per-pool scales 4 sigma / 448), the pools converted from the bf16 ones
before timing. ``--ragged`` runs EXTEND on the ragged path: the suffix K/V read from the new
rows and stored by the same kernel (extend_attention_ragged with store_loc); kv_store then
writes only the decode requests' current tokens. ``--page-size P`` draws the workload with
pages of P slots and runs EXTEND and DECODE through the page table (the _paged calls).
``--cold`` sweeps a 1 GiB buffer (read and write, four times the 256 MB last-level cache)
before every step, outside the kernels' event windows, so the per-kernel figures are
cold-cache ones; ms_per_step then includes the sweeps.

Prints ONE JSON line. ``value`` is the EXTEND attention throughput in TFLOP/s (algorithmic
FLOPs: 4 * head_dim * q_heads per attended pair, masked pairs not counted); the DECODE KV
bandwidth is reported beside it. Per-kernel durations come from HIP events recorded on the
launch stream around each call over the timed steps.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "extend attn TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# HBM traffic per dispatch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs summarised by
# --pmc-summary. A kernel's figure is used only while its sources hash to what they were when
# the counters were taken.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "mixed_chunk_hbm_traffic.txt")
TRAFFIC_SUMMARY_FP8 = os.path.join(ROOT, "profiles", "mixed_chunk_fp8_hbm_traffic.txt")
CSRC = os.path.join(ROOT, "prefix_cached_paged_amd", "csrc")
KERNEL_SOURCES = {
    "extend_kernel": ["extend_attn.hip", "rax_device.h", "rax_launch.h"],
    "decode_split_kernel": ["decode_attn.hip", "rax_device.h", "rax_launch.h"],
    "decode_merge_kernel": ["decode_attn.hip", "rax_device.h", "rax_launch.h"],
    "decode_plan_kernel": ["decode_attn.hip", "rax_device.h", "rax_launch.h"],
    "kv_store_kernel": ["kv_store.hip", "rax_launch.h"],
    "kv_store_fp8_kernel": ["kv_store.hip", "rax_launch.h"],
}
COPY_BYTES = 1 << 30


def source_sha(kernel: str) -> str:
    """Hash of the kernel's sources with comments and blank lines removed (an edit of a comment
    does not change the kernel the counters were taken on)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def read_traffic(path: str = TRAFFIC_SUMMARY) -> dict:
    """kernel -> HBM bytes per dispatch, for kernels whose sources are unchanged."""
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        if not line.startswith("kernel="):
            continue
        kv = dict(f.split("=", 1) for f in line.split())
        k = kv["kernel"]
        if k in KERNEL_SOURCES and kv.get("source_sha") == source_sha(k):
            out[k] = int(float(kv["hbm_bytes"]))
    return out


def pmc_summary(out_path: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                command: str):
    """Write the traffic summary from four rocprofv3 --pmc output folders (FETCH_SIZE and
    WRITE_SIZE for the benchmark, the same two for --copy-calibration)."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"].split("(")[0].split("<")[0].split("::")[-1], []).append(
                        float(r["Counter_Value"]))
        # median over dispatches: a set-up dispatch of another size (the FP8 mode converts the
        # whole pool once with the store kernel) does not move the per-step figure
        return {k: (float(np.median(v)), len(v)) for k, v in vals.items()}

    def copy_kib(d, counter):
        best = 0.0
        for k, (v, n) in per_kernel(d, counter).items():
            if "copy" in k.lower() or "elementwise" in k.lower():
                best = max(best, v)
        return best

    cf, cw = copy_kib(copy_fetch_dir, "FETCH_SIZE"), copy_kib(copy_write_dir, "WRITE_SIZE")
    f_fac = COPY_BYTES / 1024 / cf
    w_fac = COPY_BYTES / 1024 / cw
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc), MI355X", "#",
             "# Each counter is scaled by what it reads for a plain device copy of 1 GiB",
             "# (bench.py --copy-calibration): bytes = KiB * 1024 * factor. Per kernel: the median",
             "# over its dispatches.", "#",
             "# Commands (from the repository root, TMPDIR=/tmp):"]
    lines += ["#   " + c for c in command.split(" ;; ")]
    lines += ["#", f"calibration copy_bytes={COPY_BYTES} copy_fetch_kib={cf:.1f} copy_write_kib={cw:.1f} "
              f"fetch_factor={f_fac:.4f} write_factor={w_fac:.4f}"]
    for k in sorted(set(fetch) & set(write)):
        if k not in KERNEL_SOURCES:
            continue
        fk, n = fetch[k]
        wk, _ = write[k]
        hbm = fk * 1024 * f_fac + wk * 1024 * w_fac
        lines.append(f"kernel={k} dispatches={n} fetch_kib={fk:.1f} write_kib={wk:.1f} "
                     f"fetch_bytes={fk * 1024 * f_fac:.0f} write_bytes={wk * 1024 * w_fac:.0f} "
                     f"hbm_bytes={hbm:.0f} source_sha={source_sha(k)}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_calibration():
    """A plain device copy of COPY_BYTES, three times: the reference for the PMC byte counters."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied 3 x {COPY_BYTES} bytes", flush=True)


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(wl, dev_outs, budget_s: float, kv8=None):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload.

    ``kv8 = (k_scale, v_scale)``: FP8 pools. The oracle then builds its own E4M3 pools from the
    generator's bf16 rows (only the rows the sample reads, converted before each timed call and
    not timed) and stores the step's new rows with its kv_store_fp8."""
    import oracle
    from threadpoolctl import threadpool_info
    from prefix_cached_paged_amd import accounting as A
    from prefix_cached_paged_amd.device import to_host_bits

    spec = wl.spec
    t0 = time.perf_counter()
    if kv8 is None:
        ks = vs = 1.0
        eb = spec.elem_bytes
        kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)
        prep = lambda rows: None
    else:
        ks, vs = kv8
        eb = 1
        kp = np.full(wl.k_pool.shape, 0x7F, np.uint8)     # E4M3 NaN until a row is converted
        vp = np.full(wl.v_pool.shape, 0x7F, np.uint8)
        kp, vp = oracle.kv_store_fp8(kp, vp, wl.k_new, wl.v_new, wl.store_loc, ks, vs)
        done = np.zeros(kp.shape[0], bool)
        done[np.asarray(wl.store_loc, np.int64)] = True

        def prep(rows):
            rows = np.unique(np.asarray(rows, np.int64))
            rows = rows[~done[rows]]
            kp[rows] = oracle.quantize_bf16(wl.k_pool[rows], ks)
            vp[rows] = oracle.quantize_bf16(wl.v_pool[rows], vs)
            done[rows] = True
    t_store = time.perf_counter() - t0
    res = {}
    parity = {}
    if wl.extend is not None:
        e = wl.extend
        b = int(np.argmax(e.extend_lens))
        n = int(e.extend_lens[b])
        s0 = int(e.extend_start_loc[b])
        # last rows first: they see the most keys; grow the sample until about half the budget
        toks, flops, t_ext = [], 0, 0.0
        step = 8
        while t_ext < budget_s / 2 and len(toks) < n:
            new = [s0 + n - 1 - i for i in range(len(toks), min(n, len(toks) + step))]
            prep(wl.req_to_token[int(e.req_pool_indices[b]), :int(e.prefix_lens[b]) + n])
            t1 = time.perf_counter()
            ref = oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                          e.extend_lens, e.extend_start_loc, spec.n_kv_heads, wl.sm_scale,
                                          tokens=new, k_scale=ks, v_scale=vs)
            t_ext += time.perf_counter() - t1
            p = int(e.prefix_lens[b])
            flops += sum(4 * spec.head_dim * spec.n_q_heads * (p + (t - s0) + 1) for t in new)
            got = oracle.to_f64(to_host_bits(dev_outs["extend"][new]))
            parity.setdefault("extend_max_abs", 0.0)
            parity["extend_max_abs"] = max(parity["extend_max_abs"], float(np.max(np.abs(got - ref))))
            toks += new
            step *= 2
        res["extend"] = dict(tflops=flops / t_ext / 1e12, tokens=len(toks), seconds=t_ext)
    if wl.decode is not None:
        d = wl.decode
        reqs, nbytes, t_dec = [], 0, 0.0
        order = list(range(d.batch))
        while t_dec < budget_s / 2 and len(reqs) < d.batch:
            new = order[len(reqs):len(reqs) + max(1, len(reqs))]
            if kv8 is not None:
                prep(np.concatenate([wl.req_to_token[int(d.req_pool_indices[r]), :int(d.seq_lens[r])] for r in new]))
            t1 = time.perf_counter()
            ref = oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                          spec.n_kv_heads, wl.sm_scale, requests=new, k_scale=ks, v_scale=vs)
            t_dec += time.perf_counter() - t1
            nbytes += A.decode_kv_bytes(d.seq_lens[new], spec.n_kv_heads, spec.head_dim, eb)
            got = oracle.to_f64(to_host_bits(dev_outs["decode"][new]))
            parity.setdefault("decode_max_abs", 0.0)
            parity["decode_max_abs"] = max(parity["decode_max_abs"], float(np.max(np.abs(got - ref))))
            reqs += new
        res["decode"] = dict(GBps=nbytes / t_dec / 1e9, requests=len(reqs), seconds=t_dec)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    sample = []
    if "extend" in res:
        sample.append(f"EXTEND: last {res['extend']['tokens']} suffix rows of the chunk, all heads")
    if "decode" in res:
        sample.append(f"DECODE: {res['decode']['requests']} of {wl.decode.batch} requests, all heads")
    store_note = (f"kv_store copy {t_store:.1f} s not counted" if kv8 is None else
                  f"kv_store_fp8 {t_store:.1f} s and the E4M3 conversion of the sampled rows not counted")
    out = dict(value=res.get("extend", {}).get("tflops"), unit="TFLOP/s", cores=threads, kind="oracle",
               sample="; ".join(sample) + f"; float64 numpy, {store_note}",
               decode_GBps=res.get("decode", {}).get("GBps"), parity_vs_gpu=parity)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="workload id (1..5)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=16.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="KV pool element: the workload's bf16, or FP8 E4M3 with per-pool scales")
    ap.add_argument("--ragged", action="store_true",
                    help="EXTEND via extend_attention_ragged with the fused store of the suffix rows")
    ap.add_argument("--page-size", type=int, default=1,
                    help="pool pages of this many slots, read through a page table (1 = token table)")
    ap.add_argument("--cold", action="store_true",
                    help="sweep 1 GiB through the caches before every step (per-kernel times are then cold)")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip timing a plain bf16 GEMM (torch.matmul) and a torch gather of the DECODE rows "
                         "as the box's practical MFMA and gather ceilings")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step as HIP graph replays (reported beside the eager figures)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for the PMC byte counters)")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("OUT", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                       "COPY_WRITE_DIR"),
                    help="write the HBM traffic summary from rocprofv3 --pmc output folders and exit")
    ap.add_argument("--pmc-command", default="", help="command text recorded in the traffic summary")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, command=args.pmc_command)
        return
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: librax has no multi-GPU path; rerun with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from prefix_cached_paged_amd import accounting as A
    from prefix_cached_paged_amd import rax
    from prefix_cached_paged_amd import workloads as W
    from prefix_cached_paged_amd.device import upload

    rax.load()  # fails loudly if the HIP library is missing
    cfg = args.config
    spec = W.CONFIGS[cfg]
    if args.page_size != 1:
        import dataclasses
        spec = dataclasses.replace(spec, page_size=args.page_size)
    seed = args.seed if args.seed is not None else W.TIMING_SEEDS[cfg]
    log(f"generating workload {spec.name} seed {seed}")
    wl = W.make_workload(spec, seed)
    log("uploading")
    dw = upload(wl, "cuda:0")
    dt = rax.BF16 if spec.dtype == "bf16" else rax.FP32
    kv8 = args.kv == "fp8"
    rag = args.ragged and dw.ext is not None
    paged = args.page_size != 1
    if paged and (kv8 or rag):
        print("--page-size runs the bf16/fp32 pool path only", file=sys.stderr)
        sys.exit(2)
    pt = torch.from_numpy(wl.page_table).to("cuda:0") if paged else None
    if rag and kv8:
        print("--ragged is for bf16/fp32 pools", file=sys.stderr)
        sys.exit(2)
    n_ext = wl.extend.total_tokens if wl.extend is not None else 0
    if kv8 and spec.dtype != "bf16":
        print("--kv fp8 needs a bf16 workload (--config 2 to 5)", file=sys.stderr)
        sys.exit(2)
    ws = None
    if dw.dec is not None:
        d = dw.dec
        nb = rax.decode_workspace_bytes(rax.FP8_E4M3 if kv8 else dt, d["q"].shape[0], d["max_seq_len"],
                                        spec.n_q_heads, spec.n_kv_heads, spec.head_dim)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")
    k_scale = v_scale = 1.0
    if kv8:
        # FP8 pools converted from the bf16 ones by the library's store (set-up, not timed); the
        # bf16 pools are freed. Scales put about 4 standard deviations at the top of E4M3.
        k_scale = v_scale = 4.0 * spec.sigma / 448.0
        log("converting the pools to FP8 E4M3")
        kp8 = torch.empty(dw.k_pool.shape, dtype=torch.uint8, device="cuda:0")
        vp8 = torch.empty_like(kp8)
        allslots = torch.arange(kp8.shape[0], dtype=torch.int32, device="cuda:0")
        rax.kv_store_fp8(dw.k_pool, dw.v_pool, allslots, kp8, vp8, k_scale, v_scale)
        torch.cuda.synchronize()
        dw.k_pool, dw.v_pool = kp8, vp8
        del allslots
        torch.cuda.empty_cache()

    flush = torch.empty(COPY_BYTES // 2, dtype=torch.uint8, device="cuda:0") if args.cold else None
    flush2 = torch.empty_like(flush) if args.cold else None

    def step(ev=None):
        if flush is not None:
            flush2.copy_(flush)   # 512 MiB read + 512 MiB written: evicts the step's data
        if ev is not None:
            ev[0].record()
        if kv8:
            rax.kv_store_fp8(dw.k_new, dw.v_new, dw.store_loc, dw.k_pool, dw.v_pool, k_scale, v_scale)
        elif rag:
            # the suffix rows (the first n_ext new rows) are stored by the ragged EXTEND
            if dw.store_loc.shape[0] > n_ext:
                rax.kv_store(dw.k_new[n_ext:], dw.v_new[n_ext:], dw.store_loc[n_ext:], dw.k_pool, dw.v_pool)
        else:
            rax.kv_store(dw.k_new, dw.v_new, dw.store_loc, dw.k_pool, dw.v_pool)
        if ev is not None:
            ev[1].record()
        if dw.ext is not None:
            e = dw.ext
            ea = (e["q"], e["o"], dw.k_pool, dw.v_pool, dw.req_to_token, e["req_pool_indices"], e["prefix_lens"],
                  e["extend_lens"], e["extend_start_loc"], e["max_extend_len"], e["max_seq_len"], wl.sm_scale)
            if kv8:
                rax.extend_attention_fp8(*ea, k_scale, v_scale)
            elif rag:
                rax.extend_attention_ragged(e["q"], e["o"], dw.k_new[:n_ext], dw.v_new[:n_ext], dw.k_pool,
                                            dw.v_pool, *ea[4:], store_loc=dw.store_loc[:n_ext])
            elif paged:
                rax.extend_attention_paged(e["q"], e["o"], dw.k_pool, dw.v_pool, pt, args.page_size, *ea[5:])
            else:
                rax.extend_attention(*ea)
        if ev is not None:
            ev[2].record()
        if dw.dec is not None:
            d = dw.dec
            da = (d["q"], d["o"], dw.k_pool, dw.v_pool, dw.req_to_token, d["req_pool_indices"], d["seq_lens"],
                  d["max_seq_len"], wl.sm_scale)
            if kv8:
                rax.decode_attention_fp8(*da, k_scale, v_scale, workspace=ws)
            elif paged:
                rax.decode_attention_paged(d["q"], d["o"], dw.k_pool, dw.v_pool, pt, args.page_size, *da[5:],
                                           workspace=ws)
            else:
                rax.decode_attention(*da, workspace=ws)
        if ev is not None:
            ev[3].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    per_step = {n: [evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]
                for i, n in enumerate(["kv_store", "extend", "decode"])}
    ms = {n: float(np.mean(v)) for n, v in per_step.items()}
    spread = {n: dict(median=float(np.median(v)), p10=float(np.percentile(v, 10)), p90=float(np.percentile(v, 90)))
              for n, v in per_step.items()}

    graph = None
    if args.graph:
        log("capturing one step in a HIP graph")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gev[0].record()
        for _ in range(args.steps):
            g.replay()
        gev[1].record()
        torch.cuda.synchronize()
        graph = dict(ms_per_step=gev[0].elapsed_time(gev[1]) / args.steps,
                     eager_event_ms_per_step=sum(ms.values()))

    mfma_ceiling = None
    if not args.no_mfma_ceiling and dw.ext is not None:
        # A large bf16 GEMM (hipBLASLt through torch.matmul, contiguous 2-D operands): what a
        # library contraction reaches on this machine, at the clock sustained MFMA load runs at. Shown
        # beside the EXTEND figure; the roofline fraction stays against the published peak.
        n = 8192
        a_ = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
        b_ = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(a_, b_)
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gev[0].record()
        for _ in range(10):
            torch.matmul(a_, b_)
        gev[1].record()
        torch.cuda.synchronize()
        gms = gev[0].elapsed_time(gev[1]) / 10
        mfma_ceiling = dict(kind="torch.matmul bf16 8192x8192x8192 (hipBLASLt)", ms=gms,
                            tflops=2 * n ** 3 / (gms * 1e-3) / 1e12)
        del a_, b_

    gather_ceiling = None
    if not args.no_mfma_ceiling and dw.dec is not None and not kv8 and not paged:
        # The DECODE call's K and V rows gathered by slot with torch.index_select (a library
        # gather-copy of the same random rows): its read rate is comparable to the DECODE KV GB/s.
        d = wl.decode
        rows = np.concatenate([wl.req_to_token[r, :L] for r, L in zip(d.req_pool_indices, d.seq_lens)])
        slots = torch.from_numpy(rows.astype(np.int64)).to("cuda:0")
        kf = dw.k_pool.view(dw.k_pool.shape[0], -1)
        vf = dw.v_pool.view(dw.v_pool.shape[0], -1)
        for _ in range(2):
            gk, gv = torch.index_select(kf, 0, slots), torch.index_select(vf, 0, slots)
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gev[0].record()
        for _ in range(5):
            torch.index_select(kf, 0, slots, out=gk)
            torch.index_select(vf, 0, slots, out=gv)
        gev[1].record()
        torch.cuda.synchronize()
        gms = gev[0].elapsed_time(gev[1]) / 5
        nb = 2 * gk.numel() * gk.element_size()
        gather_ceiling = dict(kind="torch.index_select of the DECODE call's K and V rows", ms=gms,
                              read_GBps=nb / (gms * 1e-3) / 1e9, read_plus_write_GBps=2 * nb / (gms * 1e-3) / 1e9)
        del gk, gv, slots

    report = {}
    hbm = lambda nbytes, t_ms: nbytes / (t_ms * 1e-3) / 1e9
    n_new = int(wl.store_loc.size) - (n_ext if rag else 0)
    pool_eb = 1 if kv8 else spec.elem_bytes
    # bf16 store: read and write s bytes per element; FP8 store: read 2, write 1
    st_bytes = (A.kv_store_bytes(n_new, spec.n_kv_heads, spec.head_dim, spec.elem_bytes) if not kv8 else
                n_new * 2 * spec.n_kv_heads * spec.head_dim * 3 + 4 * n_new)
    report["kv_store"] = dict(ms=ms["kv_store"], ms_spread=spread["kv_store"], rows=n_new,
                              GBps=hbm(st_bytes, ms["kv_store"]),
                              bytes=st_bytes)
    roofs = {}
    # The traffic summaries were counted on the default step (the mixed chunked-prefill batch,
    # --config 4, with its timing seed; token table, pool-reading EXTEND, warm caches) over bf16
    # or FP8 pools; graph replay runs the same kernels on the same data. Any other workload or
    # mode has no counted traffic: null.
    counted = cfg == 4 and seed == W.TIMING_SEEDS[4] and not rag and not paged and not args.cold
    traffic = read_traffic(TRAFFIC_SUMMARY_FP8 if kv8 else TRAFFIC_SUMMARY) if counted else {}
    if wl.extend is not None:
        e = wl.extend
        fl = A.extend_flops(e.prefix_lens, e.extend_lens, spec.n_q_heads, spec.head_dim)
        tf = fl / (ms["extend"] * 1e-3) / 1e12
        report["extend"] = dict(ms=ms["extend"], ms_spread=spread["extend"], flops=fl, tflops=tf,
                                frac=tf / PEAK_BF16_TFLOPS)
        roofs["extend"] = dict(kernel="extend_attention_ragged (fused store)" if rag else "extend_attention",
                               bound="mfma", achieved=tf, peak=PEAK_BF16_TFLOPS,
                               unit="TFLOP/s", frac=tf / PEAK_BF16_TFLOPS,
                               traffic=traffic.get("extend_kernel"),
                               per_launch=f"{fl} algorithmic FLOP", ms=ms["extend"])
    if wl.decode is not None:
        d = wl.decode
        kvb = A.decode_kv_bytes(d.seq_lens, spec.n_kv_heads, spec.head_dim, pool_eb)
        tot = A.decode_total_bytes(d.seq_lens, d.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                                   pool_eb) if not kv8 else (
            kvb + 4 * int(np.sum(d.seq_lens)) + 2 * d.batch * spec.n_q_heads * spec.head_dim * 2)
        gb = hbm(kvb, ms["decode"])
        report["decode"] = dict(ms=ms["decode"], ms_spread=spread["decode"], kv_bytes=kvb, kv_GBps=gb, frac=gb / PEAK_HBM_GBPS,
                                total_GBps=hbm(tot, ms["decode"]),
                                splits=rax.decode_num_splits(rax.FP8_E4M3 if kv8 else dt, d.batch, d.max_seq_len,
                                                             spec.n_kv_heads))
        # the plan kernel runs only for batches above 1,024 requests
        dec_kernels = ["decode_split_kernel", "decode_merge_kernel"]
        dec_traffic = (sum(traffic[k] for k in dec_kernels) + traffic.get("decode_plan_kernel", 0)
                       if all(k in traffic for k in dec_kernels) else None)
        roofs["decode"] = dict(kernel="decode_attention (split + merge)", bound="hbm", achieved=gb,
                               peak=PEAK_HBM_GBPS, unit="GB/s", frac=gb / PEAK_HBM_GBPS,
                               traffic=dec_traffic, per_launch=f"{kvb} KV bytes", ms=ms["decode"])
    dominant = max(roofs, key=lambda k: roofs[k]["ms"]) if roofs else None

    if "extend" in report:
        value, unit = report["extend"]["tflops"], "TFLOP/s"
    else:
        value, unit = report["decode"]["kv_GBps"], "GB/s"

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        outs = {}
        if dw.ext is not None:
            outs["extend"] = dw.ext["o"]
        if dw.dec is not None:
            outs["decode"] = dw.dec["o"]
        cpu = cpu_baseline(wl, outs, args.cpu_budget, kv8=(k_scale, v_scale) if kv8 else None)
        if unit == "GB/s":
            cpu["value"], cpu["unit"] = cpu.pop("decode_GBps"), "GB/s"

    cfgd = {"workload": spec.name, "config_id": cfg, "seed": seed, "dtype": spec.dtype,
            "q_heads": spec.n_q_heads, "kv_heads": spec.n_kv_heads, "head_dim": spec.head_dim,
            "pool_slots": spec.num_slots, "kv_pool": "fp8_e4m3" if kv8 else spec.dtype}
    if kv8:
        cfgd["kv_scales"] = [k_scale, v_scale]
    if rag:
        cfgd["extend_path"] = "ragged suffix, fused store"
    if paged:
        cfgd["page_size"] = args.page_size
    if args.cold:
        cfgd["caches"] = "cold: 1 GiB swept before every step"
    if wl.extend is not None:
        cfgd["extend"] = {"batch": wl.extend.batch, "new_tokens": wl.extend.total_tokens,
                          "prefix_lens": sorted(set(int(x) for x in wl.extend.prefix_lens))[:4]}
    if wl.decode is not None:
        cfgd["decode"] = {"batch": wl.decode.batch, "mean_context": float(np.mean(wl.decode.seq_lens)),
                          "total_context": int(np.sum(wl.decode.seq_lens))}
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic", "config": cfgd,
        "kernels": report,
        "roofline": roofs.get(dominant),
        "roofline_other": [roofs[k] for k in roofs if k != dominant],
        "cpu_baseline": cpu,
        "graph": graph,
        "mfma_ceiling": mfma_ceiling,
        "gather_ceiling": gather_ceiling,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
