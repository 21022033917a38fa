"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one pass of the whole path over one batch: kv_store of the step's new rows, EXTEND
of the prefill chunk, DECODE of the running requests, all on one stream, inputs resident in
HBM. Default workload: the long-context step (one EXTEND of 8,192 new tokens on a
65,536-token cached prefix plus 8 decode requests with 32,768..131,072 tokens of context,
64 q / 8 kv heads, head_dim 128, bf16, values N(0, 0.5), a 2,097,152-slot pool of 4 GiB per
K and V), the largest workload, which exercises every call. ``--config 4`` is the mixed
chunked-prefill batch (a 2,048-token chunk on a 14,336-token prefix plus 128 decode requests
of 1,024..8,192 tokens, 32 q / 8 kv heads, a 1,048,576-slot pool); ``--config 2`` and ``3``
the 64-request decode batch and the shared-prefix EXTEND.
``--kv fp8`` runs the same step over FP8 E4M3 pools (kv_store_fp8, extend_attention_fp8,
decode_attention_fp8; per-pool scales 4 sigma / 448), the pools converted from the bf16 ones
before timing. ``--ragged`` runs EXTEND on the ragged path: the suffix K/V read from the new
rows and stored by the same kernel (extend_attention_ragged with store_loc); kv_store then
writes only the decode requests' current tokens. ``--page-size P`` draws the workload with
pages of P slots and runs EXTEND and DECODE through the page table (the _paged calls; with
``--kv fp8`` the _paged_fp8 calls).
``--cold`` sweeps a 1 GiB buffer (read and write, four times the 256 MB last-level cache)
before every step, outside the kernels' event windows, so the per-kernel figures are
cold-cache ones; ms_per_step then includes the sweeps.

Prints ONE JSON line. ``value`` is the EXTEND attention throughput in TFLOP/s (algorithmic
FLOPs: 4 * head_dim * q_heads per attended pair, masked pairs not counted); the DECODE KV
bandwidth is reported beside it (workloads without EXTEND report it as ``value``). Per-kernel
durations come from HIP events recorded on the launch stream around each call over the timed
steps. ``cpu_baseline`` is the float64 oracle timed on a bounded sample of the same workload
in worker processes on the host's cores (see CpuOracle).
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
# --pmc-summary, per (workload id, KV pool element); each was counted on that workload's timing
# seed with the token table, the pool-reading EXTEND and warm caches. A kernel's figure is used
# only while its sources hash to what they were when the counters were taken.
TRAFFIC_SUMMARIES = {
    (2, "bf16"): "decode_64req_hbm_traffic.txt",
    (3, "bf16"): "shared_prefix_hbm_traffic.txt",
    (4, "bf16"): "mixed_chunk_hbm_traffic.txt",
    (4, "fp8"): "mixed_chunk_fp8_hbm_traffic.txt",
    (5, "bf16"): "long_context_hbm_traffic.txt",
}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", TRAFFIC_SUMMARIES[(4, "bf16")])
CSRC = os.path.join(ROOT, "prefix_cached_paged_amd", "csrc")
KERNEL_SOURCES = {
    "extend_kernel": ["extend_attn_kernel.h", "rax_device.h", "rax_launch.h"],
    "decode_split_kernel": ["decode_attn.hip", "rax_device.h", "rax_launch.h"],
    "decode_merge_kernel": ["decode_attn.hip", "rax_device.h", "rax_launch.h"],
    "decode_plan_kernel": ["decode_attn.hip", "rax_device.h", "rax_launch.h"],
    "kv_store_kernel": ["kv_store.hip", "rax_launch.h"],
    "kv_store_fp8_kernel": ["kv_store.hip", "rax_launch.h"],
}
COPY_BYTES = 1 << 30


def source_sha(kernel: str) -> str:
    """Hash of the kernel's sources with comments and blank lines removed (an edit of a comment
    does not change the kernel the counters were taken on), and of the compiler flags."""
    import hashlib
    import re
    from prefix_cached_paged_amd.build import HIPCC_FLAGS
    h = hashlib.sha256()
    h.update(" ".join(f for f in HIPCC_FLAGS if os.sep not in f).encode())
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


def cpu_model() -> str:
    """The host CPU's model name (what lscpu prints as "Model name")."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers() -> tuple[int, int]:
    """(workers, affinity CPUs): one worker process per CPU this process may run on, capped by
    the OMP_NUM_THREADS share when the environment sets one (the host's share for one GPU)."""
    aff = len(os.sched_getaffinity(0))
    n = aff
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n), aff


# What the forked oracle workers read (copy-on-write from the parent): workload, stored pools,
# scales. Set before the pool is forked.
_CPU = {}


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limit"] = threadpool_limits(1)   # one BLAS thread per worker process


def _cpu_call(kind, idx, g):
    import oracle
    wl, kp, vp, ks, vs = _CPU["wl"], _CPU["kp"], _CPU["vp"], _CPU["ks"], _CPU["vs"]
    spec = wl.spec
    if kind == "extend":
        e = wl.extend
        return oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                       e.extend_lens, e.extend_start_loc, spec.n_kv_heads, wl.sm_scale,
                                       tokens=idx, k_scale=ks, v_scale=vs, kv_heads=[g])
    d = wl.decode
    return oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                   spec.n_kv_heads, wl.sm_scale, requests=idx, k_scale=ks, v_scale=vs,
                                   kv_heads=[g])


def _cpu_task(task):
    kind, idx, g = task
    G = _CPU["wl"].spec.n_q_heads // _CPU["wl"].spec.n_kv_heads
    out = _cpu_call(kind, idx, g)
    return kind, idx, g, out[:, g * G:(g + 1) * G]


class CpuOracle:
    """The float64 oracle, as it stands, timed on the host's cores beside the GPU.

    Work is split into (rows or request, kv head) units run by a pool of worker processes, one
    BLAS thread each. The pool is forked before the GPU is initialised (the workers share the
    workload copy-on-write and never touch the GPU). A short single-thread calibration sizes a
    bounded sample of the same workload so that each call's sample takes about half of
    ``budget_s`` of wall time on the pool: EXTEND the last suffix rows (they see the most keys),
    DECODE whole requests in order. ``kv8 = (k_scale, v_scale)``: FP8 pools; the oracle then
    builds its own E4M3 rows of the sample from the generator's bf16 rows (not timed) and stores
    the step's new rows with its kv_store_fp8.
    """

    def __init__(self, wl, budget_s: float, kv8=None):
        import multiprocessing as mp

        import oracle
        from threadpoolctl import threadpool_limits
        from prefix_cached_paged_amd import accounting as A

        self.wl, self.spec = wl, wl.spec
        self.kv8 = kv8
        spec = self.spec
        t0 = time.perf_counter()
        if kv8 is None:
            ks = vs = 1.0
            self.eb = spec.elem_bytes
            kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)
            prep = lambda rows: None
        else:
            ks, vs = kv8
            self.eb = 1
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
        self.t_store = time.perf_counter() - t0
        _CPU.update(wl=wl, kp=kp, vp=vp, ks=ks, vs=vs)
        self.workers, self.affinity = cpu_workers()
        wall = budget_s / 2
        Hkv, Hq, D = spec.n_kv_heads, spec.n_q_heads, spec.head_dim
        self.plan = {}

        def timed(kind, idx):       # best of two single-thread calls on kv head 0
            best = float("inf")
            for _ in range(2):
                t = time.perf_counter()
                _cpu_call(kind, idx, 0)
                best = min(best, time.perf_counter() - t)
            return best

        self.wall = wall
        with threadpool_limits(1):
            if wl.extend is not None:
                e = wl.extend
                order = sorted(range(e.batch), key=lambda b: -int(e.extend_lens[b]))
                order = [b for b in order if int(e.extend_lens[b]) > 0]
                for b in order:     # FP8: every row a sampled EXTEND row may read, before the fork
                    prep(wl.req_to_token[int(e.req_pool_indices[b]), :int(e.prefix_lens[b]) + int(e.extend_lens[b])])
                # candidate rows, most keys first: the last rows of each request, request after request
                self.ext_rows = [(int(e.extend_start_loc[b]) + i, 4 * D * Hq * (int(e.prefix_lens[b]) + i + 1))
                                 for b in order for i in range(int(e.extend_lens[b]) - 1, -1, -1)]
                tok, fl = self.ext_rows[0]
                rate = fl / Hkv / timed("extend", [tok])
                self.plan["extend"] = self._extend_plan(rate * self.workers * wall)
            if wl.decode is not None:
                d = wl.decode
                for b in range(d.batch):
                    prep(wl.req_to_token[int(d.req_pool_indices[b]), :int(d.seq_lens[b])])
                rate = A.decode_kv_bytes(d.seq_lens[:1], 1, D, self.eb) / timed("decode", [0])
                self.plan["decode"] = self._decode_plan(rate * self.workers * wall)
            # fork the workers now, before anything initialises the GPU in this process
            self.pool = mp.get_context("fork").Pool(self.workers, initializer=_cpu_worker_init)

    def _extend_plan(self, target_flops):
        """Tasks, FLOPs, row count and rows of an EXTEND sample of about target_flops."""
        Hkv = self.spec.n_kv_heads
        toks, flops = [], 0
        for tok, fl in self.ext_rows:
            if flops >= target_flops:
                break
            toks.append(tok)
            flops += fl
        chunks = max(1, min(len(toks), -(-2 * self.workers // Hkv)))
        parts = [sorted(toks[c::chunks]) for c in range(chunks)]
        return [("extend", part, g) for part in parts for g in range(Hkv)], flops, len(toks), sorted(toks)

    def _decode_plan(self, target_bytes):
        """Tasks, KV bytes, request count and requests of a DECODE sample of about target_bytes."""
        from prefix_cached_paged_amd import accounting as A
        d, Hkv, D = self.wl.decode, self.spec.n_kv_heads, self.spec.head_dim
        reqs, nbytes = [], 0
        for b in range(d.batch):
            if nbytes >= target_bytes:
                break
            reqs.append(b)
            nbytes += A.decode_kv_bytes(d.seq_lens[b:b + 1], Hkv, D, self.eb)
        return [("decode", [b], g) for b in reqs for g in range(Hkv)], nbytes, len(reqs), reqs

    def run(self, dev_outs) -> dict:
        from prefix_cached_paged_amd.device import to_host_bits
        import oracle

        spec = self.spec
        G = spec.n_q_heads // spec.n_kv_heads
        res, parity = {}, {}
        for kind in ("extend", "decode"):
            if kind not in self.plan:
                continue
            # The calibration was one single-thread call; the first pool run measures the real
            # rate, and a sample far below the wall-time target is grown from it and run again
            # (only the last run is reported). A DECODE sample that is the whole batch is
            # repeated until the runs add up to the target, and their mean is reported.
            tasks, work, count, idx = self.plan[kind]
            runs = []
            while True:
                t0 = time.perf_counter()
                outs = list(self.pool.imap_unordered(_cpu_task, tasks))
                runs.append(time.perf_counter() - t0)
                grow = self.wall / runs[-1]
                if kind == "extend" and grow > 2 and count < len(self.ext_rows) and len(runs) == 1:
                    tasks, work, count, idx = self._extend_plan(work * grow * 0.9)
                    runs = []
                    continue
                if kind == "decode" and grow > 2 and count < self.wl.decode.batch and len(runs) == 1:
                    tasks, work, count, idx = self._decode_plan(work * grow * 0.9)
                    runs = []
                    continue
                if kind == "decode" and count == self.wl.decode.batch and sum(runs) < self.wall and len(runs) < 20:
                    continue
                break
            wall = float(np.mean(runs))
            got = oracle.to_f64(to_host_bits(dev_outs[kind][idx]))
            pos = {t: i for i, t in enumerate(idx)}
            err = 0.0
            for _, part, g, ref in outs:
                rows = [pos[t] for t in part]
                err = max(err, float(np.max(np.abs(got[rows, g * G:(g + 1) * G] - ref))))
            parity[f"{kind}_max_abs"] = err
            if kind == "extend":
                res[kind] = dict(tflops=work / wall / 1e12, tokens=count, seconds=wall, runs=len(runs))
            else:
                res[kind] = dict(GBps=work / wall / 1e9, requests=count, seconds=wall, runs=len(runs))
        sample = []
        if "extend" in res:
            sample.append(f"EXTEND: last {res['extend']['tokens']} suffix rows, all heads "
                          f"({res['extend']['seconds']:.1f} s wall)")
        if "decode" in res:
            sample.append(f"DECODE: {res['decode']['requests']} of {self.wl.decode.batch} requests, all heads "
                          f"({res['decode']['seconds']:.2f} s wall, mean of {res['decode']['runs']} runs)")
        store_note = (f"kv_store copy {self.t_store:.1f} s not counted" if self.kv8 is None else
                      f"kv_store_fp8 {self.t_store:.1f} s and the E4M3 conversion of the sampled rows not counted")
        return dict(value=res.get("extend", {}).get("tflops"), unit="TFLOP/s", cores=self.workers, kind="oracle",
                    sample="; ".join(sample) + f"; float64 numpy in {self.workers} worker processes over "
                    f"(rows or request, kv head), one BLAS thread each; {store_note}",
                    cpu_model=cpu_model(), affinity_cpus=self.affinity,
                    decode_GBps=res.get("decode", {}).get("GBps"), parity_vs_gpu=parity)

    def close(self):
        self.pool.terminate()
        self.pool.join()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload id (1..5; 6: 100 new tokens on a 10,000-token prefix)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=16.0,
                    help="seconds of wall time for the CPU oracle's samples (about half per call)")
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
    from prefix_cached_paged_amd import workloads as W

    cfg = args.config
    spec = W.workload_spec(cfg)
    if args.page_size != 1:
        import dataclasses
        spec = dataclasses.replace(spec, page_size=args.page_size)
    kv8 = args.kv == "fp8"
    paged = args.page_size != 1
    if paged and args.ragged:
        print("--ragged reads the prefix through a token table (no --page-size)", file=sys.stderr)
        sys.exit(2)
    if args.ragged and kv8:
        print("--ragged is for bf16/fp32 pools", file=sys.stderr)
        sys.exit(2)
    if kv8 and spec.dtype != "bf16":
        print("--kv fp8 needs a bf16 workload (--config 2 to 5)", file=sys.stderr)
        sys.exit(2)
    # FP8 pools: scales put about 4 standard deviations at the top of E4M3.
    k_scale = v_scale = 4.0 * spec.sigma / 448.0 if kv8 else 1.0
    seed = args.seed if args.seed is not None else W.TIMING_SEEDS[cfg]
    log(f"generating workload {spec.name} seed {seed}")
    wl = W.make_workload(spec, seed)

    # The CPU oracle's worker processes are forked here, before this process touches the GPU.
    cpu_oracle = None
    if not args.no_cpu_baseline:
        log("preparing the CPU oracle (store, calibration, worker pool)")
        cpu_oracle = CpuOracle(wl, args.cpu_budget, kv8=(k_scale, v_scale) if kv8 else None)

    from prefix_cached_paged_amd import rax
    from prefix_cached_paged_amd.device import upload

    rax.load()  # fails loudly if the HIP library is missing
    log("uploading")
    dw = upload(wl, "cuda:0")
    dt = rax.BF16 if spec.dtype == "bf16" else rax.FP32
    rag = args.ragged and dw.ext is not None
    pt = torch.from_numpy(wl.page_table).to("cuda:0") if paged else None
    n_ext = wl.extend.total_tokens if wl.extend is not None else 0
    ws = None
    if dw.dec is not None:
        d = dw.dec
        nb = rax.decode_workspace_bytes(rax.FP8_E4M3 if kv8 else dt, d["q"].shape[0], d["max_seq_len"],
                                        spec.n_q_heads, spec.n_kv_heads, spec.head_dim)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")
    if kv8:
        # FP8 pools converted from the bf16 ones by the library's store (set-up, not timed); the
        # bf16 pools are freed.
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
            if kv8 and paged:
                rax.extend_attention_paged_fp8(e["q"], e["o"], dw.k_pool, dw.v_pool, pt, args.page_size, *ea[5:],
                                               k_scale, v_scale)
            elif kv8:
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
            if kv8 and paged:
                rax.decode_attention_paged_fp8(d["q"], d["o"], dw.k_pool, dw.v_pool, pt, args.page_size, *da[5:],
                                               k_scale, v_scale, workspace=ws)
            elif kv8:
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
    # A traffic summary counts only for the run it was taken on (its workload with the timing
    # seed; token table, pool-reading EXTEND, warm caches, the same pool element); graph replay
    # runs the same kernels on the same data. Any other workload or mode: null.
    summary = TRAFFIC_SUMMARIES.get((cfg, "fp8" if kv8 else spec.dtype))
    counted = (summary is not None and seed == W.TIMING_SEEDS[cfg] and not rag and not paged and not args.cold)
    traffic = read_traffic(os.path.join(ROOT, "profiles", summary)) if counted else {}
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
    if cpu_oracle is not None:
        log(f"timing the CPU oracle on a sample ({cpu_oracle.workers} worker processes)")
        outs = {}
        if dw.ext is not None:
            outs["extend"] = dw.ext["o"]
        if dw.dec is not None:
            outs["decode"] = dw.dec["o"]
        try:
            cpu = cpu_oracle.run(outs)
        finally:
            cpu_oracle.close()
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
