"""bench.py on the CPU: the one-GPU guard and the traffic-summary reader (no GPU needed)."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_cli_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod   # the CPU oracle's worker tasks are pickled by module name
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_traffic_summaries_parse(tmp_path):
    b = load_bench()
    # a summary whose hashes match nothing yields no figures; a matching one yields bytes
    k = "extend_kernel"
    good = tmp_path / "good.txt"
    good.write_text(f"# header\nkernel={k} dispatches=4 hbm_bytes=1234 source_sha={b.source_sha(k)}\n")
    stale = tmp_path / "stale.txt"
    stale.write_text(f"kernel={k} dispatches=4 hbm_bytes=1234 source_sha=0000000000000000\n")
    assert b.read_traffic(str(good)) == {k: 1234}
    assert b.read_traffic(str(stale)) == {}


def test_cpu_oracle_pool_on_a_small_workload():
    """The CPU baseline's worker pool: every sampled (rows, kv head) unit comes back, the figures
    are positive, and feeding the oracle's own outputs back as the "device" outputs gives zero
    parity error (bf16 rows rounded from the float64 result: at most half a bf16 ulp)."""
    import numpy as np
    import torch

    import oracle
    from prefix_cached_paged_amd import workloads as W
    from prefix_cached_paged_amd.workloads import round_to_bf16_bits

    b = load_bench()
    spec = W.Spec("cpu-pool", "bf16", 8, 2, 64, 4000, extend_prefix=(300, 40), extend_lens=(64, 9),
                  decode_lens=(5, 700, 33))
    wl = W.make_workload(spec, 5)
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)
    e, d = wl.extend, wl.decode
    ref_e = oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens, e.extend_lens,
                                    e.extend_start_loc, 2, wl.sm_scale)
    ref_d = oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens, 2, wl.sm_scale)
    as_bf16 = lambda a: torch.from_numpy(round_to_bf16_bits(a.astype(np.float32)).view(np.int16)).view(torch.bfloat16)
    cpu = b.CpuOracle(wl, budget_s=2.0)
    try:
        assert cpu.workers >= 1 and cpu.affinity >= cpu.workers
        res = cpu.run({"extend": as_bf16(ref_e), "decode": as_bf16(ref_d)})
    finally:
        cpu.close()
    assert res["cores"] == cpu.workers and res["kind"] == "oracle" and res["cpu_model"]
    assert res["value"] > 0 and res["decode_GBps"] > 0
    assert res["parity_vs_gpu"]["extend_max_abs"] <= 2.0 ** -8 * np.abs(ref_e).max()
    assert res["parity_vs_gpu"]["decode_max_abs"] <= 2.0 ** -8 * np.abs(ref_d).max()
