"""Throughput of shared-KV sparse flash MLA attention on one MI355X.

One step is one pass of the whole path on one batch: the plan
(sfmla_metadata), the forward kernel (resolve, gather, QK^T, online softmax,
PV) and the split merge (sfmla_combine), all through the C ABI.  Inputs are
resident in HBM before timing starts.  Between steps the TopK index set is
rotated through several independently drawn replicas, so consecutive steps
gather different rows and the 256 MB Infinity Cache cannot serve them.

Prints one JSON line.  The headline workload is the token-wise sparse
MLA-absorb decode with rope (B=32, q_s=2, q_n=128, d_qk=576, d_v=512, TopK
2048 over a 65536-token paged cache).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "sparse_shared_kv_amd", "csrc", "sfmla_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_kernel_%s.txt")

DESCR = {
    "sfa_mla_rope": "token-wise sparse MLA-absorb decode with rope: B=32, q_s=2, q_n=128, "
                    "d_qk=576 (512+64 rope), separate V (512), TopK 2048 of 65536 cached tokens, "
                    "PA_BSND block 64, bf16",
    "c8_packed_int8": "INT8 per-128-tile packed KV (656-B rows), TND B=8, q_n=128, d_qk=576, "
                      "TopK 2048 of 16K-131K tokens",
    "c8_packed_fp8": "FP8-E4M3 per-128-tile packed KV (656-B rows), TND B=8, q_n=128, d_qk=576, "
                     "TopK 2048 of 16K-131K tokens",
    "hca_varlen": "HCA varlen TND: B=8, q_n=128, window 128 + all visible compressed rows "
                  "(ratio 128), contexts 16K-131K, sinks",
    "csa_decode_paged": "CSA paged decode: B=4, q_n=64, window 128 + TopK 512 of 8192 "
                        "compressed rows (ratio 4), PA block 128, sinks",
    "swa_decode": "SWA decode: B=2, q_n=16, window 128 of 512, BSND",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def row_bytes(P) -> tuple:
    """Bytes of one gathered KV row and flops per (row, head)."""
    p = P.params
    d_qk = 512 + int(p["rope_head_dim"])
    if p["kv_dtype"] == "bf16":
        b = 2 * d_qk + (1024 if p.get("separate_v") else 0)
    else:
        b = 512 + 2 * int(p["rope_head_dim"]) + 16
    return b, 2 * (d_qk + 512)


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source (else None)."""
    path = TRAFFIC_FILE % workload
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(P, flops_per_row, bytes_per_row, budget_s=10.0):
    """The oracle, as it stands, on a bounded sample: passes over the query
    rows (one row per call) until about budget_s of CPU work is done."""
    import numpy as np
    import threadpoolctl

    import oracle
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    rows = list(range(P.query_rows))
    done, t0 = [], time.perf_counter()
    while time.perf_counter() - t0 < budget_s and len(done) < 50 * len(rows):
        r = rows[len(done) % len(rows)]
        oracle.forward(P, rows=[r])
        done.append(r)
    dt = time.perf_counter() - t0
    fl = float(np.sum([flops_per_row[r] for r in done]))
    by = float(np.sum([bytes_per_row[r] for r in done]))
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d query-row calls over the %d query rows (all heads), %.1f s; "
                      "%.3f GB/s gathered KV" % (len(done), len(rows), dt, by / dt / 1e9)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sfa_mla_rope", choices=sorted(DESCR))
    ap.add_argument("--replicas", type=int, default=4,
                    help="index-set replicas rotated between steps (TopK workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_shared_kv_amd as s
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log("[bench] building workload", args.workload)
    P = synth.make_workload(args.workload)
    call = s.Call(P.params, P.arrays, device=dev)
    reps = synth.index_replicas(P, args.replicas - 1) if args.replicas > 1 else []
    idx_sets = []
    if reps:
        name = reps[0][0]
        idx_sets = [call.d[name]] + [torch.from_numpy(a).to(dev) for _, a in reps]
    log("[bench] index replicas:", len(idx_sets) or 1)

    # algorithmic work: resolved rows per query row (from the library's resolver)
    rb, fl_row = row_bytes(P)
    qn = int(P.params["num_heads_q"])
    counts_all = []
    for k in range(max(1, len(idx_sets))):
        if idx_sets:
            setattr(call.tensors, reps[0][0], idx_sets[k].data_ptr())
        call.plan()
        _, counts = call.resolve(1)
        counts_all.append(counts.cpu().numpy().astype(np.int64))
    torch.cuda.synchronize()
    rows_per_step = [int(c.sum()) for c in counts_all]
    flops_step = [n * fl_row * qn for n in rows_per_step]
    bytes_step = [n * rb for n in rows_per_step]

    stream = torch.cuda.current_stream()

    def step(k):
        if idx_sets:
            setattr(call.tensors, reps[0][0], idx_sets[k % len(idx_sets)].data_ptr())
        call.plan()
        call.forward()
        call.combine()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if idx_sets:
            setattr(call.tensors, reps[0][0], idx_sets[k % len(idx_sets)].data_ptr())
        e = ev[k]
        e[0].record(stream)
        call.plan()
        e[1].record(stream)
        call.forward()
        e[2].record(stream)
        call.combine()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(call.status.item()) == 0, "device status %d" % int(call.status.item())

    plan_ms = [e[0].elapsed_time(e[1]) for e in ev]
    fwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    comb_ms = [e[2].elapsed_time(e[3]) for e in ev]
    ms_per_step = wall * 1e3 / args.steps
    nrep = max(1, len(idx_sets))
    tot_flops = sum(flops_step[k % nrep] for k in range(args.steps))
    tot_bytes = sum(bytes_step[k % nrep] for k in range(args.steps))
    tflops = tot_flops / wall / 1e12
    gbps = tot_bytes / wall / 1e9
    fwd_avg_s = float(np.mean(fwd_ms)) / 1e3
    fwd_bytes = float(np.mean([bytes_step[k % nrep] for k in range(args.steps)]))
    fwd_flops = float(np.mean([flops_step[k % nrep] for k in range(args.steps)]))
    intensity = fwd_flops / fwd_bytes
    hbm_bound = intensity < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if hbm_bound:
        achieved, peak, unit = fwd_bytes / fwd_avg_s / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        achieved, peak, unit = fwd_flops / fwd_avg_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = read_traffic(args.workload)

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy probe: %d MiB device copy" % args.copy_probe_mb)

    result = {
        "metric": "decode TFLOP/s + gathered-KV HBM GB/s vs roofline, q_n=128 topk=2048",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": P.params["kv_dtype"] if P.params["kv_dtype"] != "bf16" else "bf16",
        "data": "synthetic (seeded; %s)" % P.recipe,
        "config": {"workload": args.workload, "description": DESCR[args.workload],
                   "query_rows": int(P.query_rows), "q_n": qn,
                   "d_qk": 512 + int(P.params["rope_head_dim"]), "d_v": 512,
                   "rows_per_step": rows_per_step[0], "index_replicas": nrep},
        "gathered_kv_gbps": round(gbps, 2),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernel_ms": {"plan": round(float(np.mean(plan_ms)), 5),
                      "forward": round(float(np.mean(fwd_ms)), 5),
                      "combine": round(float(np.mean(comb_ms)), 5)},
        "roofline": {"kernel": "sfmla::fwd_kernel",
                     "bound": "hbm" if hbm_bound else "mfma",
                     "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": None if traffic is None else round(traffic, 0),
                     "algorithmic_bytes_per_launch": round(fwd_bytes, 0),
                     "algorithmic_flops_per_launch": round(fwd_flops, 0),
                     "bytes_per_row": rb, "flops_per_row_head": fl_row},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        c = counts_all[0]
        result["cpu_baseline"] = cpu_baseline(P, c * fl_row * qn, c * rb)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
