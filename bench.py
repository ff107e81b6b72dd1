"""Throughput of shared-KV sparse flash MLA attention on one MI355X.

One step is one pass of the whole path on one batch: the plan
(sfmla_metadata) and the forward kernel (resolve, gather, QK^T, online
softmax, PV and the merge of the KV splits), all through the C ABI.  Inputs are
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
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_%s_%s.txt")      # (kernel, workload)
MFMA_FILE = os.path.join(PROFILES, "mfma_%s_%s.txt")            # (kernel, workload)

DESCR = {
    "sfa_mla_rope": "token-wise sparse MLA-absorb decode with rope: B=32, q_s=2, q_n=128, "
                    "d_qk=576 (512+64 rope), separate V (512), TopK 2048 of 65536 cached tokens, "
                    "PA_BSND block 64, bf16",
    "sfa_mla_rope_fp16": "the headline decode in float16 (q, K, V and output): B=32, q_s=2, "
                         "q_n=128, d_qk=576, separate V, TopK 2048 of 65536 tokens, PA block 64",
    "sfa_mla_rope_block16": "the headline decode with block-wise TopK: 128 entries of 16 "
                            "consecutive tokens (2048 tokens) per query, bf16, PA block 64",
    "c8_packed_int8": "INT8 per-128-tile packed KV (656-B rows), TND B=8, q_n=128, d_qk=576, "
                      "TopK 2048 of 16K-131K tokens",
    "c8_packed_fp8": "FP8-E4M3 per-128-tile packed KV (656-B rows), TND B=8, q_n=128, d_qk=576, "
                     "TopK 2048 of 16K-131K tokens",
    "hca_varlen": "HCA varlen TND: B=8, q_n=128, window 128 + all visible compressed rows "
                  "(ratio 128), contexts 16K-131K, sinks",
    "c8_packed_int8_rope0": "INT8 packed KV without rope (528-B rows), TND B=8, q_n=128, "
                            "d_qk=512, TopK 2048 of 16K-131K tokens",
    "c8_packed_int8_value": "INT8 packed KV (656-B rows) with a value tensor of 512 INT8 codes per "
                            "row (scaled by the key rows' tiles), TND B=8, q_n=128, d_qk=576, "
                            "TopK 2048 of 16K-131K tokens",
    "hca_prefill": "HCA prefill (the SparseAttnSharedkv call example's shapes with all "
                   "visible compressed rows): B=4 x 128 query tokens, q_n=64, window 128 + "
                   "<=1024 compressed rows (ratio 4), 4096 cached tokens, PA block 128, sinks",
    "swa_prefill": "SWA prefill: B=4 x 128 query tokens, q_n=64, window 128 of 4096 cached "
                   "tokens, PA block 128, sinks",
    "swa_prefill_h16": "SWA prefill with 16 heads: B=4 x 128 query tokens, q_n=16, window 128 "
                       "of 4096 cached tokens, PA block 128, sinks",
    "c8_packed_int8_q32": "throughput mode of c8_packed_int8: the same 8 contexts with 32 query "
                          "tokens each (256 query rows, each its own causal TopK 2048), INT8 "
                          "packed KV, q_n=128, d_qk=576",
    "hca_varlen_q32": "throughput mode of hca_varlen: the same 8 contexts with 32 query tokens "
                      "each (256 query rows, window 128 + all visible compressed rows), sinks",
    "csa_decode_paged": "CSA paged decode: B=4, q_n=64, window 128 + TopK 512 of 8192 "
                        "compressed rows (ratio 4), PA block 128, sinks",
    "swa_decode": "SWA decode: B=2, q_n=16, window 128 of 512, BSND",
    "csa_prefill": "CSA prefill (the SparseAttnSharedkv call example's shapes): B=4 x 128 "
                   "query tokens, q_n=64, window 128 + TopK 512 of 1024 compressed rows "
                   "(ratio 4), 4096 cached tokens, PA block 128, sinks",
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
    if p["kv_dtype"] in ("bf16", "fp16"):
        b = 2 * d_qk + (1024 if p.get("separate_v") else 0)
    else:
        b = 512 + 2 * int(p["rope_head_dim"]) + 16 + (512 if p.get("separate_v") else 0)
    return b, 2 * (d_qk + 512)


def recipe_rows(P):
    """Rows each query row of a workload attends to, counted here from how
    the workload is built (not by the library's resolver): queries sit at
    the last positions of their sequence (query i of q_len at position
    len - q_len + i); TopK entries count where they are >= 0 and (causal
    mode) their token is at or before the position; windows are (win_left,
    win_right) around the position clipped to the sequence; compressed rows
    are the TopK entries a position has completed, or all it has completed
    ((p + 1) // ratio).  The CPU tests check it against the oracle's lists
    on every benchmark workload's recipe."""
    import numpy as np
    p = P.params
    a = P.arrays
    B = int(p["batch_size"])
    if p["layout_q"] == "BSND":
        q_lens = [int(p["q_s"])] * B
    else:
        q_lens = np.diff(a["cu_seqlens_q"]).astype(int).tolist()

    def lens(side):
        su = a.get("seqused_%s_kv" % side)
        if su is not None:
            return [int(x) for x in su]
        cu = a.get("cu_seqlens_%s_kv" % side)
        if cu is not None:
            return np.diff(cu).astype(int).tolist()
        return [int(p["%s_kv_s" % side])] * B

    ori = lens("ori")
    cmp_ = lens("cmp") if p["has_cmp_kv"] else [0] * B
    out = []
    row = 0
    for b in range(B):
        for i in range(q_lens[b]):
            pos = ori[b] - q_lens[b] + i
            if p["ori_topk"]:
                sbs = int(p.get("sparse_block_size", 1))
                ent = np.asarray(a["ori_sparse_indices"][row, 0])
                ent = ent[ent >= 0].astype(np.int64)
                tok = (ent[:, None] * sbs + np.arange(sbs)[None, :]).ravel()
                n = int((tok <= pos).sum()) if p["ori_mask_mode"] == 3 else int((tok < ori[b]).sum())
            else:
                lo = 0 if p["ori_win_left"] < 0 else max(0, pos - p["ori_win_left"])
                hi = ori[b] - 1 if p["ori_win_right"] < 0 else min(ori[b] - 1, pos + p["ori_win_right"])
                n = max(0, hi - lo + 1)
            if p["has_cmp_kv"]:
                vis = min(cmp_[b], (pos + 1) // int(p["cmp_ratio"]))
                if p["cmp_topk"]:
                    ent = np.asarray(a["cmp_sparse_indices"][row, 0])
                    n += int(((ent >= 0) & (ent < vis)).sum())
                else:
                    n += vis
            out.append(n)
            row += 1
    return np.asarray(out, dtype=np.int64)


def kernel_name(P) -> str:
    """The forward kernel (one template for every KV format)."""
    return "fwd_kernel"


def read_summary(path: str):
    """key = value lines of a committed rocprofv3 summary, if it was taken
    on the current kernel source (else None)."""
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals if vals.get("kernel_source_sha256_16") == kernel_source_hash() else None


def read_mfma(kernel: str, workload: str):
    """MFMA utilisation (%) and issued MFMA flops per launch from the committed
    counter summary of the current kernel source (else None)."""
    v = read_summary(MFMA_FILE % (kernel, workload))
    if v is None:
        return None
    try:
        return {"util_pct": float(v["mfma_util_pct"]),
                "flops_issued": float(v["mfma_flops_bf16_per_dispatch"]) +
                                float(v["mfma_flops_f16_per_dispatch"])}
    except (KeyError, ValueError):
        return None


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source (else None)."""
    path = TRAFFIC_FILE % (kernel, workload)
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
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": model,
            "threads": "numpy float64 oracle; %d BLAS threads (threadpoolctl)" % threads,
            "sample": "%d query-row calls over the %d query rows (all heads), %.1f s; "
                      "%.3f GB/s gathered KV" % (len(done), len(rows), dt, by / dt / 1e9)}


COPY_PROBE_MB = 256


def profile_commands(outdir: str, workload: str) -> list:
    """The rocprofv3 runs whose summaries are kept under profiles/: one
    kernel trace with statistics, then one counter pass each for FETCH_SIZE
    and WRITE_SIZE (with a plain device copy of known size for calibration)
    and one for the MFMA counters (rocprofv3's derived MfmaUtil, MFMA busy
    cycles over active cycles of all SIMDs, and MfmaFlopsBF16 / F16, the
    MFMA operations issued)."""
    b = "python3 bench.py --workload %s --no-cpu-baseline --no-sub-configs" % workload
    return [
        "rocprofv3 --kernel-trace --stats --output-format csv -d %s/trace -o trace -- %s"
        % (outdir, b),
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/fetch -o fetch -- %s --steps 5 "
        "--warmup 2 --settle-ms 0 --copy-probe-mb %d" % (outdir, b, COPY_PROBE_MB),
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s/write -o write -- %s --steps 5 "
        "--warmup 2 --settle-ms 0 --copy-probe-mb %d" % (outdir, b, COPY_PROBE_MB),
        "rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF16 --output-format csv -d %s/mfma "
        "-o mfma -- %s --steps 5 --warmup 2 --settle-ms 0" % (outdir, b),
    ]


def write_profiles(outdir: str, workload: str) -> None:
    """Summarise the runs of profile_commands() into profiles/ (text)."""
    import csv
    import glob
    from collections import defaultdict

    cmds = profile_commands(outdir, workload)
    kern = "fwd_kernel"
    src = kernel_source_hash()

    # kernel trace statistics
    stats = glob.glob(os.path.join(outdir, "trace", "**", "*kernel_stats.csv"), recursive=True)
    assert stats, "no kernel_stats.csv under %s/trace" % outdir
    rows = list(csv.DictReader(open(stats[0])))
    lines = ["# rocprofv3 kernel trace, workload %s" % workload,
             "# command (from the repository root):", "#   " + cmds[0],
             "# kernel_source_sha256_16 = %s" % src, "",
             "%-62s %6s %11s %11s %11s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct")]
    for r in rows:
        lines.append("%-62s %6d %11.3f %11.3f %11.3f %7.2f" % (
            r["Name"][:62], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    path = os.path.join(PROFILES, "%s_%s.txt" % (kern, workload))
    open(path, "w").write("\n".join(lines) + "\n")
    log("[profiles] wrote", path)

    # HBM traffic from FETCH_SIZE / WRITE_SIZE, calibrated on the copy probe
    def counters(sub, name):
        f = glob.glob(os.path.join(outdir, sub, "**", "*counter_collection.csv"), recursive=True)
        assert f, "no counter_collection.csv under %s/%s" % (outdir, sub)
        per = defaultdict(list)
        copy = []
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] != name:
                continue
            v = float(r["Counter_Value"])
            if kern + "<" in r["Kernel_Name"] or ("::" + kern + "(") in r["Kernel_Name"]:
                per["k"].append(v)
            if "copyBuffer" in r["Kernel_Name"]:
                copy.append((int(r["Grid_Size"]), v))
        assert per["k"] and copy, "kernel or copy probe missing in %s" % f[0]
        return sum(per["k"]) / len(per["k"]), max(copy)[1], len(per["k"])

    fk, fc, nf = counters("fetch", "FETCH_SIZE")
    wk, wc, nw = counters("write", "WRITE_SIZE")
    probe = COPY_PROBE_MB * (1 << 20)
    ff, wf = probe / (fc * 1024.0), probe / (wc * 1024.0)
    hbm = fk * 1024.0 * ff + wk * 1024.0 * wf
    lines = ["# HBM traffic of %s, workload %s (rocprofv3 counters, KiB per dispatch)" % (kern, workload),
             "# commands (from the repository root):", "#   " + cmds[1], "#   " + cmds[2],
             "# calibration: the %d MiB device copy (reads and writes %d bytes each) reads"
             % (COPY_PROBE_MB, probe),
             "#   FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB: scale factors %.4f and %.4f" % (fc, wc, ff, wf),
             "kernel = %s" % kern,
             "workload = %s" % workload,
             "kernel_source_sha256_16 = %s" % src,
             "dispatches_fetch = %d" % nf,
             "dispatches_write = %d" % nw,
             "fetch_kib_per_dispatch = %.1f" % fk,
             "write_kib_per_dispatch = %.1f" % wk,
             "fetch_scale = %.4f" % ff,
             "write_scale = %.4f" % wf,
             "hbm_read_bytes_per_launch = %.0f" % (fk * 1024.0 * ff),
             "hbm_write_bytes_per_launch = %.0f" % (wk * 1024.0 * wf),
             "hbm_bytes_per_launch = %.0f" % hbm]
    path = TRAFFIC_FILE % (kern, workload)
    open(path, "w").write("\n".join(lines) + "\n")
    log("[profiles] wrote", path)

    # MFMA utilisation and issued MFMA flops
    f = glob.glob(os.path.join(outdir, "mfma", "**", "*counter_collection.csv"), recursive=True)
    assert f, "no counter_collection.csv under %s/mfma" % outdir
    per = defaultdict(list)
    for r in csv.DictReader(open(f[0])):
        if kern + "<" in r["Kernel_Name"] or ("::" + kern + "(") in r["Kernel_Name"]:
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    assert per.get("MfmaUtil"), "no MfmaUtil values for %s in %s" % (kern, f[0])
    mean = lambda k: sum(per[k]) / len(per[k]) if per.get(k) else 0.0
    lines = ["# MFMA counters of %s, workload %s (rocprofv3 derived counters, per dispatch)"
             % (kern, workload),
             "# command (from the repository root):", "#   " + cmds[3],
             "# MfmaUtil = 100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs);",
             "# MfmaFlops* = SQ_INSTS_VALU_MFMA_MOPS_* * 512 (issued MFMA flops)",
             "kernel = %s" % kern,
             "workload = %s" % workload,
             "kernel_source_sha256_16 = %s" % src,
             "dispatches = %d" % len(per["MfmaUtil"]),
             "mfma_util_pct = %.2f" % mean("MfmaUtil"),
             "mfma_flops_bf16_per_dispatch = %.0f" % mean("MfmaFlopsBF16"),
             "mfma_flops_f16_per_dispatch = %.0f" % mean("MfmaFlopsF16")]
    path = MFMA_FILE % (kern, workload)
    open(path, "w").write("\n".join(lines) + "\n")
    log("[profiles] wrote", path)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--time-every", type=int, default=8,
                    help="stamp the forward kernel of every N-th timed step with HIP events "
                         "(the stamping itself delays the next dispatch by a few us)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps run for at least this long before the warm-up "
                         "steps (the GPU clocks settle under sustained load)")
    ap.add_argument("--workload", default="sfa_mla_rope", choices=sorted(DESCR))
    ap.add_argument("--replicas", type=int, default=4,
                    help="index-set replicas rotated between steps (TopK workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--merge-wait-us", type=int, default=0,
                    help="sfmla_params.merge_wait_us (0: the library's rule; -1: the last "
                         "split to arrive merges)")
    ap.add_argument("--no-sub-configs", action="store_true",
                    help="time only --workload (by default the other configurations follow it)")
    ap.add_argument("--split-rows", type=int, default=0,
                    help="sfmla_params.split_rows (0: the library's rule)")
    ap.add_argument("--query-tile", type=int, default=0,
                    help="sfmla_params.query_tile (0: the library's rule; 1: no query tiles)")
    ap.add_argument("--head-blocks-per-group", type=int, default=0,
                    help="sfmla_params.head_blocks_per_group (0: the library's rule)")
    ap.add_argument("--wave-pairs", type=int, default=0,
                    help="sfmla_params.wave_pairs (0: the library's rule; 1: off; 2: on)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one device copy of this size (counter calibration)")
    ap.add_argument("--profile-commands", metavar="OUTDIR",
                    help="print the rocprofv3 commands whose summaries go to profiles/, and exit")
    ap.add_argument("--write-profiles", metavar="OUTDIR",
                    help="summarise the output of those commands into profiles/, and exit")
    args = ap.parse_args()

    if args.profile_commands:
        print("\n".join(profile_commands(args.profile_commands, args.workload)))
        return
    if args.write_profiles:
        write_profiles(args.write_profiles, args.workload)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log("[bench] building workload", args.workload)
    P = synth.make_workload(args.workload)
    m = measure(P, args, dev, args.steps, args.warmup, args.settle_ms, args.time_every,
                args.replicas)
    rb, fl_row = row_bytes(P)
    qn = int(P.params["num_heads_q"])
    kern = kernel_name(P)
    traffic = read_traffic(kern, args.workload)
    mfma = read_mfma(kern, args.workload)

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy probe: %d MiB device copy" % args.copy_probe_mb)

    rl = m["roofline"]
    result = {
        "metric": "decode TFLOP/s + gathered-KV HBM GB/s vs roofline, q_n=128 topk=2048",
        "value": round(m["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": round(m["settle_ms"], 1), "steps": m["settle_steps"]},
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": P.params["kv_dtype"],
        "data": "synthetic (seeded; %s)" % P.recipe,
        "config": {"workload": args.workload, "description": DESCR[args.workload],
                   "query_rows": int(P.query_rows), "q_n": qn,
                   "d_qk": 512 + int(P.params["rope_head_dim"]), "d_v": 512,
                   "rows_per_step": m["rows_per_step"][0], "index_replicas": m["nrep"],
                   "rows_counted_by": "bench.recipe_rows (the workload's construction)"},
        "gathered_kv_gbps": round(m["gbps"], 2),
        "hbm_frac": round(m["gbps"] / HBM_PEAK_GBPS, 4),
        "mfma_frac": round(m["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernel_ms": {"plan": round(m["plan_ms"], 5), "forward": round(m["forward_ms"], 5),
                      "empty_event_bracket": round(m["empty_ms"], 5)},
        "roofline": dict(rl, kernel="sfmla::" + kern,
                         traffic=None if traffic is None else round(traffic, 0),
                         bytes_per_row=rb, flops_per_row_head=fl_row,
                         # rocprofv3 MfmaUtil of the same kernel source (profiles/), or null
                         mfma_util_pct=None if mfma is None else mfma["util_pct"],
                         mfma_flops_issued=None if mfma is None else round(mfma["flops_issued"], 0)),
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        c = m["counts"]
        result["cpu_baseline"] = cpu_baseline(P, c * fl_row * qn, c * rb)
    if not args.no_sub_configs:
        # the other configurations, each timed the same way on fewer steps
        subs = {}
        for name in SUB_CONFIGS:
            if name == args.workload:
                continue
            log("[bench] sub-config", name)
            Q = synth.make_workload(name)
            sm = measure(Q, args, dev, 100, 10, 100.0, 4, args.replicas)
            subs[name] = {"what": SUB_CONFIGS[name], "description": DESCR[name],
                          "forward_us": round(sm["forward_ms"] * 1e3, 2),
                          "ms_per_step": round(sm["ms_per_step"], 5),
                          "tflops_per_step": round(sm["tflops"], 3),
                          "gathered_kv_gbps_per_step": round(sm["gbps"], 2),
                          "rows_per_step": sm["rows_per_step"][0],
                          "roofline": sm["roofline"]}
            del Q
            torch.cuda.empty_cache()
        result["sub_configs"] = subs
    print(json.dumps(result), flush=True)


# The other configurations of the measured set (timed after the headline in
# the same run), with what each stands for.
SUB_CONFIGS = {
    "swa_decode": "c1 SWA decode",
    "csa_decode_paged": "c2 CSA paged decode",
    "hca_varlen": "c3 HCA varlen decode",
    "c8_packed_int8": "c5 packed INT8 KV",
    "c8_packed_fp8": "c5 packed FP8-E4M3 KV",
    "c8_packed_int8_value": "c5 packed INT8 KV with a value tensor of codes",
    "c8_packed_int8_q32": "c5 shapes, 32 query tokens per sequence (throughput mode)",
    "hca_varlen_q32": "c3 shapes, 32 query tokens per sequence (throughput mode)",
    "csa_prefill": "prefill: the SparseAttnSharedkv call example's shapes",
    "swa_prefill": "prefill, window only (four-wave kernel, two workgroups per CU)",
    "swa_prefill_h16": "prefill, window only, 16 heads (four-wave kernel, two workgroups per CU)",
    "hca_prefill": "prefill, window and every visible compressed row (four-wave kernel)",
}


def measure(P, args, dev, steps, warmup, settle_ms, time_every, replicas):
    """Time whole steps (plan + forward) of one workload; the forward of
    every time_every-th step is stamped by its own dispatch.  Inputs are
    resident on the device first; the TopK index set rotates through
    `replicas` independently drawn sets."""
    import numpy as np
    import torch

    import sparse_shared_kv_amd as s
    import synth

    spec = dict(P.params, merge_wait_us=args.merge_wait_us, split_rows=args.split_rows,
                query_tile=args.query_tile, head_blocks_per_group=args.head_blocks_per_group,
                wave_pairs=args.wave_pairs)
    call = s.Call(spec, P.arrays, device=dev)
    reps = synth.index_replicas(P, replicas - 1) if replicas > 1 else []
    idx_sets, counts_all = [], [recipe_rows(P)]
    if reps:
        name = reps[0][0]
        idx_sets = [call.d[name]] + [torch.from_numpy(a).to(dev) for _, a in reps]
        for _, arr in reps:
            counts_all.append(recipe_rows(synth.Problem(P.name, P.seed, P.params,
                                                        dict(P.arrays, **{name: arr}))))
    idx_ptrs = [t.data_ptr() for t in idx_sets]
    nrep = max(1, len(idx_sets))
    rb, fl_row = row_bytes(P)
    qn = int(P.params["num_heads_q"])
    rows_per_step = [int(c.sum()) for c in counts_all]
    flops_step = [n * fl_row * qn for n in rows_per_step]
    bytes_step = [n * rb for n in rows_per_step]
    stream = torch.cuda.current_stream()

    def select(k):
        if idx_sets:
            setattr(call.tensors, reps[0][0], idx_ptrs[k % nrep])

    # clock settle: the first ~150 back-to-back steps on an idle GPU run
    # ~10 % slower than the steady state, whatever the warm-up count
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for k in range(25):
            select(k)
            call.plan(stream)
            call.forward(stream)
        settle_steps += 25
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for k in range(warmup):
        select(k)
        call.plan(stream)
        call.forward(stream)
    torch.cuda.synchronize()

    # timed region: K whole steps.  The forward kernel of every N-th step is
    # timed by a pair of HIP events on the launch stream that the kernel's
    # own dispatch stamps at its start and end (sfmla_time_next_forward):
    # event records queued around the launch would add their own dispatch gap
    # to the measured duration, and even the dispatch-stamped pair delays the
    # next kernel by ~6 us (rocprofv3 kernel trace), so only a sample of the
    # steps carries it.
    every = max(1, time_every)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(0, steps, every)]
    for a, b in ev:                     # create the events (a first record)
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        select(k)
        call.plan(stream)
        if k % every == 0:
            s.sfmla_time_next_forward(ev[k // every][0], ev[k // every][1])
        call.forward(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(call.status.item()) == 0, "device status %d" % int(call.status.item())
    fwd_ms = [a.elapsed_time(b) for a, b in ev]

    # untimed: plan duration for the report, bracketed by event records on
    # the stream (which include the cost of the records themselves; an empty
    # bracket is measured beside it)
    pe = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(10)]
    for k, e in enumerate(pe):
        select(k)
        e[0].record(stream)
        call.plan(stream)
        e[1].record(stream)
        call.forward(stream)
        e[2].record(stream)
        e[3].record(stream)
    torch.cuda.synchronize()
    plan_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in pe]))
    empty_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in pe]))

    tot_flops = sum(flops_step[k % nrep] for k in range(steps))
    tot_bytes = sum(bytes_step[k % nrep] for k in range(steps))
    fwd_avg_s = float(np.mean(fwd_ms)) / 1e3
    fwd_bytes = float(np.mean([bytes_step[k % nrep] for k in range(0, steps, every)]))
    fwd_flops = float(np.mean([flops_step[k % nrep] for k in range(0, steps, every)]))
    hbm_bound = fwd_flops / fwd_bytes < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if hbm_bound:
        achieved, peak, unit = fwd_bytes / fwd_avg_s / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        achieved, peak, unit = fwd_flops / fwd_avg_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    del call
    return {
        "tflops": tot_flops / wall / 1e12, "gbps": tot_bytes / wall / 1e9,
        "ms_per_step": wall * 1e3 / steps, "forward_ms": float(np.mean(fwd_ms)),
        "plan_ms": plan_ms, "empty_ms": empty_ms, "settle_ms": settle_ms,
        "settle_steps": settle_steps, "rows_per_step": rows_per_step, "nrep": nrep,
        "counts": counts_all[0],
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "algorithmic_bytes_per_launch": round(fwd_bytes, 0),
                     "algorithmic_flops_per_launch": round(fwd_flops, 0),
                     "timed_launches": len(fwd_ms)},
    }


if __name__ == "__main__":
    main()
